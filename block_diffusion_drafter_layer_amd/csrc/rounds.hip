// Bookkeeping kernels of the device-resident speculative round (txtmix
// article section 9: after verification the cache is cropped to the accepted
// prefix and the accepted rows' features are appended): the context lengths
// stay in device memory, so a round needs no read-back of tau and can be
// captured into a graph.
#include "common.h"
#include "launch.h"

namespace dfl {

__global__ void __launch_bounds__(64)
advance_len(int32_t* __restrict__ len, const int32_t* __restrict__ tau, SeqTable seqs, int n) {
  const int s = blockIdx.x * 64 + threadIdx.x;
  if (s >= n) return;
  const int cur = seq_len(seqs, s);  // (clamped to the buffer)
  const int t = tau[s] < 0 ? 0 : tau[s];
  const int nxt = cur + t;
  len[s] = nxt > seqs.s[s].max_ctx ? seqs.s[s].max_ctx : nxt;
}

__global__ void __launch_bounds__(64) trim_len(int32_t* __restrict__ len, int n, int32_t keep) {
  const int s = blockIdx.x * 64 + threadIdx.x;
  if (s < n && len[s] > keep) len[s] = keep;
}

hipError_t launch_advance_len(int32_t* len, const int32_t* tau, const SeqTable& seqs, int n_seqs,
                              hipStream_t st) {
  hipLaunchKernelGGL(advance_len, dim3((n_seqs + 63) / 64), dim3(64), 0, st, len, tau, seqs, n_seqs);
  return hipGetLastError();
}

hipError_t launch_trim_len(int32_t* len, int n, int32_t keep, hipStream_t st) {
  hipLaunchKernelGGL(trim_len, dim3((n + 63) / 64), dim3(64), 0, st, len, n, keep);
  return hipGetLastError();
}

}  // namespace dfl
