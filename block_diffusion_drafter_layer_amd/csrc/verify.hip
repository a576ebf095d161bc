// Verification of drafted blocks against the target's logits (txtmix article
// section 8).
//
// Greedy: every target row is reduced to its argmax (lowest index on exact
// ties) by many workgroups per row writing (value, index) keys; one wave per
// sequence then takes the prefix rule - the accepted length a is the number
// of leading positions j with block[j+1] == posterior[j] - and emits
// tau = a + 1 and bonus = posterior[a].
//
// p/q: per-row softmax statistics in fp64 (max and sum of exp) over vocab
// slices, merged per row; one workgroup per sequence runs the accept tests
// u_j < p_j(x)/q_j(x) in order and draws the replacement token from
// max(p - q, 0), or the bonus from the last target row, by an inverse CDF in
// fp64 over the vocab in index order. Uniforms come from Philox4x64-10
// (Salmon et al., SC 2011) with key (seed, 0) and counter
// (offset + row, sequence, purpose, 0).
//
// Sampling-mode drafting draws the block's tokens from the draft's own
// distribution the same way (purpose 2), so that the p/q rule sees x ~ q.
#include "common.h"
#include "launch.h"

namespace dfl {

// ---------------------------------------------------------------------------
// Philox4x64-10 from the Random123 paper's round function
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t row, uint64_t seq,
                                                 uint64_t purpose) {
  uint64_t c[4] = {row, seq, purpose, 0ull};
  philox4x64_10(c, seed, 0ull);
  return (double)(c[0] >> 11) * 0x1.0p-53;
}

// ---------------------------------------------------------------------------
// greedy
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
row_argmax_part(const float* __restrict__ logits, int V, int splits, uint64_t* __restrict__ part) {
  const int split = blockIdx.x, row = blockIdx.y;
  const int chunk = ((V + splits - 1) / splits + 3) & ~3;
  const int v0 = split * chunk, v1 = min(v0 + chunk, V);
  const float* x = logits + (size_t)row * V;
  uint64_t best = 0;
  if ((V & 3) == 0) {
    for (int v = v0 + 4 * threadIdx.x; v < v1; v += 4 * 256) {
      const float4 q = *reinterpret_cast<const float4*>(x + v);
      best = umax64(best, argmax_key(q.x, v));
      best = umax64(best, argmax_key(q.y, v + 1));
      best = umax64(best, argmax_key(q.z, v + 2));
      best = umax64(best, argmax_key(q.w, v + 3));
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) best = umax64(best, argmax_key(x[v], v));
  }
  best = wave_max_u64(best);
  __shared__ uint64_t wb[4];
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    part[(size_t)row * splits + split] = umax64(umax64(wb[0], wb[1]), umax64(wb[2], wb[3]));
}

__global__ void __launch_bounds__(64)
greedy_accept(const uint64_t* __restrict__ part, int splits, int Bl,
              const int32_t* __restrict__ block, int32_t* __restrict__ tau,
              int32_t* __restrict__ bonus) {
  const int s = blockIdx.x, j = threadIdx.x;
  __shared__ int32_t post[64];
  if (j < Bl) {
    uint64_t best = 0;
    const uint64_t* p = part + (size_t)(s * Bl + j) * splits;
#pragma unroll 8
    for (int k = 0; k < splits; ++k) best = umax64(best, p[k]);
    post[j] = (int32_t)argmax_key_index(best);
  }
  __syncthreads();
  if (j == 0) {
    const int32_t* b = block + (size_t)s * Bl;
    int a = 0;
    while (a < Bl - 1 && b[a + 1] == post[a]) ++a;
    tau[s] = a + 1;
    bonus[s] = post[a];
  }
}

hipError_t launch_verify_greedy(const VerifyLaunch& P, hipStream_t st) {
  uint64_t* part = reinterpret_cast<uint64_t*>(P.part);
  hipLaunchKernelGGL(row_argmax_part, dim3(P.splits, P.n_seqs * P.Bl), dim3(256), 0, st,
                     P.target, P.V, P.splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_accept, dim3(P.n_seqs), dim3(64), 0, st, part, P.splits, P.Bl,
                     P.block_ids, P.tau, P.bonus);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// p/q rejection sampling
// ---------------------------------------------------------------------------
struct RowStat {
  double m, z;  // max of x/T and sum of exp(x/T - m) over a vocab slice
};

__device__ __forceinline__ const float* pq_row(const VerifyLaunch& P, int row) {
  // rows [0, n_seqs*Bl) are target rows, the rest draft rows
  const int nt = P.n_seqs * P.Bl;
  return row < nt ? P.target + (size_t)row * P.V : P.draft + (size_t)(row - nt) * P.V;
}

__global__ void __launch_bounds__(256)
row_softmax_part(VerifyLaunch P, RowStat* part) {
  const int split = blockIdx.x, row = blockIdx.y;
  const int chunk = (P.V + P.splits - 1) / P.splits;
  const int v0 = split * chunk, v1 = min(v0 + chunk, P.V);
  const float* x = pq_row(P, row);
  __shared__ double sh[4];
  double m = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) m = fmax(m, (double)x[v] / P.temperature);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
  __syncthreads();
  double z = 0.0;
  if (m != -INFINITY)
    for (int v = v0 + threadIdx.x; v < v1; v += 256) z += exp((double)x[v] / P.temperature - m);
  z = wave_sum_d(z);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = z;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowStat r;
    r.m = m;
    r.z = sh[0] + sh[1] + sh[2] + sh[3];
    part[(size_t)row * P.splits + split] = r;
  }
}

constexpr int kPQThreads = 1024;

__global__ void __launch_bounds__(kPQThreads)
pq_accept_sample(VerifyLaunch P, const RowStat* part) {
  const int s = blockIdx.x, tid = threadIdx.x;
  const int Bl = P.Bl, gamma = Bl - 1;
  const int nt = P.n_seqs * Bl;
  __shared__ double rm[2 * 16], rz[2 * 16];  // target rows then draft rows
  __shared__ int jr_sh;
  __shared__ double csum[kPQThreads];
  __shared__ double total_sh;
  __shared__ int found;

  // merge slice statistics: one thread per row of this sequence
  if (tid < Bl + gamma) {
    const int row = tid < Bl ? s * Bl + tid : nt + s * gamma + (tid - Bl);
    const RowStat* p = part + (size_t)row * P.splits;
    double M = -INFINITY;
    for (int k = 0; k < P.splits; ++k) M = fmax(M, p[k].m);
    double Z = 0.0;
    for (int k = 0; k < P.splits; ++k)
      if (p[k].m != -INFINITY) Z += p[k].z * exp(p[k].m - M);
    rm[tid] = M;
    rz[tid] = Z;
  }
  __syncthreads();
  if (tid == 0) {
    int jr = gamma;
    for (int j = 0; j < gamma; ++j) {
      int x = P.block_ids[(size_t)s * Bl + j + 1];
      x = x < 0 ? 0 : (x >= P.V ? P.V - 1 : x);  // keep the read in bounds
      const float* tr = P.target + (size_t)(s * Bl + j) * P.V;
      const float* dr = P.draft + (size_t)(s * gamma + j) * P.V;
      const double p = exp((double)tr[x] / P.temperature - rm[j]) / rz[j];
      const double q = exp((double)dr[x] / P.temperature - rm[Bl + j]) / rz[Bl + j];
      const double u = philox_uniform(P.seed, P.offset + j, s, 0);
      if (!(u < p / q)) { jr = j; break; }
    }
    jr_sh = jr;
    found = 0;
  }
  __syncthreads();
  const int jr = jr_sh;
  const bool resid = jr < gamma;
  const float* tr = P.target + (size_t)(s * Bl + jr) * P.V;
  const float* dr = resid ? P.draft + (size_t)(s * gamma + jr) * P.V : nullptr;
  const double mT = rm[jr], zT = rz[jr];
  const double mQ = resid ? rm[Bl + jr] : 0.0, zQ = resid ? rz[Bl + jr] : 1.0;

  // contiguous chunk per thread; weights summed in vocab order inside a chunk
  const int chunk = (P.V + kPQThreads - 1) / kPQThreads;
  const int v0 = tid * chunk, v1 = min(v0 + chunk, P.V);
  auto weight = [&](int v) -> double {
    const double p = exp((double)tr[v] / P.temperature - mT) / zT;
    if (!resid) return p;
    const double q = exp((double)dr[v] / P.temperature - mQ) / zQ;
    const double r = p - q;
    return r > 0.0 ? r : 0.0;
  };
  double local = 0.0;
  for (int v = v0; v < v1; ++v) local += weight(v);
  csum[tid] = local;
  __syncthreads();
  if (tid == 0) {  // exclusive running sums of the chunk totals, in thread order
    double run = 0.0;
    for (int t = 0; t < kPQThreads; ++t) {
      const double c = csum[t];
      csum[t] = run;
      run += c;
    }
    total_sh = run;
  }
  __syncthreads();
  const double total = total_sh;
  const double u2 = philox_uniform(P.seed, P.offset + jr, s, 1);
  const double target = u2 * total;
  const double before = csum[tid];
  if (v0 < v1 && before <= target && target < before + local) {
    double run = before;
    int pick = v1 - 1;
    for (int v = v0; v < v1; ++v) {
      run += weight(v);
      if (run > target) { pick = v; break; }
    }
    found = 1;
    P.bonus[s] = pick;
    P.tau[s] = jr + 1;
  }
  __syncthreads();
  if (tid == 0 && !found) {  // target at or beyond the total: last index
    P.bonus[s] = P.V - 1;
    P.tau[s] = jr + 1;
  }
}

// ---------------------------------------------------------------------------
// sampling-mode drafting: x_j ~ softmax(draft_logits[j] / T)
// ---------------------------------------------------------------------------
// One workgroup per drafted row: the row's slice statistics are merged, the
// weights exp(x/T - m)/Z are summed per contiguous vocab chunk (one per
// thread), the chunk totals are prefix-summed in thread order, and the
// thread whose chunk brackets u * total finds the token by running its
// chunk in vocab order. Here the launch's "target" rows are the draft rows
// ([n_seqs * gamma] of them, P.Bl = gamma) and the output is the block.
__global__ void __launch_bounds__(kPQThreads)
draft_sample(VerifyLaunch P, const RowStat* part, int32_t* __restrict__ block, int Bl) {
  const int row = blockIdx.x, tid = threadIdx.x;
  const int gamma = P.Bl, s = row / gamma, j = row - s * gamma;
  __shared__ double csum[kPQThreads];
  __shared__ double stat_sh[3];
  __shared__ int found;
  if (tid == 0) {
    const RowStat* p = part + (size_t)row * P.splits;
    double M = -INFINITY;
    for (int k = 0; k < P.splits; ++k) M = fmax(M, p[k].m);
    double Z = 0.0;
    for (int k = 0; k < P.splits; ++k)
      if (p[k].m != -INFINITY) Z += p[k].z * exp(p[k].m - M);
    stat_sh[0] = M;
    stat_sh[1] = Z;
    found = 0;
  }
  __syncthreads();
  const double m = stat_sh[0], z = stat_sh[1];
  const float* x = P.target + (size_t)row * P.V;
  const int chunk = (P.V + kPQThreads - 1) / kPQThreads;
  const int v0 = tid * chunk, v1 = min(v0 + chunk, P.V);
  auto weight = [&](int v) -> double { return exp((double)x[v] / P.temperature - m) / z; };
  double local = 0.0;
  for (int v = v0; v < v1; ++v) local += weight(v);
  csum[tid] = local;
  __syncthreads();
  if (tid == 0) {  // exclusive running sums of the chunk totals, in thread order
    double run = 0.0;
    for (int t = 0; t < kPQThreads; ++t) {
      const double c = csum[t];
      csum[t] = run;
      run += c;
    }
    stat_sh[2] = run;
  }
  __syncthreads();
  const double u = philox_uniform(P.seed, P.offset + j, s, 2);
  const double target = u * stat_sh[2];
  const double before = csum[tid];
  int32_t* out = block + (size_t)s * Bl + 1 + j;
  if (v0 < v1 && before <= target && target < before + local) {
    double run = before;
    int pick = v1 - 1;
    for (int v = v0; v < v1; ++v) {
      run += weight(v);
      if (run > target) { pick = v; break; }
    }
    found = 1;
    *out = pick;
  }
  __syncthreads();
  if (tid == 0 && !found) *out = P.V - 1;  // target at or beyond the total: last index
}

hipError_t launch_sample_draft(const VerifyLaunch& P, int32_t* block, int Bl, hipStream_t st) {
  RowStat* part = reinterpret_cast<RowStat*>(P.part);
  const int rows = P.n_seqs * P.Bl;
  hipLaunchKernelGGL(row_softmax_part, dim3(P.splits, rows), dim3(256), 0, st, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(draft_sample, dim3(rows), dim3(kPQThreads), 0, st, P, part, block, Bl);
  return hipGetLastError();
}

hipError_t launch_verify_pq(const VerifyLaunch& P, hipStream_t st) {
  RowStat* part = reinterpret_cast<RowStat*>(P.part);
  const int rows = P.n_seqs * P.Bl + P.n_seqs * (P.Bl - 1);
  hipLaunchKernelGGL(row_softmax_part, dim3(P.splits, rows), dim3(256), 0, st, P, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pq_accept_sample, dim3(P.n_seqs), dim3(kPQThreads), 0, st, P, part);
  return hipGetLastError();
}

}  // namespace dfl
