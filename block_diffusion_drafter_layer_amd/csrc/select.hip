// DFlash 2 candidate selector ([Code] sections 13 and 14): for each drafted
// row t of a block, the top-k tokens of the row's logits are the candidates;
// every pair (a, b) of a predecessor a and a candidate b is scored as
// S_t(a, b) = U_t(b) + sum_x A[a][x] g_t[x] B[b][x], with U_t the drafter's
// logit, A and B the predecessor and successor code tables and g_t = W_h h_t
// the projection of the row's hidden state h_t (the LM head's input, final
// RMSNorm applied); a walk from the anchor then takes the best (or a sampled)
// candidate given the previous choice. The scoring is parallel; the walk is
// the one serial step.
//
// Kernels, in order:
//   sel_topk_slices  (row, vocab slice): the slice's k largest (logit, index)
//                    keys, in decreasing order
//   sel_project      (64 outputs, 16 rows, 256-wide k slice): partial sums of
//                    W_h (x * gain) and of x^2 for the final norm
//   sel_pairs        (row, sequence): merges the slice lists of the row and of
//                    the row before (the predecessors; the anchor for row 0),
//                    then scores all k x k pairs: one thread per pair, a
//                    rank-long dot product over LDS-resident codes
//   sel_walk         (sequence): one wave walks the row tables (in LDS)
#include "common.h"
#include "launch.h"

namespace dfl {

namespace {

constexpr int kSelPer = 8;                      // logits per thread in a slice
constexpr int kSelSlice = 256 * kSelPer;        // vocab entries per slice
constexpr int kSelMergePer = 8;                 // slice keys per thread in a merge
constexpr int kSelKSlice = 256;                 // k extent of one projection partial
constexpr int kSelMaxWalkRows = 64;             // rows a walk keeps in LDS

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

// Block-wide maximum of one key per thread (256 threads); wb: 4 slots of LDS.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* wb) {
  v = wave_max_u64(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) wb[w] = v;
  __syncthreads();
  v = umax64(umax64(wb[0], wb[1]), umax64(wb[2], wb[3]));
  __syncthreads();  // wb is reused by the next call
  return v;
}

__global__ void __launch_bounds__(256)
sel_topk_slices(const float* __restrict__ logits, int V, int n_slices, int k,
                uint64_t* __restrict__ part) {
  __shared__ uint64_t wb[4];
  const int sl = blockIdx.x, row = blockIdx.y;
  const float* z = logits + (size_t)row * V;
  const int v0 = sl * kSelSlice;
  uint64_t key[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int v = v0 + (int)threadIdx.x + 256 * i;
    key[i] = v < V ? argmax_key(z[v], (uint32_t)v) : 0ull;  // 0: no entry (below every key)
  }
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) best = umax64(best, key[i]);
    best = block_max_u64(best, wb);
#pragma unroll
    for (int i = 0; i < kSelPer; ++i)
      if (key[i] == best) key[i] = 0;  // keys are unique (the index is part of them)
    if (threadIdx.x == 0) part[((size_t)row * n_slices + sl) * k + r] = best;
  }
}

// Partial sums over k slice kz (k0 = kz * kSelKSlice) of
// G[m][o] = sum_k x[m][k] gain[k] W[o][k] and of the squares x[m][k]^2, for
// the 16 drafted rows m0 .. m0+15 and outputs o0 .. o0+63. Drafted row m is
// sequence m / P, block row 1 + m % P of x.
__global__ void __launch_bounds__(256)
sel_project(const float* __restrict__ x, int D, int Bl, int P, int rows,
            const bf16_t* __restrict__ gain, const bf16_t* __restrict__ W, int rank,
            float* __restrict__ gpart, float* __restrict__ spart) {
  __shared__ float xs[16][64 + 1];
  __shared__ float ws[64][64 + 1];
  const int t = threadIdx.x;
  const int o0 = blockIdx.x * 64, m0 = blockIdx.y * 16, kz = blockIdx.z;
  const int k0 = kz * kSelKSlice, k1 = min(D, k0 + kSelKSlice);
  const int orow = t >> 4, ocol = (t & 15) * 4;
  // the x row this thread loads (4 consecutive k of row t / 16)
  const int lm = m0 + (t >> 4);
  const float* xr = nullptr;
  if (lm < rows) xr = x + ((size_t)(lm / P) * Bl + 1 + lm % P) * D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;
  for (int kc = k0; kc < k1; kc += 64) {
    {
      const int col = (t & 15) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (xr) v = *reinterpret_cast<const float4*>(xr + kc + col);
      sq += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      xs[t >> 4][col + 0] = v.x * bf2f(gain[kc + col + 0]);
      xs[t >> 4][col + 1] = v.y * bf2f(gain[kc + col + 1]);
      xs[t >> 4][col + 2] = v.z * bf2f(gain[kc + col + 2]);
      xs[t >> 4][col + 3] = v.w * bf2f(gain[kc + col + 3]);
    }
    {
      // 64 W rows x 64 k: thread t covers row t / 4, k (t % 4) * 16 .. +15
      const int wr = t >> 2, wc = (t & 3) * 16;
      const bf16_t* src = W + (size_t)(o0 + wr) * D + kc + wc;
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
      const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ws[wr][wc + 2 * i] = __uint_as_float(u[i] << 16);
        ws[wr][wc + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) {
      const float xv = xs[orow][kk];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += xv * ws[ocol + c][kk];
    }
    __syncthreads();
  }
  // the 16 threads of a row hold its squares: sum them (16-lane groups)
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, kWave);
  const int m = m0 + orow;
  if (m < rows) {
    float* g = gpart + ((size_t)kz * rows + m) * rank + o0 + ocol;
#pragma unroll
    for (int c = 0; c < 4; ++c) g[c] = acc[c];
    if (blockIdx.x == 0 && (t & 15) == 0) spart[(size_t)kz * rows + m] = sq;
  }
}

// Top-k of one row from its slice lists: k rounds of a block-wide maximum
// over n keys (n <= 256 * kSelMergePer). Returns the keys in decreasing order
// in out[0..k).
__device__ __forceinline__ void merge_row(const uint64_t* __restrict__ src, int n, int k,
                                          uint64_t* out, uint64_t* wb) {
  uint64_t key[kSelMergePer];
#pragma unroll
  for (int i = 0; i < kSelMergePer; ++i) {
    const int e = (int)threadIdx.x + 256 * i;
    key[i] = e < n ? src[e] : 0ull;
  }
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kSelMergePer; ++i) best = umax64(best, key[i]);
    best = block_max_u64(best, wb);
#pragma unroll
    for (int i = 0; i < kSelMergePer; ++i)
      if (key[i] == best) key[i] = 0;
    if (threadIdx.x == 0) out[r] = best;
  }
}

__global__ void __launch_bounds__(256)
sel_pairs(const uint64_t* __restrict__ part, int n_slices, int k, const float* __restrict__ gpart,
          const float* __restrict__ spart, int kz_n, int rows, int D, float eps,
          const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int rank,
          const int32_t* __restrict__ anchors, int P, int V, float* __restrict__ S,
          int32_t* __restrict__ cand) {
  __shared__ uint64_t wb[4];
  __shared__ uint64_t top[2][kSelMaxK];
  __shared__ int32_t pid[kSelMaxK], cid[kSelMaxK];
  __shared__ float unary[kSelMaxK];
  __shared__ float g[kSelMaxRank];
  __shared__ float ta[kSelMaxK][kSelMaxRank + 1];  // A[pred a] * g
  __shared__ float tb[kSelMaxK][kSelMaxRank + 1];  // B[candidate b]
  const int j = blockIdx.x, s = blockIdx.y, m = s * P + j;
  const int t = threadIdx.x;
  const int n = n_slices * k;
  if (j > 0) merge_row(part + (size_t)(m - 1) * n, n, k, top[0], wb);
  merge_row(part + (size_t)m * n, n, k, top[1], wb);
  __syncthreads();  // top[] complete
  // g = rs * sum of the k-slice partials (slice order), rs the final norm's
  // row scale of row m
  float ss = 0.f;
  for (int z = 0; z < kz_n; ++z) ss += spart[(size_t)z * rows + m];
  const float rs = rsqrtf(ss / (float)D + eps);
  for (int o = t; o < rank; o += 256) {
    float acc = 0.f;
    for (int z = 0; z < kz_n; ++z) acc += gpart[((size_t)z * rows + m) * rank + o];
    g[o] = acc * rs;
  }
  if (t < kSelMaxK) {
    const bool live = t < k;
    const uint64_t kb = top[1][live ? t : 0];
    cid[t] = live ? (int32_t)argmax_key_index(kb) : 0;
    unary[t] = live ? key_value(kb) : -INFINITY;
    int an = j == 0 ? anchors[s] : 0;
    an = an < 0 ? 0 : (an >= V ? V - 1 : an);  // keep the code lookup in bounds
    pid[t] = j == 0 ? an : (live ? (int32_t)argmax_key_index(top[0][t]) : 0);
  }
  __syncthreads();
  for (int e = t; e < kSelMaxK * rank; e += 256) {
    const int row = e / rank, x = e - row * rank;
    ta[row][x] = bf2f(A[(size_t)pid[row] * rank + x]) * g[x];
    tb[row][x] = bf2f(B[(size_t)cid[row] * rank + x]);
  }
  __syncthreads();
  const int a = t >> 4, b = t & 15;
  float dot = 0.f;
  for (int x = 0; x < rank; ++x) dot += ta[a][x] * tb[b][x];
  S[((size_t)m * kSelMaxK + a) * kSelMaxK + b] = b < k ? unary[b] + dot : -INFINITY;
  if (t < kSelMaxK) cand[(size_t)m * kSelMaxK + t] = t < k ? cid[t] : -1;
}

// One wave per sequence: row tables into LDS, then the walk. Greedy (inv_T
// == 0): the candidate of largest score, lowest position on ties. Sampling:
// q = softmax(S / T) over the k candidates in fp64, running sums in candidate
// order, the first candidate whose running sum exceeds u * total, u the
// Philox uniform of counter (offset + row, sequence, 3, 0).
__global__ void __launch_bounds__(64)
sel_walk(const float* __restrict__ S, const int32_t* __restrict__ cand, int P, int k, int Bl,
         double inv_T, uint64_t seed, uint64_t offset, int32_t* __restrict__ block,
         int32_t* __restrict__ cand_out, float* __restrict__ q_out) {
  __shared__ float tab[kSelMaxWalkRows][kSelMaxK][kSelMaxK];
  __shared__ int32_t ct[kSelMaxWalkRows][kSelMaxK];
  __shared__ double ex[kSelMaxK];
  const int s = blockIdx.x, lane = threadIdx.x;
  const float* src = S + (size_t)s * P * kSelMaxK * kSelMaxK;
  for (int e = lane; e < P * kSelMaxK * kSelMaxK; e += 64) (&tab[0][0][0])[e] = src[e];
  for (int e = lane; e < P * kSelMaxK; e += 64) (&ct[0][0])[e] = cand[(size_t)s * P * kSelMaxK + e];
  __syncthreads();
  int a = 0;
  for (int j = 0; j < P; ++j) {
    const float x = lane < k ? tab[j][a][lane] : -INFINITY;
    int pick;
    if (inv_T == 0.0) {
      pick = (int)argmax_key_index(wave_max_u64(argmax_key(x, (uint32_t)lane)));
    } else {
      const float mx = __shfl(x, (int)argmax_key_index(wave_max_u64(argmax_key(x, (uint32_t)lane))), kWave);
      const double e = lane < k ? exp(((double)x - (double)mx) * inv_T) : 0.0;
      if (lane < kSelMaxK) ex[lane] = e;
      __syncthreads();
      if (lane == 0) {
        double tot = 0.0;
        for (int c = 0; c < k; ++c) tot += ex[c];
        const double target = philox_uniform(seed, offset + j, s, 3) * tot;
        double run = 0.0;
        int c = 0;
        for (; c < k; ++c) {
          run += ex[c];
          if (run > target) break;
        }
        ex[0] = (double)(c < k ? c : k - 1) + 0.25;  // hand the choice to the wave
        ex[1] = tot;
      }
      __syncthreads();
      pick = (int)ex[0];
      const double tot = ex[1];
      if (q_out && lane < k) q_out[((size_t)s * P + j) * k + lane] = (float)(e / tot);
      __syncthreads();  // ex is rewritten by the next row
    }
    if (inv_T == 0.0 && q_out && lane < k)
      q_out[((size_t)s * P + j) * k + lane] = lane == pick ? 1.f : 0.f;
    if (cand_out && lane < k) cand_out[((size_t)s * P + j) * k + lane] = ct[j][lane];
    if (lane == 0) block[(size_t)s * Bl + 1 + j] = ct[j][pick];
    a = pick;
  }
}

}  // namespace

int sel_slices(int V) { return (V + kSelSlice - 1) / kSelSlice; }
int sel_kz(int D) { return (D + kSelKSlice - 1) / kSelKSlice; }
int sel_max_walk_rows() { return kSelMaxWalkRows; }
int sel_max_merge_keys() { return 256 * kSelMergePer; }

hipError_t launch_select(const SelectLaunch& L, hipStream_t st) {
  const int rows = L.n_seqs * L.P;
  const int ns = sel_slices(L.V), kz = sel_kz(L.D);
  hipLaunchKernelGGL(sel_topk_slices, dim3(ns, rows), dim3(256), 0, st, L.logits, L.V, ns, L.k,
                     L.keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sel_project, dim3(L.rank / 64, (rows + 15) / 16, kz), dim3(256), 0, st,
                     L.last_hidden, L.D, L.Bl, L.P, rows, L.gain, L.w_proj, L.rank, L.gpart,
                     L.spart);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_pairs, dim3(L.P, L.n_seqs), dim3(256), 0, st, L.keys, ns, L.k, L.gpart,
                     L.spart, kz, rows, L.D, L.eps, L.pred, L.succ, L.rank, L.anchors, L.P, L.V, L.S,
                     L.cand);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_walk, dim3(L.n_seqs), dim3(64), 0, st, L.S, L.cand, L.P, L.k, L.Bl,
                     L.temperature > 0.0 ? 1.0 / L.temperature : 0.0, L.seed, L.offset, L.block,
                     L.cand_out, L.q_out);
  return hipGetLastError();
}

}  // namespace dfl
