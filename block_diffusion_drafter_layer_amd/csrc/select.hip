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
//   sel_project      (64 outputs, 16 rows, 128-wide k slice): partial sums of
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

constexpr int kSelPer = 8;                      // logits per lane in a wave's part of a slice
constexpr int kSelSlice = 4 * 64 * kSelPer;     // vocab entries per slice (4 waves)
constexpr int kSelMaxSlices = 128;              // slice lists a row merge takes (two per lane)
constexpr int kSelKSlice = 128;                 // k extent of one projection partial
constexpr int kSelMaxWalkRows = 64;             // rows a walk keeps in LDS

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

// Wave maximum of an unsigned 32-bit value: DPP shifts within each row of 16
// lanes (lane 15 of a row ends with the row's maximum), then the four row
// maxima through scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  uint32_t t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v = v > t ? v : t;
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Wave maximum of a 64-bit key: the high words (the value) by DPP; the low
// words (the index) only when several lanes hold that value. Every lane gets
// the result.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t hv = (uint32_t)(v >> 32);
  const uint32_t hi = wave_max_u32_dpp(hv);
  const uint64_t holders = __ballot(hv == hi);
  uint32_t lo;
  if (__popcll(holders) == 1) {
    lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, __ffsll((unsigned long long)holders) - 1);
  } else {
    lo = wave_max_u32_dpp(hv == hi ? (uint32_t)v : 0u);
  }
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void cswap_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = umax64(a, b), lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// the 8 keys of a lane in decreasing order (a 19-comparator sorting network)
__device__ __forceinline__ void sort8_desc(uint64_t (&k)[8]) {
  cswap_desc(k[0], k[1]); cswap_desc(k[2], k[3]); cswap_desc(k[4], k[5]); cswap_desc(k[6], k[7]);
  cswap_desc(k[0], k[2]); cswap_desc(k[1], k[3]); cswap_desc(k[4], k[6]); cswap_desc(k[5], k[7]);
  cswap_desc(k[1], k[2]); cswap_desc(k[5], k[6]); cswap_desc(k[0], k[4]); cswap_desc(k[3], k[7]);
  cswap_desc(k[1], k[5]); cswap_desc(k[2], k[6]);
  cswap_desc(k[1], k[4]); cswap_desc(k[3], k[6]);
  cswap_desc(k[2], k[4]); cswap_desc(k[3], k[5]);
  cswap_desc(k[3], k[4]);
}

// k rounds of wave maxima over sorted per-lane lists (each in decreasing
// order, 0 = empty); the lane holding a round's key drops it by shifting its
// list. Keys are unique (the index is part of them). out[r] by lane 0.
template <int N>
__device__ __forceinline__ void wave_top_k(uint64_t (&key)[N], int k, uint64_t* out) {
  for (int r = 0; r < k; ++r) {
    const uint64_t best = wave_max_key(key[0]);
    if (key[0] == best && best != 0ull) {
#pragma unroll
      for (int i = 0; i + 1 < N; ++i) key[i] = key[i + 1];
      key[N - 1] = 0;
    }
    if ((threadIdx.x & 63) == 0) out[r] = best;
  }
}

// Two sorted lists per lane (the lane's two slices of a row): the round's
// key leaves whichever list holds it.
template <int N>
__device__ __forceinline__ void wave_top_k2(uint64_t (&ka)[N], uint64_t (&kb)[N], int k,
                                            uint64_t* out) {
  for (int r = 0; r < k; ++r) {
    const uint64_t best = wave_max_key(umax64(ka[0], kb[0]));
    if (best != 0ull && ka[0] == best) {
#pragma unroll
      for (int i = 0; i + 1 < N; ++i) ka[i] = ka[i + 1];
      ka[N - 1] = 0;
    } else if (best != 0ull && kb[0] == best) {
#pragma unroll
      for (int i = 0; i + 1 < N; ++i) kb[i] = kb[i + 1];
      kb[N - 1] = 0;
    }
    if ((threadIdx.x & 63) == 0) out[r] = best;
  }
}

// Lanes below the wave's first set bit of m (the slot of this lane among the
// lanes whose bit is set)
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Each lane of the wave holds at most one of n <= 64 distinct nonzero keys
// (zero: none); out[r] receives the key of rank r (decreasing) for r < k.
// The rank of a key is the number of keys above it, counted against every
// key of cand[0 .. n) (LDS, read as broadcasts).
__device__ __forceinline__ void rank_select(uint64_t my, const uint64_t* cand, int n, int k,
                                            uint64_t* out) {
  int rank = 0;
  for (int i = 0; i < n; ++i) rank += cand[i] > my ? 1 : 0;
  if (my != 0ull && rank < k) out[rank] = my;
}

// (row, vocab slice): each wave takes the top k of its 512 logits, then wave 0
// takes the top k of the four wave lists. A wave first bounds its top k from
// below: T, the largest 32-bit value word such that at least k lanes hold a
// key whose value word is >= T (a bitwise binary search over the lanes'
// maxima, one ballot per bit). The k largest lane maxima are k distinct
// keys >= T, so every key of the top k is too; the keys >= T (typically
// ~20 of 512) are gathered into LDS and ranked against each other. More
// than 64 of them (heavy ties) take the general path: a sorting network per
// lane and k rounds of wave maxima.
__global__ void __launch_bounds__(256)
sel_topk_slices(const float* __restrict__ logits, int V, int n_slices, int k,
                uint64_t* __restrict__ part) {
  __shared__ uint64_t wl[4][kSelMaxK];
  __shared__ uint64_t cand[4][64];
  __shared__ uint64_t merged[kSelMaxK];
  const int sl = blockIdx.x, row = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* z = logits + (size_t)row * V;
  const int v0 = sl * kSelSlice + w * 64 * kSelPer;
  static_assert(kSelPer == 8, "sort8_desc sorts the lane's keys");
  // every load from a clamped address first, all in flight together
  float zv[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int v = v0 + lane + 64 * i;
    zv[i] = z[v < V ? v : V - 1];
  }
  uint64_t key[kSelPer];
  uint64_t kmax = 0ull;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int v = v0 + lane + 64 * i;
    key[i] = v < V ? argmax_key(zv[i], (uint32_t)v) : 0ull;  // 0: no entry (below every key)
    kmax = umax64(kmax, key[i]);
  }
  if (lane < kSelMaxK) wl[w][lane] = 0ull;
  // the threshold on the value word: with fewer than k lanes holding keys,
  // every key is a candidate
  const uint32_t hmax = (uint32_t)(kmax >> 32);
  uint32_t T = 1u;
  if (__popcll(__ballot(kmax != 0ull)) >= k) {
    T = 0u;
    for (int b = 31; b >= 0; --b) {
      const uint32_t t = T | (1u << b);
      if (__popcll(__ballot(hmax >= t)) >= k) T = t;
    }
  }
  int n = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const bool take = key[i] != 0ull && (uint32_t)(key[i] >> 32) >= T;
    const uint64_t m = __ballot(take);
    const int at = n + lanes_below(m);
    if (take && at < 64) cand[w][at] = key[i];
    n += __popcll(m);
  }
  if (n <= 64) {
    const uint64_t my = lane < n ? cand[w][lane] : 0ull;
    rank_select(my, cand[w], n, k, wl[w]);
  } else {
    sort8_desc(key);
    wave_top_k(key, k, wl[w]);
  }
  __syncthreads();
  if (w == 0) {  // the four wave lists: 4 x k distinct keys (or zeros)
    const int nk = 4 * k;
    const uint64_t my = lane < nk ? wl[lane / k][lane % k] : 0ull;
    if (lane < kSelMaxK) merged[lane] = 0ull;
    rank_select(my, &wl[0][0], 4 * kSelMaxK, k, merged);
    if (lane < k) part[((size_t)row * n_slices + sl) * k + lane] = merged[lane];
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
  sq = row16_sum(sq);
  const int m = m0 + orow;
  if (m < rows) {
    float* g = gpart + ((size_t)kz * rows + m) * rank + o0 + ocol;
#pragma unroll
    for (int c = 0; c < 4; ++c) g[c] = acc[c];
    if (blockIdx.x == 0 && (t & 15) == 0) spart[(size_t)kz * rows + m] = sq;
  }
}

// One wave: the top k of a row's slice lists (n_slices sorted lists of k
// keys, n_slices <= 128): lane l holds lists l and l + 64. As in the top-k
// kernel, the lanes' list heads give a lower bound T on the value word of
// the top k; the keys >= T (list prefixes) are gathered into cand (64 keys
// of LDS) and ranked, or, if more than 64, merged by k rounds of wave maxima.
__device__ __forceinline__ void wave_merge_row(const uint64_t* __restrict__ src, int n_slices, int k,
                                               uint64_t* out, uint64_t* cand) {
  const int lane = threadIdx.x & 63;
  uint64_t ka[kSelMaxK], kb[kSelMaxK];
  const int la = lane < n_slices ? lane : n_slices - 1;
  const int lb = lane + 64 < n_slices ? lane + 64 : n_slices - 1;
#pragma unroll
  for (int i = 0; i < kSelMaxK; ++i) {  // clamped loads, all in flight together
    const int ii = i < k ? i : k - 1;
    ka[i] = src[(size_t)la * k + ii];
    kb[i] = src[(size_t)lb * k + ii];
  }
#pragma unroll
  for (int i = 0; i < kSelMaxK; ++i) {
    ka[i] = lane < n_slices && i < k ? ka[i] : 0ull;
    kb[i] = lane + 64 < n_slices && i < k ? kb[i] : 0ull;
  }
  if (lane < kSelMaxK) out[lane] = 0ull;
  const uint64_t head = umax64(ka[0], kb[0]);
  const uint32_t hh = (uint32_t)(head >> 32);
  uint32_t T = 1u;
  if (__popcll(__ballot(head != 0ull)) >= k) {
    T = 0u;
    for (int b = 31; b >= 0; --b) {
      const uint32_t t = T | (1u << b);
      if (__popcll(__ballot(hh >= t)) >= k) T = t;
    }
  }
  int n = 0;
  // the lists are in decreasing order: once no lane takes slot i, none takes
  // a later one
#pragma unroll
  for (int i = 0; i < kSelMaxK; ++i) {
    const bool take = ka[i] != 0ull && (uint32_t)(ka[i] >> 32) >= T;
    const uint64_t m = __ballot(take);
    if (m == 0ull) break;
    const int at = n + lanes_below(m);
    if (take && at < 64) cand[at] = ka[i];
    n += __popcll(m);
  }
#pragma unroll
  for (int i = 0; i < kSelMaxK; ++i) {
    const bool take = kb[i] != 0ull && (uint32_t)(kb[i] >> 32) >= T;
    const uint64_t m = __ballot(take);
    if (m == 0ull) break;
    const int at = n + lanes_below(m);
    if (take && at < 64) cand[at] = kb[i];
    n += __popcll(m);
  }
  if (n <= 64) {
    const uint64_t my = lane < n ? cand[lane] : 0ull;
    rank_select(my, cand, n, k, out);
  } else {
    wave_top_k2(ka, kb, k, out);
  }
}

__global__ void __launch_bounds__(256)
sel_pairs(const uint64_t* __restrict__ part, int n_slices, int k, const float* __restrict__ gpart,
          const float* __restrict__ spart, int kz_n, int rows, int D, float eps,
          const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int rank,
          const int32_t* __restrict__ anchors, int P, int V, float* __restrict__ S,
          int32_t* __restrict__ cand) {
  __shared__ uint64_t top[2][kSelMaxK];
  __shared__ uint64_t mcand[2][64];
  __shared__ int32_t pid[kSelMaxK], cid[kSelMaxK];
  __shared__ float unary[kSelMaxK];
  __shared__ float g[kSelMaxRank];
  __shared__ float ta[kSelMaxK][kSelMaxRank + 1];  // A[pred a] * g
  __shared__ float tb[kSelMaxK][kSelMaxRank + 1];  // B[candidate b]
  const int j = blockIdx.x, s = blockIdx.y, m = s * P + j;
  const int t = threadIdx.x, w = t >> 6;
  const int n = n_slices * k;
  // wave 0 merges this row's slice lists, wave 1 the previous row's (the
  // predecessors); waves 2 and 3 form g meanwhile
  if (w == 0) wave_merge_row(part + (size_t)m * n, n_slices, k, top[1], mcand[0]);
  if (w == 1 && j > 0) wave_merge_row(part + (size_t)(m - 1) * n, n_slices, k, top[0], mcand[1]);
  if (w >= 2) {
    // g = rs * sum of the k-slice partials (slice order), rs the final norm's
    // row scale of row m; the loads of 8 slices at a time are in flight
    // together
    const int tt = t - 128;
    float ss = 0.f, acc0 = 0.f, acc1 = 0.f;
    const int o0 = tt, o1 = tt + 128;
    for (int z0 = 0; z0 < kz_n; z0 += 8) {
      float sv[8], a0[8], a1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int z = z0 + u < kz_n ? z0 + u : kz_n - 1;
        sv[u] = spart[(size_t)z * rows + m];
        a0[u] = gpart[((size_t)z * rows + m) * rank + (o0 < rank ? o0 : 0)];
        a1[u] = gpart[((size_t)z * rows + m) * rank + (o1 < rank ? o1 : 0)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < kz_n) {
          ss += sv[u];
          acc0 += a0[u];
          acc1 += a1[u];
        }
    }
    const float rs = rsqrtf(ss / (float)D + eps);
    if (o0 < rank) g[o0] = acc0 * rs;
    if (o1 < rank) g[o1] = acc1 * rs;
  }
  __syncthreads();
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
  // codes: 16-byte loads, rank / 8 per row and table
  const int per_row = rank / 8;
  for (int e = t; e < kSelMaxK * per_row; e += 256) {
    const int row = e / per_row, x8 = (e - row * per_row) * 8;
    const uint4 av = *reinterpret_cast<const uint4*>(A + (size_t)pid[row] * rank + x8);
    const uint4 bv = *reinterpret_cast<const uint4*>(B + (size_t)cid[row] * rank + x8);
    const uint32_t au[4] = {av.x, av.y, av.z, av.w}, bu[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ta[row][x8 + 2 * i] = __uint_as_float(au[i] << 16) * g[x8 + 2 * i];
      ta[row][x8 + 2 * i + 1] = __uint_as_float(au[i] & 0xffff0000u) * g[x8 + 2 * i + 1];
      tb[row][x8 + 2 * i] = __uint_as_float(bu[i] << 16);
      tb[row][x8 + 2 * i + 1] = __uint_as_float(bu[i] & 0xffff0000u);
    }
  }
  __syncthreads();
  const int a = t >> 4, b = t & 15;
  float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
  for (int x = 0; x < rank; x += 4) {
    d0 += ta[a][x] * tb[b][x];
    d1 += ta[a][x + 1] * tb[b][x + 1];
    d2 += ta[a][x + 2] * tb[b][x + 2];
    d3 += ta[a][x + 3] * tb[b][x + 3];
  }
  const float dot = (d0 + d1) + (d2 + d3);
  S[((size_t)m * kSelMaxK + a) * kSelMaxK + b] = b < k ? unary[b] + dot : -INFINITY;
  if (t < kSelMaxK) cand[(size_t)m * kSelMaxK + t] = t < k ? cid[t] : -1;
}

// v of the lane CTRL (a DPP row shift) names, 0 where that lane lies outside
// the row of 16
template <int CTRL>
__device__ __forceinline__ double row_shr_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// One wave per sequence: row tables into LDS, then the walk. Greedy (inv_T
// == 0): the candidate of largest score, lowest position on ties. Sampling:
// q = softmax(S / T) over the k candidates in fp64, running sums in candidate
// order (a parallel scan: the association differs from a left-to-right sum
// by rounding only), the first candidate whose running sum exceeds u * total, u the
// Philox uniform of counter (offset + row, sequence, 3, 0) (drawn for every
// row up front, one lane each).
__global__ void __launch_bounds__(64)
sel_walk(const float* __restrict__ S, const int32_t* __restrict__ cand, int P, int k, int Bl,
         double inv_T, uint64_t seed, uint64_t offset, int32_t* __restrict__ block,
         int32_t* __restrict__ cand_out, float* __restrict__ q_out) {
  __shared__ float4 tab4[kSelMaxWalkRows * kSelMaxK * kSelMaxK / 4];
  __shared__ int32_t ct[kSelMaxWalkRows][kSelMaxK];
  const int s = blockIdx.x, lane = threadIdx.x;
  const float4* src = reinterpret_cast<const float4*>(S + (size_t)s * P * kSelMaxK * kSelMaxK);
  const int n4 = P * kSelMaxK * kSelMaxK / 4, nc = P * kSelMaxK;
  for (int e0 = 0; e0 < n4; e0 += 64 * 8) {  // 8 loads per lane in flight together
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + lane + 64 * u;
      v[u] = src[e < n4 ? e : n4 - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // clamped lanes rewrite the last entry with its own value
      const int e = e0 + lane + 64 * u;
      tab4[e < n4 ? e : n4 - 1] = v[u];
    }
  }
  {
    const int32_t* cs = cand + (size_t)s * P * kSelMaxK;
    int32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {  // nc <= 64 * 16
      const int e = lane + 64 * u;
      v[u] = cs[e < nc ? e : nc - 1];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = lane + 64 * u;
      (&ct[0][0])[e < nc ? e : nc - 1] = v[u];
    }
  }
  const double u_lane = inv_T != 0.0 && lane < P ? philox_uniform(seed, offset + lane, s, 3) : 0.0;
  __syncthreads();
  const float* tab = reinterpret_cast<const float*>(tab4);
  int a = 0;
  for (int j = 0; j < P; ++j) {
    const float x = lane < k ? tab[(j * kSelMaxK + a) * kSelMaxK + lane] : -INFINITY;
    const uint64_t kx = lane < k ? argmax_key(x, (uint32_t)lane) : 0ull;
    const int best = (int)argmax_key_index(wave_max_key(kx));
    int pick = best;
    if (inv_T == 0.0) {
      if (q_out && lane < k) q_out[((size_t)s * P + j) * k + lane] = lane == pick ? 1.f : 0.f;
    } else {
      const float mx = __shfl(x, best, kWave);
      const double e = lane < k ? exp(((double)x - (double)mx) * inv_T) : 0.0;
      // running sums over the candidates (lanes 0..15, one DPP row): an
      // inclusive scan; the draw is the first lane whose sum exceeds u * total
      double run = e;
      run += row_shr_d<0x111>(run);
      run += row_shr_d<0x112>(run);
      run += row_shr_d<0x114>(run);
      run += row_shr_d<0x118>(run);
      const double tot = __shfl(run, k - 1, kWave);
      const double target = __shfl(u_lane, j, kWave) * tot;
      const uint64_t over = __ballot(lane < k && run > target);
      pick = over ? __ffsll((unsigned long long)over) - 1 : k - 1;
      if (q_out && lane < k) q_out[((size_t)s * P + j) * k + lane] = (float)(e / tot);
    }
    if (cand_out && lane < k) cand_out[((size_t)s * P + j) * k + lane] = ct[j][lane];
    if (lane == 0) block[(size_t)s * Bl + 1 + j] = ct[j][pick];
    a = pick;
  }
}

}  // namespace

int sel_slices(int V) { return (V + kSelSlice - 1) / kSelSlice; }
int sel_kz(int D) { return (D + kSelKSlice - 1) / kSelKSlice; }
int sel_max_walk_rows() { return kSelMaxWalkRows; }
int sel_max_slices() { return kSelMaxSlices; }

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
