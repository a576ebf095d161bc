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
// slices, merged per row; the accept tests u_j < p_j(x)/q_j(x) run in order
// and the replacement token is drawn from max(p - q, 0), or the bonus from
// the last target row, by an inverse CDF in fp64 over the vocab in index
// order, spread over vocab slices (see cdf_slice_sums / cdf_pick below). Uniforms come from Philox4x64-10
// (Salmon et al., SC 2011) with key (seed, 0) and counter
// (offset + row, sequence, purpose, 0).
//
// Sampling-mode drafting draws the block's tokens from the draft's own
// distribution the same way (purpose 2), so that the p/q rule sees x ~ q.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace dfl {

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

// One workgroup per sequence. Each row's argmax from its split partials:
// sixteen threads per row, each taking every sixteenth split (all loads
// issued before the max), then four lane exchanges. The accepted prefix
// in one step: a ballot of the rows whose target argmax differs from the
// next drafted token, the first of them ends it ([Code] section 8: the
// cumulative product of matches, plus the bonus token).
__global__ void __launch_bounds__(256)
greedy_accept(const uint64_t* __restrict__ part, int splits, int Bl,
              const int32_t* __restrict__ block, int32_t* __restrict__ tau,
              int32_t* __restrict__ bonus) {
  static_assert(kVerifyMaxSplits <= 64, "four splits per thread");
  const int s = blockIdx.x, t = threadIdx.x;
  __shared__ int32_t post[64];
  for (int j0 = 0; j0 < Bl; j0 += 16) {  // wave-uniform
    const int j = j0 + (t >> 4), q = t & 15;
    uint64_t best = 0;
    if (j < Bl) {
      const uint64_t* p = part + (size_t)(s * Bl + j) * splits;
      uint64_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = q + 16 * u < splits ? p[q + 16 * u] : 0ull;
#pragma unroll
      for (int u = 0; u < 4; ++u) best = umax64(best, v[u]);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const uint64_t other = __shfl_xor(best, o, kWave);
      best = umax64(best, other);
    }
    if (j < Bl && q == 0) post[j] = (int32_t)argmax_key_index(best);
  }
  __syncthreads();
  if (t < 64) {
    // row j < Bl - 1 verifies drafted token j + 1
    const bool miss = t < Bl - 1 && block[(size_t)s * Bl + t + 1] != post[t];
    const uint64_t m = __ballot(miss);
    const int a = m ? __ffsll((unsigned long long)m) - 1 : Bl - 1;
    if (t == 0) {
      tau[s] = a + 1;
      bonus[s] = post[a];
    }
  }
}

hipError_t launch_verify_greedy(const VerifyLaunch& P, hipStream_t st) {
  uint64_t* part = reinterpret_cast<uint64_t*>(P.part);
  hipLaunchKernelGGL(row_argmax_part, dim3(P.splits, P.n_seqs * P.Bl), dim3(256), 0, st,
                     P.target, P.V, P.splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_accept, dim3(P.n_seqs), dim3(256), 0, st, part, P.splits, P.Bl,
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

// Draws by inverse CDF over many workgroups. Stage 1 (row_softmax_part)
// leaves per-slice softmax statistics. Stage 2 (cdf_slice_sums), one
// workgroup per (vocab slice, candidate row): the weights of the slice are
// summed per contiguous thread chunk in vocab order and the chunk sums in
// thread order; split 0 also leaves the merged (M, Z) of the rows it read.
// Stage 3 (cdf_pick), one workgroup per draw: the slice totals are scanned in
// slice order to find the slice holding u * total, the chunk sums of that
// slice are recomputed and scanned in thread order (the same operations in
// the same order, so the slice total is reproduced exactly), and the thread
// whose chunk holds the target runs it in vocab order. The result is the
// smallest v whose running sum exceeds u * total, up to the association of
// the running sum.
//
// Candidate rows: p/q - row c = s * Bl + j, j < gamma: max(p_j - q_j, 0); j =
// gamma: p_gamma (the bonus row). Draft sampling - row r: q_r.
constexpr int kCdfThreads = 256;

struct Merged {
  double m, z;
};

// (M, Z) of row `row` from its split statistics, by wave 0 (splits <= 64);
// the same operations wherever it is called
__device__ __forceinline__ Merged merge_row(const RowStat* part, int row, int splits) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < splits;
  const RowStat r = in ? part[(size_t)row * splits + lane] : RowStat{-INFINITY, 0.0};
  double M = r.m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, kWave));
  const double z = (in && r.m != -INFINITY) ? r.z * exp(r.m - M) : 0.0;
  return Merged{M, wave_sum_d(z)};
}

// the weight of candidate row c at v
struct CdfRow {
  const float* t;  // p (or q when drawing from the draft) source row
  const float* d;  // q row of a p/q residual, else null
  double mt, zt, mq, zq, inv_temp;
  // q on a candidate set instead (LDS copies; cv == null: not used): q(v) is
  // the sum of cq[c] over the candidates c with cv[c] == v
  const int32_t* cv = nullptr;
  const float* cq = nullptr;
  int k = 0;
  // the candidates inside the calling thread's vocab chunk, in candidate
  // order (nl < 0: more than 4, scan them all)
  int nl = 0;
  int lv[4] = {-1, -1, -1, -1};
  double lq[4] = {0.0, 0.0, 0.0, 0.0};
  __device__ void localize(int v0, int v1) {
    if (!cv) return;
    nl = 0;
    for (int c = 0; c < k; ++c) {
      const int v = cv[c];
      if (v >= v0 && v < v1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i == nl) {
            lv[i] = v;
            lq[i] = (double)cq[c];
          }
        ++nl;
      }
    }
    if (nl > 4) nl = -1;
  }
  __device__ double w(int v) const {
    const double p = exp((double)t[v] * inv_temp - mt) / zt;
    if (cv) {
      double q = 0.0;
      if (nl >= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nl && lv[i] == v) q += lq[i];
      } else {
        for (int c = 0; c < k; ++c)
          if (cv[c] == v) q += (double)cq[c];
      }
      const double r = p - q;
      return r > 0.0 ? r : 0.0;
    }
    if (!d) return p;
    const double r = p - exp((double)d[v] * inv_temp - mq) / zq;
    return r > 0.0 ? r : 0.0;
  }
};

// the candidate list and q row of drafted row r into LDS (k <= kSelMaxK)
__device__ __forceinline__ void load_cand_row(const VerifyLaunch& P, int r, int32_t* cv, float* cq) {
  if ((int)threadIdx.x < P.k) {
    cv[threadIdx.x] = P.cand[(size_t)r * P.k + threadIdx.x];
    cq[threadIdx.x] = P.qc[(size_t)r * P.k + threadIdx.x];
  }
}

// stats rows and logits of candidate row c (PQ: p/q residual or bonus row)
template <bool PQ>
__device__ __forceinline__ void cand_rows(const VerifyLaunch& P, int c, int& trow, int& drow) {
  if (PQ) {
    const int Bl = P.Bl, gamma = Bl - 1, s = c / Bl, j = c - s * Bl;
    trow = c;
    drow = j < gamma && !P.cand ? P.n_seqs * Bl + s * gamma + j : -1;
  } else {
    trow = c;
    drow = -1;
  }
}

__device__ __forceinline__ const float* logits_row(const VerifyLaunch& P, int stat_row) {
  const int nt = P.n_seqs * P.Bl;
  return stat_row < nt ? P.target + (size_t)stat_row * P.V
                       : P.draft + (size_t)(stat_row - nt) * P.V;
}

// chunk sums of slice `split` in thread order: local[t] for every thread;
// returns this thread's chunk bounds
__device__ __forceinline__ void slice_chunk(const VerifyLaunch& P, int split, int& v0, int& v1) {
  const int sl = (P.V + P.splits - 1) / P.splits;
  const int a = split * sl, b = min(a + sl, P.V);
  const int ch = (b - a + kCdfThreads - 1) / kCdfThreads;
  v0 = min(a + (int)threadIdx.x * ch, b);
  v1 = min(v0 + ch, b);
}

template <bool PQ>
__global__ void __launch_bounds__(kCdfThreads)
cdf_slice_sums(VerifyLaunch P, const RowStat* part, Merged* merged, double* sums) {
  const int split = blockIdx.x, c = blockIdx.y;
  __shared__ Merged st[2];
  __shared__ double loc[kCdfThreads];
  int trow, drow;
  cand_rows<PQ>(P, c, trow, drow);
  if (threadIdx.x < 64) {
    const Merged a = merge_row(part, trow, P.splits);
    const Merged b = drow >= 0 ? merge_row(part, drow, P.splits) : Merged{0.0, 1.0};
    if (threadIdx.x == 0) {
      st[0] = a;
      st[1] = b;
      if (split == 0) {
        merged[trow] = a;
        if (drow >= 0) merged[drow] = b;
      }
    }
  }
  __shared__ int32_t cv[kSelMaxK];
  __shared__ float cq[kSelMaxK];
  const int gamma = P.Bl - 1, s = c / P.Bl, j = c - s * P.Bl;
  const bool sparse = PQ && P.cand && j < gamma;
  if (sparse) load_cand_row(P, s * gamma + j, cv, cq);
  __syncthreads();
  CdfRow R{logits_row(P, trow), drow >= 0 ? logits_row(P, drow) : nullptr,
           st[0].m, st[0].z, st[1].m, st[1].z, 1.0 / P.temperature};
  if (sparse) {
    R.cv = cv;
    R.cq = cq;
    R.k = P.k;
  }
  int v0, v1;
  slice_chunk(P, split, v0, v1);
  R.localize(v0, v1);
  double local = 0.0;
  for (int v = v0; v < v1; ++v) local += R.w(v);
  loc[threadIdx.x] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int t = 0; t < kCdfThreads; ++t) run += loc[t];
    sums[(size_t)c * P.splits + split] = run;
  }
}

// inverse-CDF draw on candidate row c with uniform u; returns the index.
// loc: LDS [kCdfThreads]; sh: LDS int[3]; dsh: LDS double[1].
__device__ int cdf_draw(const VerifyLaunch& P, const CdfRow& R0, const double* sums, int c, double u,
                        double* loc, int* sh, double* dsh) {
  CdfRow R = R0;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const double* sr = sums + (size_t)c * P.splits;
    double total = 0.0;
    for (int k = 0; k < P.splits; ++k) total += sr[k];
    const double target = u * total;
    int ks = -1;
    double run = 0.0;
    for (int k = 0; k < P.splits; ++k) {
      if (run + sr[k] > target) { ks = k; break; }
      run += sr[k];
    }
    sh[0] = ks;
    sh[1] = -1;
    sh[2] = -1;
    dsh[0] = target - run;
  }
  __syncthreads();
  const int ks = sh[0];
  if (ks < 0) return P.V - 1;  // target at or beyond the total: last index
  const double target = dsh[0];
  int v0, v1;
  slice_chunk(P, ks, v0, v1);
  R.localize(v0, v1);
  double local = 0.0;
  for (int v = v0; v < v1; ++v) local += R.w(v);
  loc[tid] = local;
  __syncthreads();
  if (tid == 0) {  // exclusive running sums of the chunk sums, in thread order
    double run = 0.0;
    for (int t = 0; t < kCdfThreads; ++t) {
      const double x = loc[t];
      loc[t] = run;
      run += x;
    }
  }
  __syncthreads();
  const double before = loc[tid];
  if (v0 < v1 && before <= target && target < before + local) {
    double run = before;
    int pick = v1 - 1;
    for (int v = v0; v < v1; ++v) {
      run += R.w(v);
      if (run > target) { pick = v; break; }
    }
    sh[1] = pick;
  }
  __syncthreads();
  if (sh[1] >= 0) return sh[1];
  // rounding left the target past the slice's last chunk boundary: take the
  // slice's last index with a nonzero weight
  int last = -1;
  if (local > 0.0)
    for (int v = v0; v < v1; ++v)
      if (R.w(v) > 0.0) last = v;
  if (last >= 0) atomicMax(sh + 2, last);
  __syncthreads();
  return sh[2] >= 0 ? sh[2] : P.V - 1;
}

// one workgroup per sequence: the accept tests in order, then the draw from
// the first rejected row's residual or from the bonus row
__global__ void __launch_bounds__(kCdfThreads)
pq_pick(VerifyLaunch P, const Merged* merged, const double* sums) {
  const int s = blockIdx.x, tid = threadIdx.x;
  const int Bl = P.Bl, gamma = Bl - 1, nt = P.n_seqs * Bl;
  __shared__ double loc[kCdfThreads];
  __shared__ int sh[3];
  __shared__ double dsh[1];
  __shared__ int jr_sh;
  __shared__ int32_t cv[kSelMaxK];
  __shared__ float cq[kSelMaxK];
  const double inv_t = 1.0 / P.temperature;
  // the accept tests of all rows at once, one thread each; the first
  // rejected row ends the block (rows after it do not matter)
  __shared__ int rej[64];
  if (tid < gamma) {
    const int j = tid;
    int x = P.block_ids[(size_t)s * Bl + j + 1];
    x = x < 0 ? 0 : (x >= P.V ? P.V - 1 : x);  // keep the read in bounds
    const Merged a = merged[s * Bl + j];
    const double p = exp((double)P.target[(size_t)(s * Bl + j) * P.V + x] * inv_t - a.m) / a.z;
    double q;
    if (P.cand) {  // q on the row's candidate set (zero elsewhere: always kept)
      q = 0.0;
      for (int c = 0; c < P.k; ++c)
        if (P.cand[(size_t)(s * gamma + j) * P.k + c] == x)
          q += (double)P.qc[(size_t)(s * gamma + j) * P.k + c];
    } else {
      const Merged b = merged[nt + s * gamma + j];
      q = exp((double)P.draft[(size_t)(s * gamma + j) * P.V + x] * inv_t - b.m) / b.z;
    }
    const double u = philox_uniform(P.seed, P.offset + j, s, 0);
    rej[j] = q > 0.0 && !(u < p / q);
  }
  __syncthreads();
  if (tid == 0) {
    int jr = gamma;
    for (int j = 0; j < gamma; ++j)
      if (rej[j]) { jr = j; break; }
    jr_sh = jr;
  }
  __syncthreads();
  const int jr = jr_sh;
  const int c = s * Bl + jr;
  const Merged a = merged[c];
  const bool resid = jr < gamma;
  const bool sparse = resid && P.cand;
  if (sparse) load_cand_row(P, s * gamma + jr, cv, cq);
  __syncthreads();
  const Merged b = resid && !P.cand ? merged[nt + s * gamma + jr] : Merged{0.0, 1.0};
  CdfRow R{P.target + (size_t)c * P.V,
           resid && !P.cand ? P.draft + (size_t)(s * gamma + jr) * P.V : nullptr,
           a.m, a.z, b.m, b.z, inv_t};
  if (sparse) {
    R.cv = cv;
    R.cq = cq;
    R.k = P.k;
  }
  const int pick = cdf_draw(P, R, sums, c, philox_uniform(P.seed, P.offset + jr, s, 1), loc, sh, dsh);
  if (tid == 0) {
    P.bonus[s] = pick;
    P.tau[s] = jr + 1;
  }
}

// sampling-mode drafting: one workgroup per drafted row r = s * gamma + j
// (here P.target holds the draft logits, P.Bl = gamma); writes the block
__global__ void __launch_bounds__(kCdfThreads)
draft_pick(VerifyLaunch P, const Merged* merged, const double* sums, int32_t* __restrict__ block,
           int Bl) {
  const int r = blockIdx.x, gamma = P.Bl, s = r / gamma, j = r - s * gamma;
  __shared__ double loc[kCdfThreads];
  __shared__ int sh[3];
  __shared__ double dsh[1];
  const Merged a = merged[r];
  CdfRow R{P.target + (size_t)r * P.V, nullptr, a.m, a.z, 0.0, 1.0, 1.0 / P.temperature};
  const int pick = cdf_draw(P, R, sums, r, philox_uniform(P.seed, P.offset + j, s, 2), loc, sh, dsh);
  if (threadIdx.x == 0) block[(size_t)s * Bl + 1 + j] = pick;
}

hipError_t launch_sample_draft(const VerifyLaunch& P, int32_t* block, int Bl, hipStream_t st) {
  RowStat* part = reinterpret_cast<RowStat*>(P.part);
  Merged* merged = reinterpret_cast<Merged*>(P.part2);
  double* sums = reinterpret_cast<double*>(merged + P.max_rows);
  const int rows = P.n_seqs * P.Bl;
  hipLaunchKernelGGL(row_softmax_part, dim3(P.splits, rows), dim3(256), 0, st, P, part);
  hipLaunchKernelGGL(cdf_slice_sums<false>, dim3(P.splits, rows), dim3(kCdfThreads), 0, st, P, part,
                     merged, sums);
  hipLaunchKernelGGL(draft_pick, dim3(rows), dim3(kCdfThreads), 0, st, P, merged, sums, block, Bl);
  return hipGetLastError();
}

hipError_t launch_verify_pq_cand(const VerifyLaunch& P, hipStream_t st) {
  RowStat* part = reinterpret_cast<RowStat*>(P.part);
  Merged* merged = reinterpret_cast<Merged*>(P.part2);
  double* sums = reinterpret_cast<double*>(merged + P.max_rows);
  const int rows = P.n_seqs * P.Bl;  // target rows only: q comes from the candidate sets
  hipLaunchKernelGGL(row_softmax_part, dim3(P.splits, rows), dim3(256), 0, st, P, part);
  hipLaunchKernelGGL(cdf_slice_sums<true>, dim3(P.splits, rows), dim3(kCdfThreads), 0, st, P, part,
                     merged, sums);
  hipLaunchKernelGGL(pq_pick, dim3(P.n_seqs), dim3(kCdfThreads), 0, st, P, merged, sums);
  return hipGetLastError();
}

hipError_t launch_verify_pq(const VerifyLaunch& P, hipStream_t st) {
  RowStat* part = reinterpret_cast<RowStat*>(P.part);
  Merged* merged = reinterpret_cast<Merged*>(P.part2);
  double* sums = reinterpret_cast<double*>(merged + P.max_rows);
  const int rows = P.n_seqs * P.Bl + P.n_seqs * (P.Bl - 1);
  hipLaunchKernelGGL(row_softmax_part, dim3(P.splits, rows), dim3(256), 0, st, P, part);
  hipLaunchKernelGGL(cdf_slice_sums<true>, dim3(P.splits, P.n_seqs * P.Bl), dim3(kCdfThreads), 0, st,
                     P, part, merged, sums);
  hipLaunchKernelGGL(pq_pick, dim3(P.n_seqs), dim3(kCdfThreads), 0, st, P, merged, sums);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// verification scratch without a workspace: a fixed device array per GPU
// ---------------------------------------------------------------------------
// The partials of verify_noalloc live in this file-scope array (each GPU the
// library runs on holds its own copy until the process ends). Host code must
// never pass the array's name to a kernel: in host code it is a host-side
// stand-in, not a device address. Its device address is looked up once per
// device, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[kVerifyScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kVerifyScratchDevices];
}  // namespace

hipError_t verify_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kVerifyScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dfl
