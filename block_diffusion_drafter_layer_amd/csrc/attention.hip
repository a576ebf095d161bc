// Block attention of the draft forward: every block row of a sequence attends,
// with no mask, to the sequence's context K/V followed by the block's own K/V
// (txtmix article section 5: k = cat(k_ctx, k_noise); section 6: the
// full-attention draft layers are not causal). Grouped-query heads: query
// head a reads kv head a / G.
//
// The context keys come from the bf16 KV cache; the block's own keys never
// enter the cache: the QKV epilogue leaves them in fp32 in the workspace, and
// the split that holds the context's last key takes them as one more chunk
// (K and V as bf16 hi/lo pairs).
//
// One workgroup per (key range, kv head, sequence) with one wave per query
// head of the group; each wave holds the 16 block rows of its head as the
// MFMA columns. Scores are formed transposed, S^T = K Q^T, so that a lane's
// four accumulator rows are keys: with keys assigned to A rows as
// key(t, i) = 8*(i/4) + 4*t + i%4, lane group g of both 16-key tiles holds
// keys 8g..8g+7 of the 32-key chunk, which is exactly the k-slot layout of
// the bf16 P^T operand of O^T = V^T P^T. P therefore never leaves registers,
// and V^T operands are 16-byte loads from the dim-major V plane of the cache.
// Each workgroup keeps a running max / sum / accumulator over its keys and
// writes them as a partial; a second kernel merges the partials of a head.
// Q and P enter the MFMAs as bf16 hi/lo pairs (two MFMAs each), so the only
// bf16 rounding left in attention is the KV cache's own storage format of the
// context rows.
#include "common.h"
#include "launch.h"

namespace dfl {

struct AttnArgs {
  const bf16_t* q;       // [M][Hq][HD] after RoPE, hi
  const bf16_t* q_lo;    // lo
  const float* blk_k;    // [M][Hkv][HD] the block's own K after RoPE, fp32
  const float* blk_v;    // [M][Hkv][HD] the block's own V, fp32
  float* acc;            // [(s*Hq + a)*splits + split][16][HD]
  float* ml;             // [(s*Hq + a)*splits + split][16][2]
  int Hq, Hkv, Bl, layer, splits, kps;
  // blk_wg: workgroup x = splits takes the block's own keys (else the merge
  // does); slots: partial slots per (sequence, query head), splits + blk_wg
  int blk_wg, slots;
  float scale_log2;      // log2(e) / sqrt(HD)
  SeqTable seqs;
};

template <int HD>
struct Chunk {
  static constexpr int KSTEPS = (HD + 31) / 32;  // head_dim 16 pads k to 32 with zeros
  static constexpr int HT = HD / 16;
  bf16x8 kf[2][KSTEPS];
  u32x4 v[HT];
};

// K rows of the chunk as the A operand of S^T = K Q^T (keys permuted so each
// lane group ends up with 8 consecutive keys) and the V^T rows for the same
// keys. Addresses stay inside the cache's cap rows, so they do not depend on
// the context length (which may still be on its way from device memory);
// keys past the range are masked when the chunk is processed.
template <int HD>
__device__ __forceinline__ void load_chunk(Chunk<HD>& c, int c0, const bf16_t* kbase,
                                           const bf16_t* vbase, int cap, int ql, int lg) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int key = c0 + (ql >> 2) * 8 + t * 4 + (ql & 3);
    key = key < cap ? key : cap - 1;
    const bf16_t* kr = kbase + (size_t)key * HD + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < Chunk<HD>::KSTEPS; ++ks)
      c.kf[t][ks] = (ks * 32 + 8 * lg < HD) ? ld_bf16x8(kr + ks * 32) : zero_bf16x8();
  }
  const int kl = c0 + 8 * lg;
  const int kl_ld = kl < cap ? kl : 0;  // cap is a multiple of 64: 8 keys stay in the row
#pragma unroll
  for (int h = 0; h < Chunk<HD>::HT; ++h)
    c.v[h] = *reinterpret_cast<const u32x4*>(vbase + (size_t)(h * 16 + ql) * cap + kl_ld);
}

// Online-softmax step for one 32-key chunk whose transposed scores are in st
// (lane (ql, lg): keys c0 + 8 lg .. +7 of query row ql): keys at or past ke
// masked, the running max over the row's four lanes, the rescale of the
// accumulators, and P (unnormalised, <= 1) as a bf16 hi/lo pair.
template <int HT>
__device__ __forceinline__ void softmax_step(f32x4 (&st)[2], int c0, int ke, float scale_log2,
                                             int lg, float& m_run, float& l_run, f32x4* acc,
                                             bf16x8& pf, bf16x8& pfl) {
  const int kl = c0 + 8 * lg;
  float sc[8];
  float mloc = -INFINITY;
  if (ke - c0 >= 32) {  // every key of the chunk in range (wave-uniform)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[4 * t + e] = st[t][e] * scale_log2;
        mloc = fmaxf(mloc, sc[4 * t + e]);
      }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = (kl + 4 * t + e < ke) ? st[t][e] * scale_log2 : -INFINITY;
        sc[4 * t + e] = v;
        mloc = fmaxf(mloc, v);
      }
  }
  mloc = rows4_max(mloc);
  const float m_new = fmaxf(m_run, mloc);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float pr[8], psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
    psum += pr[i];
  }
  // the accumulators are rescaled only when some lane's running max moved
  // (wave-uniform test; before the first chunk they are zero anyway)
  if (__any(m_run > -INFINITY && alpha < 1.f)) {
#pragma unroll
    for (int h = 0; h < HT; ++h) acc[h] *= alpha;
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  pack_split_bf16x8(pr, pf, pfl);
}

template <int HD>
__device__ __forceinline__ void process_chunk(const Chunk<HD>& c, int c0, int ke, const bf16x8* qf,
                                              const bf16x8* qfl, float scale_log2, int lg,
                                              float& m_run, float& l_run, f32x4* acc) {
  constexpr int KSTEPS = Chunk<HD>::KSTEPS, HT = Chunk<HD>::HT;
  // hi and lo products in separate accumulators: four independent MFMA
  // chains of KSTEPS instead of two of 2 * KSTEPS
  f32x4 st[2], stl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    stl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = mfma16x16x32(c.kf[t][ks], qf[ks], st[t]);
      stl[t] = mfma16x16x32(c.kf[t][ks], qfl[ks], stl[t]);
    }
#pragma unroll
  for (int t = 0; t < 2; ++t) st[t] += stl[t];
  bf16x8 pf, pfl;
  softmax_step<HT>(st, c0, ke, scale_log2, lg, m_run, l_run, acc, pf, pfl);
  if (ke - c0 >= 32) {  // a whole chunk of valid keys (wave-uniform)
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, c.v[h]);
      acc[h] = mfma16x16x32(vf, pf, acc[h]);
      acc[h] = mfma16x16x32(vf, pfl, acc[h]);
    }
    return;
  }
  // keys past the range contribute zero V, never NaN
  const int nvalid = ke - (c0 + 8 * lg);
  uint32_t keep[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    keep[i] = ((2 * i < nvalid) ? 0x0000ffffu : 0u) | ((2 * i + 1 < nvalid) ? 0xffff0000u : 0u);
#pragma unroll
  for (int h = 0; h < HT; ++h) {
    u32x4 raw = c.v[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] &= keep[i];
    const bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
    acc[h] = mfma16x16x32(vf, pf, acc[h]);
    acc[h] = mfma16x16x32(vf, pfl, acc[h]);
  }
}

// The block's own Bl keys (<= 16, fp32 rows of the workspace: key j of this
// kv head at bk + j * kvd, its value at bv + j * kvd) as one more chunk of
// the running softmax, laid out like a context chunk. K and V enter the
// MFMAs as bf16 hi/lo pairs like Q and P (the lo x lo term dropped), so the
// products keep about fp32 accuracy.
template <int HD>
__device__ __forceinline__ void process_block(const float* bk, const float* bv, int kvd, int Bl,
                                              const bf16x8* qf, const bf16x8* qfl, float scale_log2,
                                              int ql, int lg, float& m_run, float& l_run,
                                              f32x4* acc) {
  constexpr int KSTEPS = Chunk<HD>::KSTEPS, HT = Chunk<HD>::HT;
  // every load first (one round trip): K rows as the A operand of each
  // score tile and k step, then the V^T values (dim 16 h + ql, keys 8 lg ..
  // 8 lg + 7), zero past Bl
  float kf[2][KSTEPS][8], vf[HT][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = 8 * (ql >> 2) + 4 * t + (ql & 3);  // A row ql of score tile t
    const bool kv = key < Bl;
    const float* kr = bk + (size_t)(kv ? key : 0) * kvd + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bool in = kv && ks * 32 + 8 * lg < HD;
      const float4 a = in ? *reinterpret_cast<const float4*>(kr + ks * 32) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 b = in ? *reinterpret_cast<const float4*>(kr + ks * 32 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      kf[t][ks][0] = a.x; kf[t][ks][1] = a.y; kf[t][ks][2] = a.z; kf[t][ks][3] = a.w;
      kf[t][ks][4] = b.x; kf[t][ks][5] = b.y; kf[t][ks][6] = b.z; kf[t][ks][7] = b.w;
    }
  }
#pragma unroll
  for (int h = 0; h < HT; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 8 * lg + e;
      vf[h][e] = key < Bl ? bv[(size_t)key * kvd + h * 16 + ql] : 0.f;
    }
  f32x4 st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      bf16x8 kh, klo;
      pack_split_bf16x8(kf[t][ks], kh, klo);
      st[t] = mfma16x16x32(kh, qf[ks], st[t]);
      st[t] = mfma16x16x32(kh, qfl[ks], st[t]);
      st[t] = mfma16x16x32(klo, qf[ks], st[t]);
    }
  }
  bf16x8 pf, pfl;
  softmax_step<HT>(st, 0, Bl, scale_log2, lg, m_run, l_run, acc, pf, pfl);
#pragma unroll
  for (int h = 0; h < HT; ++h) {
    bf16x8 vh, vlo;
    pack_split_bf16x8(vf[h], vh, vlo);
    acc[h] = mfma16x16x32(vh, pf, acc[h]);
    acc[h] = mfma16x16x32(vh, pfl, acc[h]);
    acc[h] = mfma16x16x32(vlo, pf, acc[h]);
  }
}

// A wave's partial (running max, sum and accumulator of its query head's 16
// rows; l already summed over the row's lanes), written through the L2: the
// merge is another launch.
template <int HD>
__device__ __forceinline__ void write_partial(const AttnArgs& p, size_t slot, int ql, int lg,
                                              const f32x4* acc, float m_run, float l_run) {
  constexpr int HT = Chunk<HD>::HT;
  float* out = p.acc + slot * 16 * HD;
#pragma unroll
  for (int h = 0; h < HT; ++h)
    store16_wt(out, (uint32_t)((ql * HD + h * 16 + 4 * lg) * 4), acc[h]);
  if (lg == 0) {
    p.ml[(slot * 16 + ql) * 2 + 0] = m_run;
    p.ml[(slot * 16 + ql) * 2 + 1] = l_run;
  }
}

// The workgroup past the context's splits: each query-head wave takes only
// the block's own keys, into the head's last partial slot. It runs beside
// the context splits, so the block adds no step to their chains.
template <int HD>
__device__ __forceinline__ void block_partial(const AttnArgs& p, int s, int g, int a, int ql, int lg) {
  constexpr int KSTEPS = Chunk<HD>::KSTEPS, HT = Chunk<HD>::HT;
  bf16x8 qf[KSTEPS], qfl[KSTEPS];
  const bool qv = ql < p.Bl;
  const size_t qoff = ((size_t)(s * p.Bl + (qv ? ql : 0)) * p.Hq + a) * HD + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const bool in = qv && ks * 32 + 8 * lg < HD;
    qf[ks] = in ? ld_bf16x8(p.q + qoff + ks * 32) : zero_bf16x8();
    qfl[ks] = in ? ld_bf16x8(p.q_lo + qoff + ks * 32) : zero_bf16x8();
  }
  f32x4 acc[HT];
#pragma unroll
  for (int h = 0; h < HT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const size_t kvd = (size_t)p.Hkv * HD;
  const size_t b0 = (size_t)(s * p.Bl) * kvd + (size_t)g * HD;
  process_block<HD>(p.blk_k + b0, p.blk_v + b0, (int)kvd, p.Bl, qf, qfl, p.scale_log2, ql, lg,
                    m_run, l_run, acc);
  l_run = rows4_sum(l_run);
  write_partial<HD>(p, (size_t)(s * p.Hq + a) * p.slots + p.splits, ql, lg, acc, m_run, l_run);
}

// Workgroup = G query-head waves x W key columns for one (key range, kv head,
// sequence). Column c of the range's 32-key chunks goes to key column c % W.
// The W partial softmax states of a head are merged through LDS, so one
// partial per (range, head) reaches memory.
template <int HD, int G, int W, bool PIPE>
__global__ void __launch_bounds__(G * W * 64)
attn_split(AttnArgs p) {
  constexpr int KSTEPS = Chunk<HD>::KSTEPS;
  constexpr int HT = Chunk<HD>::HT;
  __shared__ float lds_acc[(W > 1 ? W - 1 : 1) * G][16 * HD];
  __shared__ float lds_ml[(W > 1 ? W - 1 : 1) * G][16][2];
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  // the wave index in a scalar register: the key-column loop then branches
  // uniformly and the wait counts on its loads stay exact
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gi = w % G, wi = w / G;
  const int a = g * G + gi;
  const int ql = lane & 15, lg = lane >> 4;
  if (p.blk_wg && split == p.splits) {  // the block's own keys (whole workgroup)
    if (wi == 0) block_partial<HD>(p, s, g, a, ql, lg);
    return;
  }
  const SeqDesc sd = p.seqs.s[s];
  const int kb = split * p.kps;
  const size_t plane = (size_t)sd.cap * HD;
  const bf16_t* kbase = sd.kv + (size_t)((2 * p.layer) * p.Hkv + g) * plane;
  const bf16_t* vbase = sd.kv + (size_t)((2 * p.layer + 1) * p.Hkv + g) * plane;

  // the queries and the first chunk are requested together
  bf16x8 qf[KSTEPS], qfl[KSTEPS];
  const bool qv = ql < p.Bl;
  const size_t qoff = ((size_t)(s * p.Bl + (qv ? ql : 0)) * p.Hq + a) * HD + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const bool in = qv && ks * 32 + 8 * lg < HD;
    qf[ks] = in ? ld_bf16x8(p.q + qoff + ks * 32) : zero_bf16x8();
    qfl[ks] = in ? ld_bf16x8(p.q_lo + qoff + ks * 32) : zero_bf16x8();
  }
  constexpr int STEP = 32 * W;
  int c0 = kb + 32 * wi;
  Chunk<HD> ca, cb;
  if (PIPE) load_chunk<HD>(ca, c0, kbase, vbase, sd.cap, ql, lg);
  // the context length (host value or device memory) is needed only now
  const int n_keys = seq_len(p.seqs, s);  // context keys only
  const int ke = split == p.splits - 1 ? n_keys : min(kb + p.kps, n_keys);  // last: the rest

  f32x4 acc[HT];
#pragma unroll
  for (int h = 0; h < HT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  if (!PIPE) {  // one register stage
    for (; c0 < ke; c0 += STEP) {
      Chunk<HD> ca;
      Chunk<HD> cs;
      load_chunk<HD>(cs, c0, kbase, vbase, sd.cap, ql, lg);
      process_chunk<HD>(cs, c0, ke, qf, qfl, p.scale_log2, lg, m_run, l_run, acc);
    }
  }
  // two register stages: the next chunk of this column is in flight while
  // the current one is processed. The next load is issued unconditionally
  // (past the column's last chunk it re-reads that chunk, a cache hit), so
  // that every wait on a chunk is an exact count rather than a full drain.
  if (PIPE && c0 < ke) {
    const int last = c0 + (ke - 1 - c0) / STEP * STEP;  // the column's last chunk
    for (;;) {
      load_chunk<HD>(cb, min(c0 + STEP, last), kbase, vbase, sd.cap, ql, lg);
      process_chunk<HD>(ca, c0, ke, qf, qfl, p.scale_log2, lg, m_run, l_run, acc);
      c0 += STEP;
      if (c0 > last) break;
      load_chunk<HD>(ca, min(c0 + STEP, last), kbase, vbase, sd.cap, ql, lg);
      process_chunk<HD>(cb, c0, ke, qf, qfl, p.scale_log2, lg, m_run, l_run, acc);
      c0 += STEP;
      if (c0 > last) break;
    }
  }
  l_run = rows4_sum(l_run);

  if (W > 1) {
    if (wi > 0) {
      const int slot = (wi - 1) * G + gi;
#pragma unroll
      for (int h = 0; h < HT; ++h)
        *reinterpret_cast<f32x4*>(&lds_acc[slot][ql * HD + h * 16 + 4 * lg]) = acc[h];
      if (lg == 0) {
        lds_ml[slot][ql][0] = m_run;
        lds_ml[slot][ql][1] = l_run;
      }
    }
    __syncthreads();
    if (wi > 0) return;
    float mm[W], sc[W];
    mm[0] = m_run;
#pragma unroll
    for (int j = 1; j < W; ++j) mm[j] = lds_ml[(j - 1) * G + gi][ql][0];
    float M = mm[0];
#pragma unroll
    for (int j = 1; j < W; ++j) M = fmaxf(M, mm[j]);
#pragma unroll
    for (int j = 0; j < W; ++j) sc[j] = mm[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm[j] - M);
    l_run *= sc[0];
#pragma unroll
    for (int j = 1; j < W; ++j) l_run += sc[j] * lds_ml[(j - 1) * G + gi][ql][1];
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      acc[h] *= sc[0];
#pragma unroll
      for (int j = 1; j < W; ++j)
        acc[h] += sc[j] * *reinterpret_cast<const f32x4*>(&lds_acc[(j - 1) * G + gi][ql * HD + h * 16 + 4 * lg]);
    }
    m_run = M;
  }
  write_partial<HD>(p, (size_t)(s * p.Hq + a) * p.slots + split, ql, lg, acc, m_run, l_run);
}

// ---------------------------------------------------------------------------
// head_dim 128, G = 4 or 8 query heads per kv head: the workgroup's waves
// share every 32-key chunk through LDS. Each chunk (K rows, then V^T rows:
// 16 KB) is loaded once by direct global->LDS loads into a ring of
// kRingSlots slots, kRingSlots - 1 chunks in flight, instead of once per
// wave into registers with one chunk in flight. Each wave issues 16 / G of a
// chunk's sixteen 1 KB loads; a barrier per chunk makes the chunk visible to
// all waves and frees the slot read in the previous step. In a K slot,
// 16-byte chunk c of key row k sits at c ^ kswz(k), kswz(k) = (k & 3) |
// ((k >> 3) & 3) << 2: the sixteen keys an A-fragment read touches map to
// sixteen distinct bank groups. In a V slot (dim rows of 64 bytes), key chunk
// kc of dim d sits at kc ^ ((d >> 2) & 3). The math per chunk is
// process_chunk's. Past the split's last chunk the loads re-read that chunk
// (in-bounds, unread), so every wait is an exact count.
constexpr int kRingSlots = 4;
constexpr int kSlotBytes = 2 * 32 * 128 * 2;  // K rows then V^T rows of one chunk

__device__ __forceinline__ int kswz(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }

template <int N>
__device__ __forceinline__ void attn_wait_vm() {
  // vmcnt <= N, the other counters open
  __builtin_amdgcn_s_waitcnt(((N & 15) | ((N >> 4) << 14)) | 0xF70);
}

// 16 fragment reads of one slot (8 K, 8 V), complete on return, in one
// inline-assembly block (the compiler would otherwise wait for every direct
// load in flight into the other slots before each read, and must not touch
// the results before the closing wait). K rows of score tile 1 sit 1 KB after
// those of tile 0 and V rows of dim tile h 1 KB * h after tile 0, so four K
// addresses and one V address with immediate offsets cover all reads.
__device__ __forceinline__ void slot_read(Chunk<128>& c, uint32_t base, const uint32_t (&ko)[4],
                                          uint32_t vo) {
  u32x4 k[8], v[8];
  asm volatile(
      "ds_read_b128 %0, %16\n\t"
      "ds_read_b128 %1, %17\n\t"
      "ds_read_b128 %2, %18\n\t"
      "ds_read_b128 %3, %19\n\t"
      "ds_read_b128 %4, %16 offset:1024\n\t"
      "ds_read_b128 %5, %17 offset:1024\n\t"
      "ds_read_b128 %6, %18 offset:1024\n\t"
      "ds_read_b128 %7, %19 offset:1024\n\t"
      "ds_read_b128 %8, %20\n\t"
      "ds_read_b128 %9, %20 offset:1024\n\t"
      "ds_read_b128 %10, %20 offset:2048\n\t"
      "ds_read_b128 %11, %20 offset:3072\n\t"
      "ds_read_b128 %12, %20 offset:4096\n\t"
      "ds_read_b128 %13, %20 offset:5120\n\t"
      "ds_read_b128 %14, %20 offset:6144\n\t"
      "ds_read_b128 %15, %20 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
        "=&v"(k[6]), "=&v"(k[7]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
        "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(base + ko[0]), "v"(base + ko[1]), "v"(base + ko[2]), "v"(base + ko[3]),
        "v"(base + vo)
      : "memory");
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) c.kf[t][ks] = __builtin_bit_cast(bf16x8, k[t * 4 + ks]);
#pragma unroll
  for (int h = 0; h < 8; ++h) c.v[h] = v[h];
}

template <int G>
__global__ void __launch_bounds__(G * 64)
attn_lds(AttnArgs p) {
  constexpr int HD = 128, KSTEPS = 4, HT = 8;
  constexpr int NQ = 16 / G;  // load instructions per wave and chunk
  static_assert(16 % G == 0, "whole load instructions per wave");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRingSlots][kSlotBytes];
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int a = g * G + w;
  const int ql = lane & 15, lg = lane >> 4;
  if (p.blk_wg && split == p.splits) {  // the block's own keys (whole workgroup)
    block_partial<HD>(p, s, g, a, ql, lg);
    return;
  }
  const SeqDesc sd = p.seqs.s[s];
  const int kb = split * p.kps;
  const size_t plane = (size_t)sd.cap * HD;
  const bf16_t* kbase = sd.kv + (size_t)((2 * p.layer) * p.Hkv + g) * plane;
  const bf16_t* vbase = sd.kv + (size_t)((2 * p.layer + 1) * p.Hkv + g) * plane;

  // Load instruction q of a chunk: K rows 4q .. 4q+3 (256 bytes each) for q
  // < 8, else V^T rows (dims) 16(q-8) .. +15 (64 bytes each). A wave's
  // instructions are all of one kind; each lane's address for chunk start
  // c0 is a fixed per-lane pointer plus c0 * HD (K) or c0 (V^T).
  const bool kload = w * NQ < 8;  // wave-uniform
  const bf16_t* lp[NQ];
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int q = w * NQ + u;
    if (kload) {
      const int kl = 4 * q + (lane >> 4);
      lp[u] = kbase + (size_t)kl * HD + (((lane & 15) ^ kswz(kl)) << 3);
    } else {
      const int d = 16 * (q - 8) + (lane >> 2);
      lp[u] = vbase + (size_t)d * sd.cap + 8 * ((lane & 3) ^ ((d >> 2) & 3));
    }
  }
  // chunk j of the split into slot j % kRingSlots; jj: the chunk actually
  // read. Its start is clamped to cap - 32 (cap is a multiple of 64): a
  // chunk of the range starts at most there anyway, and the reads issued
  // before the range is known (or for an empty split) stay in the planes.
  auto issue = [&](int j, int jj) {
    const int c0 = min(kb + 32 * jj, sd.cap - 32);
    const size_t step = kload ? (size_t)c0 * HD : (size_t)c0;
    uint8_t* slot = &ring[j % kRingSlots][0];
#pragma unroll
    for (int u = 0; u < NQ; ++u) dma16(lp[u] + step, slot + (w * NQ + u) * 1024);
  };
  // queries and the context length first: a wait for them then leaves the
  // ring's loads, issued after them, in flight
  bf16x8 qf[KSTEPS], qfl[KSTEPS];
  const bool qv = ql < p.Bl;
  const size_t qoff = ((size_t)(s * p.Bl + (qv ? ql : 0)) * p.Hq + a) * HD + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = qv ? ld_bf16x8(p.q + qoff + ks * 32) : zero_bf16x8();
    qfl[ks] = qv ? ld_bf16x8(p.q_lo + qoff + ks * 32) : zero_bf16x8();
  }
  const int n_keys = seq_len(p.seqs, s);  // context keys only
  constexpr int R = kRingSlots;
#pragma unroll
  for (int j = 0; j < R - 1; ++j) issue(j, j);
  attn_wait_vm<NQ * (R - 1)>();  // queries and length in, the ring's loads in flight

  // fragment offsets inside a slot (lane-dependent, the same for every
  // slot): A row ql of score tile 0 is key kl, that of tile 1 key kl + 4
  // (same swizzle, 1 KB further); the V row of dim 16 h + ql is 1 KB * h
  // after that of dim ql (same swizzle)
  uint32_t ko[KSTEPS];
  const int kl0 = 8 * (ql >> 2) + (ql & 3);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) ko[ks] = kl0 * 256 + (((4 * ks + lg) ^ kswz(kl0)) << 4);
  const uint32_t vo = 8192 + ql * 64 + ((lg ^ ((ql >> 2) & 3)) << 4);

  const int ke = split == p.splits - 1 ? n_keys : min(kb + p.kps, n_keys);
  const int nch = ke > kb ? (ke - kb + 31) / 32 : 0;

  f32x4 acc[HT];
#pragma unroll
  for (int h = 0; h < HT; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[0][0];
  for (int i = 0; i < nch; ++i) {
    // this wave's loads of chunk i are done (R - 2 chunks issued after it),
    // then everyone's; past the barrier nobody reads slot (i - 1) % R
    attn_wait_vm<NQ * (R - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(i + R - 1, min(i + R - 1, nch - 1));
    Chunk<HD> c;
    slot_read(c, ring0 + (uint32_t)((i % R) * kSlotBytes), ko, vo);
    process_chunk<HD>(c, kb + 32 * i, ke, qf, qfl, p.scale_log2, lg, m_run, l_run, acc);
  }
  // no direct load may still be writing the ring when the workgroup ends
  attn_wait_vm<0>();
  l_run = rows4_sum(l_run);
  write_partial<HD>(p, (size_t)(s * p.Hq + a) * p.slots + split, ql, lg, acc, m_run, l_run);
}

// Merge of a head's partials, one thread per (block row, query head, dim):
// with M the largest of the partials' running maxima,
//   o = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k.
// The block's own keys (the last slot; never empty, so M is finite) are
// requested together with the first NB context splits, and the splits are
// taken in order, NB per batch, folded into a running max (an empty split
// has m = -inf and weight 0). The threads of a (row, head) read the same
// (m, l) words, one request per wave. Scores are in log2 units (scaled by
// log2(e)/sqrt(hd)), as in the split kernels.
struct MergeArgs {
  const float* acc;
  const float* ml;
  int Hq, Bl, splits, n_rows;  // splits: context splits (slots: splits + 1)
  bf16_t *ob_h, *ob_l;
};
template <int HD, int NB>
__global__ void __launch_bounds__(256)
attn_merge(MergeArgs p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int rh = t / HD, d = t % HD;  // rh = row * Hq + head
  if (rh >= p.n_rows * p.Hq) return;
  const int row = rh / p.Hq, a = rh % p.Hq;
  const int s = row / p.Bl, r = row % p.Bl;
  const size_t slot0 = (size_t)(s * p.Hq + a) * (p.splits + 1);
  const float* pa = p.acc + (slot0 * 16 + r) * HD + d;
  const float* pm = p.ml + (slot0 * 16 + r) * 2;
  const size_t blk = (size_t)p.splits;
  // the block's partial
  float M = pm[blk * 32], L = pm[blk * 32 + 1], o = pa[blk * 16 * HD];
  const int last = p.splits - 1;
  for (int k0 = 0; k0 < p.splits; k0 += NB) {
    float mk[NB], lk[NB], ak[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const size_t kk = (size_t)min(k0 + k, last);
      mk[k] = pm[kk * 32];
      lk[k] = pm[kk * 32 + 1];
      ak[k] = pa[kk * 16 * HD];
    }
    float bm = M;
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (k0 + k < p.splits) bm = fmaxf(bm, mk[k]);
    const float c = __builtin_amdgcn_exp2f(M - bm);
    L *= c;
    o *= c;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float wk = (k0 + k < p.splits && mk[k] != -INFINITY) ? __builtin_amdgcn_exp2f(mk[k] - bm) : 0.f;
      L += wk * lk[k];
      o += wk * ak[k];
    }
    M = bm;
  }
  const size_t i = (size_t)rh * HD + d;
  split_bf16(o / L, p.ob_h[i], p.ob_l[i]);
}

// Merge that also takes the block's own keys (used when the context splits
// are short, where a separate workgroup for the block would lengthen the
// attention launch): one workgroup per (block row, query head, sequence),
// one thread per output dim (at least one wave). Each thread first requests its dim of the first
// MB split accumulators and of the block's Bl fp32 values (clamped
// indices, straight-line loads). Wave 0 then forms the block scores: lane
// 4j + t holds a quarter of the dims of block key j and of the query (hi +
// lo), so one dot product of HD/4 terms and two lane exchanges give q.k_j.
// The same wave holds split k's (m, l) in lane k (and k + 64), takes the
// running max over the splits and the block scores, and the normaliser
//   L = sum_k 2^(m_k - M) l_k + sum_j 2^(s_j - M),
// with one wave reduction each, and leaves each split's weight
// 2^(m_k - M) / L and the block keys' weights 2^(s_j - M) / L in LDS.
// Scores are in log2 units (scaled by log2(e)/sqrt(hd)), as in the split
// kernels.
static_assert(kAttnMaxSplits <= 128, "two splits per lane of wave 0");
struct MergeBlkArgs {
  const float* acc;
  const float* ml;
  const bf16_t *q, *q_lo;     // [M][Hq][hd]
  const float *blk_k, *blk_v; // [M][Hkv][hd]
  int Hq, Hkv, Bl, splits;
  float scale_log2;
  bf16_t *ob_h, *ob_l;
};
// MB: split accumulators requested per batch (8 when the splits are that
// few, so that no loads of clamped duplicates are issued)
template <int HD, int MB>
__global__ void __launch_bounds__(HD < 64 ? 64 : HD)
attn_merge_blk(MergeBlkArgs p) {
  constexpr int kMergeBatch = MB;
  constexpr int STRIDE = 16 * HD;  // floats between the splits of one (row, dim)
  constexpr int DPL = HD / 4;      // dims per lane of a block score
  static_assert(DPL % 4 == 0, "whole float4 pieces of a key per lane");
  const int r = blockIdx.x, a = blockIdx.y, s = blockIdx.z;
  const int d = threadIdx.x, lane = d & 63, w = d >> 6;
  const int g = a / (p.Hq / p.Hkv);
  const int dc = d < HD ? d : HD - 1;
  __shared__ float wts[kAttnMaxSplits];
  __shared__ float bw[16];
  const size_t slot0 = (size_t)(s * p.Hq + a) * p.splits;
  const float* pb = p.acc + (slot0 * 16 + r) * HD + dc;
  const int last = p.splits - 1;
  float v[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) v[k] = pb[(size_t)min(k, last) * STRIDE];
  const size_t kvd = (size_t)p.Hkv * HD;
  float vb[16];
  {
    const float* vr = p.blk_v + (size_t)s * p.Bl * kvd + (size_t)g * HD + dc;
#pragma unroll
    for (int j = 0; j < 16; ++j) vb[j] = vr[(size_t)(j < p.Bl ? j : p.Bl - 1) * kvd];
  }
  if (w == 0) {
    const int j = lane >> 2, part = lane & 3;
    const int jj = j < p.Bl ? j : p.Bl - 1;
    const float4* kr = reinterpret_cast<const float4*>(
        p.blk_k + (size_t)(s * p.Bl + jj) * kvd + (size_t)g * HD + part * DPL);
    const size_t qi = ((size_t)(s * p.Bl + r) * p.Hq + a) * HD + part * DPL;
    float4 kv4[DPL / 4];
#pragma unroll
    for (int i = 0; i < DPL / 4; ++i) kv4[i] = kr[i];
    uint2 qh2[DPL / 4], ql2[DPL / 4];  // four bf16 per piece
#pragma unroll
    for (int i = 0; i < DPL / 4; ++i) {
      qh2[i] = *reinterpret_cast<const uint2*>(p.q + qi + 4 * i);
      ql2[i] = *reinterpret_cast<const uint2*>(p.q_lo + qi + 4 * i);
    }
    float mk[2], lk[2];
#pragma unroll
    for (int jx = 0; jx < 2; ++jx) {
      const int k = lane + 64 * jx;
      const bool in = k < p.splits;
      mk[jx] = in ? p.ml[((slot0 + k) * 16 + r) * 2] : -INFINITY;
      lk[jx] = in ? p.ml[((slot0 + k) * 16 + r) * 2 + 1] : 0.f;
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DPL / 4; ++i) {
      const uint32_t hw[2] = {qh2[i].x, qh2[i].y}, lw[2] = {ql2[i].x, ql2[i].y};
      const float kk[4] = {kv4[i].x, kv4[i].y, kv4[i].z, kv4[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t hb = e & 1 ? hw[e >> 1] & 0xffff0000u : hw[e >> 1] << 16;
        const uint32_t lb = e & 1 ? lw[e >> 1] & 0xffff0000u : lw[e >> 1] << 16;
        dot += (__uint_as_float(hb) + __uint_as_float(lb)) * kk[e];
      }
    }
    dot = quad_sum(dot);
    const float sj = j < p.Bl ? dot * p.scale_log2 : -INFINITY;
    const float M = wave_max(fmaxf(fmaxf(mk[0], mk[1]), sj));  // finite: Bl >= 1
    float e[2];
#pragma unroll
    for (int jx = 0; jx < 2; ++jx) e[jx] = mk[jx] == -INFINITY ? 0.f : exp2f(mk[jx] - M);
    const float pj = (part == 0 && j < p.Bl) ? exp2f(sj - M) : 0.f;
    const float inv = 1.f / wave_sum(e[0] * lk[0] + e[1] * lk[1] + pj);
#pragma unroll
    for (int jx = 0; jx < 2; ++jx) {
      const int k = lane + 64 * jx;
      if (k < p.splits) wts[k] = e[jx] * inv;
    }
    if (part == 0) bw[j] = pj * inv;
  }
  __syncthreads();
  float o = 0.f;
  for (int k0 = 0; k0 < p.splits; k0 += kMergeBatch) {
    if (k0) {
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) v[k] = pb[(size_t)min(k0 + k, last) * STRIDE];
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) o += (k0 + k < p.splits ? wts[k0 + k] : 0.f) * v[k];
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) o += bw[j] * vb[j];  // zero weight past Bl
  if (d < HD) {
    const size_t i = ((size_t)(s * p.Bl + r) * p.Hq + a) * HD + d;
    split_bf16(o, p.ob_h[i], p.ob_l[i]);
  }
}

template <int HD>
static hipError_t launch_attn_hd(const DraftLaunch& L, int layer, hipStream_t st) {
  AttnArgs p;
  p.q = L.q; p.q_lo = L.q_lo; p.acc = L.att_acc; p.ml = L.att_ml;
  p.blk_k = L.blk_k; p.blk_v = L.blk_v;
  p.Hq = L.Hq; p.Hkv = L.Hkv; p.Bl = L.Bl; p.layer = layer;
  p.splits = L.att_splits; p.kps = L.att_keys_per_split;
  p.blk_wg = L.att_blk_wg ? 1 : 0; p.slots = L.att_splits + p.blk_wg;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)HD));
  p.seqs = *L.seqs;
  const int G = L.Hq / L.Hkv;
  const dim3 grid(p.slots, L.Hkv, L.n_seqs);
  // G query-head waves; groups of one or two heads also get two key columns.
  // Up to 256 threads per workgroup keep two register stages (the next chunk
  // in flight while one is processed); 512-thread groups of head_dim 128
  // keep one, as two would not fit the 256 registers a wave gets there.
  constexpr bool P2 = HD < 128;
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_split<HD, 1, 2, true>), grid, dim3(128), 0, st, p); break;
    case 2: hipLaunchKernelGGL((attn_split<HD, 2, 2, true>), grid, dim3(256), 0, st, p); break;
    case 4:
      if constexpr (HD == 128)
        hipLaunchKernelGGL((attn_lds<4>), grid, dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((attn_split<HD, 4, 1, true>), grid, dim3(256), 0, st, p);
      break;
    case 8:
      if constexpr (HD == 128)
        hipLaunchKernelGGL((attn_lds<8>), grid, dim3(512), 0, st, p);
      else
        hipLaunchKernelGGL((attn_split<HD, 8, 1, P2>), grid, dim3(512), 0, st, p);
      break;
    case 16: hipLaunchKernelGGL((attn_split<HD, 16, 1, false>), grid, dim3(1024), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!p.blk_wg) {
    MergeBlkArgs m;
    m.acc = L.att_acc; m.ml = L.att_ml; m.q = L.q; m.q_lo = L.q_lo; m.blk_k = L.blk_k; m.blk_v = L.blk_v;
    m.Hq = L.Hq; m.Hkv = L.Hkv; m.Bl = L.Bl; m.splits = L.att_splits; m.scale_log2 = p.scale_log2;
    m.ob_h = L.ob_h; m.ob_l = L.ob_l;
    if (L.att_splits <= 8)
      hipLaunchKernelGGL((attn_merge_blk<HD, 8>), dim3(L.Bl, L.Hq, L.n_seqs), dim3(HD < 64 ? 64 : HD), 0, st, m);
    else
      hipLaunchKernelGGL((attn_merge_blk<HD, 32>), dim3(L.Bl, L.Hq, L.n_seqs), dim3(HD < 64 ? 64 : HD), 0, st, m);
    return hipGetLastError();
  }
  MergeArgs m;
  m.acc = L.att_acc; m.ml = L.att_ml; m.Hq = L.Hq; m.Bl = L.Bl; m.splits = L.att_splits;
  m.n_rows = L.n_seqs * L.Bl; m.ob_h = L.ob_h; m.ob_l = L.ob_l;
  const int blocks = (m.n_rows * L.Hq * HD + 255) / 256;
  // batches no wider than the splits need (a clamped duplicate is a request
  // too), at most 32
  if (m.splits <= 8)
    hipLaunchKernelGGL((attn_merge<HD, 8>), dim3(blocks), dim3(256), 0, st, m);
  else if (m.splits <= 16)
    hipLaunchKernelGGL((attn_merge<HD, 16>), dim3(blocks), dim3(256), 0, st, m);
  else
    hipLaunchKernelGGL((attn_merge<HD, 32>), dim3(blocks), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_attention(const DraftLaunch& L, int layer, hipStream_t st) {
  switch (L.hd) {
    case 16: return launch_attn_hd<16>(L, layer, st);
    case 32: return launch_attn_hd<32>(L, layer, st);
    case 64: return launch_attn_hd<64>(L, layer, st);
    case 128: return launch_attn_hd<128>(L, layer, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dfl
