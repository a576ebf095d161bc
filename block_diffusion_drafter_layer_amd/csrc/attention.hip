// Block attention of the draft forward: every block row of a sequence attends,
// with no mask, to the sequence's context K/V followed by the block's own K/V
// (txtmix article section 5: k = cat(k_ctx, k_noise); section 6: the
// full-attention draft layers are not causal). Grouped-query heads: query
// head a reads kv head a / G.
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
// bf16 rounding left in attention is the KV cache's own storage format.
#include "common.h"
#include "launch.h"

namespace dfl {

struct AttnArgs {
  const bf16_t* q;       // [M][Hq][HD] after RoPE, hi
  const bf16_t* q_lo;    // lo
  float* acc;            // [(s*Hq + a)*splits + split][16][HD]
  float* ml;             // [(s*Hq + a)*splits + split][16][2]
  int Hq, Hkv, Bl, layer, splits, kps;
  float scale_log2;      // log2(e) / sqrt(HD)
  SeqTable seqs;
};

template <int HD, int MAXG>
__global__ void __launch_bounds__(MAXG * 64)
attn_split(AttnArgs p) {
  constexpr int KSTEPS = (HD + 31) / 32;  // head_dim 16 pads k to 32 with zeros
  constexpr int HT = HD / 16;
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int a = g * G + w;
  const int ql = lane & 15, lg = lane >> 4;
  const SeqDesc sd = p.seqs.s[s];
  const int n_keys = sd.len + p.Bl;
  const int kb = split * p.kps;
  const int ke = min(kb + p.kps, n_keys);
  const size_t plane = (size_t)sd.cap * HD;
  const bf16_t* kbase = sd.kv + (size_t)((2 * p.layer) * p.Hkv + g) * plane;
  const bf16_t* vbase = sd.kv + (size_t)((2 * p.layer + 1) * p.Hkv + g) * plane;

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

  for (int c0 = kb; c0 < ke; c0 += 32) {
    // issue this chunk's K and V loads together; V does not depend on the
    // scores. Lane group lg holds keys c0 + 8*lg .. +7 of both.
    const int kl = c0 + 8 * lg;
    const int kl_ld = kl < n_keys ? kl : 0;  // in-bounds address, masked below
    const int nvalid = ke - kl;
    bf16x8 kf[2][KSTEPS];
    u32x4 vraw[HT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int key = c0 + (ql >> 2) * 8 + t * 4 + (ql & 3);
      key = key < n_keys ? key : n_keys - 1;
      const bf16_t* kr = kbase + (size_t)key * HD + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        kf[t][ks] = (ks * 32 + 8 * lg < HD) ? ld_bf16x8(kr + ks * 32) : zero_bf16x8();
    }
#pragma unroll
    for (int h = 0; h < HT; ++h)
      vraw[h] = *reinterpret_cast<const u32x4*>(vbase + (size_t)(h * 16 + ql) * sd.cap + kl_ld);

    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        st[t] = mfma16x16x32(kf[t][ks], qf[ks], st[t]);
        st[t] = mfma16x16x32(kf[t][ks], qfl[ks], st[t]);
      }
    }
    float sc[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = (kl + 4 * t + e < ke) ? st[t][e] * p.scale_log2 : -INFINITY;
        sc[4 * t + e] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    float pr[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = exp2f(sc[i] - m_new);
      psum += pr[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    float prl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) prl[i] = pr[i] - bf2f(f2bf(pr[i]));
    const bf16x8 pf = pack_bf16x8(pr);
    const bf16x8 pfl = pack_bf16x8(prl);

    // keys past the range (or past the cache) contribute zero V, never NaN
    uint32_t keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      keep[i] = ((2 * i < nvalid) ? 0x0000ffffu : 0u) | ((2 * i + 1 < nvalid) ? 0xffff0000u : 0u);
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      acc[h] *= alpha;
      u32x4 raw = vraw[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] &= keep[i];
      const bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
      acc[h] = mfma16x16x32(vf, pf, acc[h]);
      acc[h] = mfma16x16x32(vf, pfl, acc[h]);
    }
  }

  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  const size_t slot = ((size_t)(s * p.Hq + a) * p.splits + split);
  float* out = p.acc + slot * 16 * HD + (size_t)ql * HD;
#pragma unroll
  for (int h = 0; h < HT; ++h)
    *reinterpret_cast<f32x4*>(out + h * 16 + 4 * lg) = acc[h];
  if (lg == 0) {
    p.ml[(slot * 16 + ql) * 2 + 0] = m_run;
    p.ml[(slot * 16 + ql) * 2 + 1] = l_run;
  }
}

template <int HD>
__global__ void __launch_bounds__(256)
attn_merge(const float* acc, const float* ml, int Hq, int Bl, int splits,
           bf16_t* ob_h, bf16_t* ob_l) {
  const int a = blockIdx.x, s = blockIdx.y;
  __shared__ float sm[kAttnMaxSplits][16], sl[kAttnMaxSplits][16];
  __shared__ float wgt[kAttnMaxSplits][16];
  const size_t slot0 = (size_t)(s * Hq + a) * splits;
  // every (split, row) statistic is loaded by its own thread
  for (int e = threadIdx.x; e < splits * 16; e += 256) {
    const int k = e / 16, r = e % 16;
    sm[k][r] = ml[((slot0 + k) * 16 + r) * 2];
    sl[k][r] = ml[((slot0 + k) * 16 + r) * 2 + 1];
  }
  __syncthreads();
  if (threadIdx.x < Bl) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int k = 0; k < splits; ++k) M = fmaxf(M, sm[k][r]);
    float Lsum = 0.f;
    for (int k = 0; k < splits; ++k) {
      const float wk = sm[k][r] == -INFINITY ? 0.f : exp2f(sm[k][r] - M);
      wgt[k][r] = wk;
      Lsum += wk * sl[k][r];
    }
    const float inv = 1.f / Lsum;
    for (int k = 0; k < splits; ++k) wgt[k][r] *= inv;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Bl * HD; e += 256) {
    const int r = e / HD, d = e % HD;
    const float* src = acc + (slot0 * 16 + r) * HD + d;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;  // independent chains keep loads in flight
    int k = 0;
    for (; k + 4 <= splits; k += 4) {
      o0 += wgt[k][r] * src[(size_t)k * 16 * HD];
      o1 += wgt[k + 1][r] * src[(size_t)(k + 1) * 16 * HD];
      o2 += wgt[k + 2][r] * src[(size_t)(k + 2) * 16 * HD];
      o3 += wgt[k + 3][r] * src[(size_t)(k + 3) * 16 * HD];
    }
    for (; k < splits; ++k) o0 += wgt[k][r] * src[(size_t)k * 16 * HD];
    const float o = (o0 + o1) + (o2 + o3);
    const size_t i = ((size_t)(s * Bl + r) * Hq + a) * HD + d;
    split_bf16(o, ob_h[i], ob_l[i]);
  }
}

template <int HD>
static hipError_t launch_attn_hd(const DraftLaunch& L, int layer, hipStream_t st) {
  AttnArgs p;
  p.q = L.q; p.q_lo = L.q_lo; p.acc = L.att_acc; p.ml = L.att_ml;
  p.Hq = L.Hq; p.Hkv = L.Hkv; p.Bl = L.Bl; p.layer = layer;
  p.splits = L.att_splits; p.kps = L.att_keys_per_split;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)HD));
  p.seqs = *L.seqs;
  const int G = L.Hq / L.Hkv;
  const dim3 grid(L.att_splits, L.Hkv, L.n_seqs), block(G * 64);
  // the launch bound follows the group size so small groups keep the full
  // register file
  if (G <= 4)
    hipLaunchKernelGGL((attn_split<HD, 4>), grid, block, 0, st, p);
  else if (G <= 8)
    hipLaunchKernelGGL((attn_split<HD, 8>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((attn_split<HD, 16>), grid, block, 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge<HD>, dim3(L.Hq, L.n_seqs), dim3(256), 0, st, L.att_acc,
                     L.att_ml, L.Hq, L.Bl, L.att_splits, L.ob_h, L.ob_l);
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
