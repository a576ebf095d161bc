// The context-side GEMMs of the prefill on the tiled MFMA kernel of
// tiled_gemm.h.
//
// A is read through a segmented loader so the fusion GEMM never materialises
// the concatenation of the target layers (A3-dflash tutorial, section 2.1.1:
// concat along the hidden axis): k in [j*D, (j+1)*D) reads layer j's array.
//
// Epilogues run on 64-row slices of the fp32 tile staged through LDS:
//   fuse   - y in fp32 plus per-(row, 256-column tile) sums of y^2; a second
//            kernel applies RMSNorm and the gain and rounds to bf16 once
//            (tutorial section 2.1.2);
//   inject - every draft layer's K (RoPE at position pos0 + row) and V,
//            written into the KV-cache layout (txtmix article section 5).
#include "common.h"
#include "launch.h"
#include "tiled_gemm.h"

namespace dfl {

struct EpiFuse {
  static constexpr bool kStack = false;
  struct P {
    const bf16_t* w;  // [N][K]
    int K, N;
    float* y;         // [M][N] fp32, normalised and rounded once afterwards
    float* ssq;       // [M][n_tiles]
    int n_tiles;
  };
  __device__ static const bf16_t* wrow(const P& p, int n) { return p.w + (size_t)n * p.K; }
  __device__ static void prologue(const P&, int, int, int) {}
  // rows [m0, m0 + kSlice) of the tile starting at column n0, C[r][c] at C[r * ld + c]
  template <int BN>
  __device__ static void run(const P& p, const float* C, int ld, int m0, int n0, int M) {
    // fp32 y, 4 columns (16 bytes) per thread-step where the row allows
    for (int e = threadIdx.x; e < kSlice * (BN / 4); e += blockDim.x) {
      const int r = e / (BN / 4), c = 4 * (e % (BN / 4));
      const int m = m0 + r, n = n0 + c;
      if (m >= M || n >= p.N) continue;
      const float* y = C + r * ld + c;
      float* dst = p.y + (size_t)m * p.N + n;
      if (n + 4 <= p.N && (p.N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
      } else {
        for (int h = 0; h < 4 && n + h < p.N; ++h) dst[h] = y[h];
      }
    }
    // per-row sum of squares over the tile's columns: 8 lanes per row
    for (int e = threadIdx.x; e < kSlice * 8; e += blockDim.x) {
      const int r = e >> 3, q = e & 7;
      float s = 0.f;
      for (int c = q; c < BN && n0 + c < p.N; c += 8) s += C[r * ld + c] * C[r * ld + c];
      s = row8_sum(s);
      const int m = m0 + r;
      if (q == 0 && m < M) p.ssq[(size_t)m * p.n_tiles + n0 / BN] = s;
    }
  }
};

// Virtual column order of the injection GEMM: per layer, the K columns then
// the V columns; inside a K head, groups of PW = min(hd, 64) columns each
// hold PW/2 RoPE pairs, virtual o and o + PW/2 being dims d and d + hd/2.
// Tiles are multiples of 64 columns wide, so a pair never straddles two.
struct InjectCol {
  int layer, head, dim;
  bool is_k;
};
__device__ __forceinline__ InjectCol inject_col(int vc, int Hkv, int hd) {
  const int kvd = Hkv * hd;
  InjectCol c;
  c.layer = vc / (2 * kvd);
  int r = vc - c.layer * 2 * kvd;
  c.is_k = r < kvd;
  if (!c.is_k) r -= kvd;
  c.head = r / hd;
  const int q = r - c.head * hd;
  if (c.is_k) {
    const int PW = hd < 64 ? hd : 64, hw = PW >> 1;
    const int s = q / PW, o = q - s * PW;
    c.dim = o < hw ? s * hw + o : (hd >> 1) + s * hw + (o - hw);
  } else {
    c.dim = q;
  }
  return c;
}

struct EpiInject {
  static constexpr bool kStack = false;
  struct P {
    const bf16_t* wk[kMaxLayers];
    const bf16_t* wv[kMaxLayers];
    int K, N;        // N = L * 2 * Hkv * hd
    int Hkv, hd, pos0, cap;
    double log2_theta;
    bf16_t* kv;
  };
  __device__ static const bf16_t* wrow(const P& p, int n) {
    const InjectCol c = inject_col(n, p.Hkv, p.hd);
    return (c.is_k ? p.wk[c.layer] : p.wv[c.layer]) + (size_t)(c.head * p.hd + c.dim) * p.K;
  }
  __device__ static void prologue(const P&, int, int, int) {}
  static constexpr int kVFlag = 1 << 16;  // column-table dim entries of V columns
  template <int BN>
  __device__ static void run(const P& p, const float* C, int ld, int m0, int n0, int M) {
    const size_t plane = (size_t)p.cap * p.hd;
    const int PW = p.hd < 64 ? p.hd : 64, hw = PW >> 1;
    // the tile's column table, in LDS after the slice (16 bytes a column),
    // once per slice: plane index (-1 past N), dim (| kVFlag for V), RoPE
    // frequency in revolutions per position; the per-element work is then a
    // table read, an fp64 product reduced to [-1/2, 1/2] revolution and the
    // hardware sine and cosine
    int* col_plane = reinterpret_cast<int*>(const_cast<float*>(C) + kSlice * ld);
    int* col_dim = col_plane + BN;
    double* col_inv = reinterpret_cast<double*>(col_dim + BN);
    for (int c = threadIdx.x; c < BN; c += blockDim.x) {
      const int n = n0 + c;
      if (n < p.N) {
        const InjectCol ci = inject_col(n, p.Hkv, p.hd);
        col_plane[c] = (2 * ci.layer + (ci.is_k ? 0 : 1)) * p.Hkv + ci.head;
        col_dim[c] = ci.dim | (ci.is_k ? 0 : kVFlag);
        col_inv[c] = ci.is_k ? rope_rev_freq(ci.dim, p.hd, p.log2_theta) : 0.0;
      } else {
        col_plane[c] = -1;
      }
    }
    __syncthreads();
    // K: octets of pair slots (the slots of column group g cover virtual
    // columns g*PW + o and g*PW + o + PW/2, o < hw); an octet is eight
    // consecutive dims of one head (hw is a multiple of 8), rotated and
    // stored as two 16-byte pieces of the position's row. A wave takes the
    // octets of one column group on consecutive rows, and each thread reads
    // the two 16-byte halves of an octet in the order of its lane's parity:
    // with the slice's row pitch at 8 words mod 64, one read instruction then
    // starts at 16 distinct bank quartets (octets of one row side by side
    // started at only the 8 multiples of 8, a 15-way conflict). The halves
    // are 16-byte aligned: the pitch (the tile width + 8) is a multiple of 4.
    const int hd2 = p.hd >> 1;
    const int opg = hw >> 3;  // octets per column group
    for (int e = threadIdx.x; e < kSlice * (BN / 16); e += blockDim.x) {
      const int oi = e % opg, r = (e / opg) % kSlice, g = e / (opg * kSlice);
      const int c1 = g * PW + 8 * oi, c2 = c1 + hw;
      const int m = m0 + r;
      const int pl = col_plane[c1], dv = col_dim[c1];
      if (m >= M || pl < 0 || (dv & kVFlag)) continue;
      const int pos = p.pos0 + m, d = dv;
      const int h = e & 1;
      const float4* q1 = reinterpret_cast<const float4*>(C + r * ld + c1);
      const float4* q2 = reinterpret_cast<const float4*>(C + r * ld + c2);
      const float4 a0 = q1[h], a1 = q1[h ^ 1], b0 = q2[h], b1 = q2[h ^ 1];
      const float4 x1l = h ? a1 : a0, x1h = h ? a0 : a1, x2l = h ? b1 : b0, x2h = h ? b0 : b1;
      const float x1[8] = {x1l.x, x1l.y, x1l.z, x1l.w, x1h.x, x1h.y, x1h.z, x1h.w};
      const float x2[8] = {x2l.x, x2l.y, x2l.z, x2l.w, x2h.x, x2h.y, x2h.z, x2h.w};
      float o1[8], o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float cs, sn;
        rope_cs_rev(pos, col_inv[c1 + i], cs, sn);
        o1[i] = x1[i] * cs - x2[i] * sn;
        o2[i] = x2[i] * cs + x1[i] * sn;
      }
      bf16_t* kp = p.kv + (size_t)pl * plane + (size_t)pos * p.hd;
      *reinterpret_cast<bf16x8*>(kp + d) = pack_bf16x8(o1);
      *reinterpret_cast<bf16x8*>(kp + d + hd2) = pack_bf16x8(o2);
    }
    // V (dim-major planes: a dim's positions are contiguous): eight
    // consecutive rows of one column per thread, one 16-byte store where the
    // position allows (two 8-byte ones at a multiple of 4); eight threads
    // cover a column's 64 rows
    for (int e = threadIdx.x; e < (kSlice / 8) * BN; e += blockDim.x) {
      const int c = e / (kSlice / 8), r = 8 * (e % (kSlice / 8));
      const int pl = col_plane[c], dv = col_dim[c];
      const int m = m0 + r;
      if (m >= M || pl < 0 || !(dv & kVFlag)) continue;
      const int pos = p.pos0 + m;
      bf16_t* vp = p.kv + (size_t)pl * plane + (size_t)(dv & (kVFlag - 1)) * p.cap + pos;
      const float* x = C + r * ld + c;
      if (m + 8 <= M && (pos & 7) == 0) {
        *reinterpret_cast<u32x4*>(vp) = u32x4{f2bf2(x[0], x[ld]), f2bf2(x[2 * ld], x[3 * ld]),
                                              f2bf2(x[4 * ld], x[5 * ld]), f2bf2(x[6 * ld], x[7 * ld])};
      } else if (m + 8 <= M && (pos & 3) == 0) {
        *reinterpret_cast<uint2*>(vp) = make_uint2(f2bf2(x[0], x[ld]), f2bf2(x[2 * ld], x[3 * ld]));
        *reinterpret_cast<uint2*>(vp + 4) = make_uint2(f2bf2(x[4 * ld], x[5 * ld]), f2bf2(x[6 * ld], x[7 * ld]));
      } else {
        for (int i = 0; i < 8 && m + i < M; ++i) vp[i] = f2bf(x[i * ld]);
      }
    }
  }
};

size_t ctx_gemm_part_floats() { return (size_t)256 * BM * 320; }

// H_t row m = bf16(y[m] * rsqrt(mean(y[m]^2) + eps) * gain): the fp32
// projection is rounded to bf16 once, here. With out_lo the row is kept as a
// bf16 hi/lo pair instead (out = hi).
__global__ void __launch_bounds__(256)
fuse_normalize(bf16_t* __restrict__ out, bf16_t* __restrict__ out_lo, const float* __restrict__ y,
               const float* __restrict__ ssq, int n_tiles, int D, const bf16_t* __restrict__ gain,
               float eps) {
  const int m = blockIdx.x;
  __shared__ float rs;
  if (threadIdx.x < 64) {
    float s = 0.f;
    for (int t = threadIdx.x; t < n_tiles; t += 64) s += ssq[(size_t)m * n_tiles + t];
    s = wave_sum(s);
    if (threadIdx.x == 0) rs = rsqrtf(s / (float)D + eps);
  }
  __syncthreads();
  const float r = rs;
  // D is a multiple of 64: 4 columns per thread-step
  const float* yr = y + (size_t)m * D;
  bf16_t* orow = out + (size_t)m * D;
  for (int n = 4 * threadIdx.x; n < D; n += 4 * 256) {
    const float4 v = *reinterpret_cast<const float4*>(yr + n);
    const uint2 g = *reinterpret_cast<const uint2*>(gain + n);
    const float g0 = bf2f((bf16_t)(g.x & 0xffff)), g1 = bf2f((bf16_t)(g.x >> 16));
    const float g2 = bf2f((bf16_t)(g.y & 0xffff)), g3 = bf2f((bf16_t)(g.y >> 16));
    const float h0 = v.x * r * g0, h1 = v.y * r * g1, h2 = v.z * r * g2, h3 = v.w * r * g3;
    const uint2 hi = make_uint2(f2bf2(h0, h1), f2bf2(h2, h3));
    *reinterpret_cast<uint2*>(orow + n) = hi;
    if (out_lo) {
      const float l0 = h0 - __uint_as_float(hi.x << 16), l1 = h1 - __uint_as_float(hi.x & 0xffff0000u);
      const float l2 = h2 - __uint_as_float(hi.y << 16), l3 = h3 - __uint_as_float(hi.y & 0xffff0000u);
      *reinterpret_cast<uint2*>(out_lo + (size_t)m * D + n) = make_uint2(f2bf2(l0, l1), f2bf2(l2, l3));
    }
  }
}

hipError_t launch_fuse(const FuseLaunch& F, hipStream_t st) {
  GemmA a;
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = i < F.n_feat ? F.feats[i] : F.feats[0];
  a.ld = F.ld; a.seg_k = F.D; a.M = F.T; a.K = F.n_feat * F.D;
  gemm_a_plain(a);
  EpiFuse::P p;
  p.w = F.w_c; p.K = a.K; p.N = F.D; p.y = F.y; p.ssq = F.ssq;
  p.n_tiles = (F.D + kFuseTileN - 1) / kFuseTileN;
  hipError_t e = launch_tiled<kFuseTileN, EpiFuse>(a, p, F.D, F.gemm, st);
  if (e != hipSuccess) return e;
  return launch_fuse_normalize(F.out, F.out_lo, F.y, F.ssq, p.n_tiles, F.T, F.D, F.gain, F.eps, st);
}

hipError_t launch_fuse_normalize(bf16_t* out, bf16_t* out_lo, const float* y, const float* ssq,
                                 int n_parts, int T, int D, const bf16_t* gain, float eps,
                                 hipStream_t st) {
  hipLaunchKernelGGL(fuse_normalize, dim3(T), dim3(256), 0, st, out, out_lo, y, ssq, n_parts, D,
                     gain, eps);
  return hipGetLastError();
}

hipError_t launch_inject(const InjectLaunch& I, hipStream_t st) {
  GemmA a;
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = I.ctx;
  a.ld = I.D; a.seg_k = I.D; a.M = I.T; a.K = I.D;
  gemm_a_plain(a);
  EpiInject::P p;
  for (int i = 0; i < kMaxLayers; ++i) {
    p.wk[i] = i < I.L ? I.wk[i] : I.wk[0];
    p.wv[i] = i < I.L ? I.wv[i] : I.wv[0];
  }
  p.K = I.D; p.N = I.L * 2 * I.Hkv * I.hd; p.Hkv = I.Hkv; p.hd = I.hd; p.pos0 = I.pos0;
  p.cap = I.cap; p.log2_theta = I.log2_theta; p.kv = I.kv;
  if (p.N % 320 == 0) return launch_tiled<320, EpiInject>(a, p, p.N, I.gemm, st);
  return launch_tiled<256, EpiInject>(a, p, p.N, I.gemm, st);
}

}  // namespace dfl
