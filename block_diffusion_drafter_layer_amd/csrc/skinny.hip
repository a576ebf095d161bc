// Weight-streaming GEMMs of the draft forward (few activation rows, wide
// weights): Y[m][n] = sum_k X[m][k] W[n][k], X given as a bf16 hi/lo pair,
// W bf16 in nn.Linear [out, in] layout, read straight from HBM into MFMA
// operand registers (16 bytes per lane, no LDS staging). A workgroup owns
// 16*NCT columns; its waves interleave the 32-wide k steps of its K range and
// are reduced through LDS. Narrow matrices also split K over workgroups: each
// writes an fp32 partial tile and a second, small kernel sums the partials of
// a column block in split order (deterministic) and runs the epilogue. (A
// last-arriving-workgroup reduction inside one launch needs a device-scope
// fence per workgroup, which on this chip writes back and invalidates an XCD's
// L2 - far more costly than the extra launch.) Each use has its own epilogue:
//   qkv    - RMSNorm row scale, RoPE on q/k, q (bf16 hi/lo) and the block's
//            own k/v (fp32) to the workspace (txtmix article section 5: q
//            from the draft tokens, the block's k/v follow the context's);
//   resid  - o_proj / down_proj: x += y, the next RMSNorm's input (x*gain as a
//            bf16 hi/lo pair) and per-32-column sums of x^2;
//   swiglu - gate/up pairs: silu(g)*u (the decoder layer's SwiGLU MLP);
//   lm     - final RMSNorm row scale, optional logits, per-tile argmax keys
//            (txtmix article section 9: LM head on the rows after the anchor).
// Also here: the block embedding (section 6: anchor + mask tokens) and the
// argmax reduction that writes the drafted block.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiled_gemm.h"

namespace dfl {

struct SkinnyA {
  const bf16_t* xh;   // activations hi [rows_in, lda]
  const bf16_t* xl;   // activations lo (unused when the kernel has no lo half)
  int lda;
  // optional k-segmentation: k in [j*seg_k, (j+1)*seg_k) reads seg[j] (the
  // context fusion reads each target layer's array in place); seg_k = K and
  // seg[0] = xh otherwise
  const bf16_t* seg[kMaxFeat];
  int seg_k;
  int M;              // output rows
  int K;              // contraction length (multiple of 32)
  // output row m reads input row (m / a_group) * a_stride + a_off + m % a_group
  int a_group, a_stride, a_off;
  const float* ssq;   // optional: per-row partial sums of x^2 [rows_in][ssq_ld]
  int ssq_ld;
  float eps;
};

__device__ __forceinline__ int in_row(const SkinnyA& a, int m) {
  return (m / a.a_group) * a.a_stride + a.a_off + (m % a.a_group);
}

// dim of virtual column vi inside a head: each 16-wide group holds the dims
// 8t..8t+7 and hd/2+8t..hd/2+8t+7 so a RoPE pair shares a group
__device__ __forceinline__ int paired_dim(int vi, int hd) {
  int t = vi >> 4, j = vi & 15;
  return j < 8 ? (t << 3) + j : (hd >> 1) + (t << 3) + (j - 8);
}

// ---------------------------------------------------------------------------
// epilogues
// ---------------------------------------------------------------------------

struct EpiQKV {
  struct P {
    const bf16_t *wq, *wk, *wv;
    int D, Hq, Hkv, hd, Bl, layer;
    double log2_theta;
    bf16_t* q_out;     // [M][Hq*hd] hi
    bf16_t* q_lo;      // [M][Hq*hd] lo
    float* blk_k;      // [M][Hkv*hd] the block's own K after RoPE, fp32
    float* blk_v;      // [M][Hkv*hd] the block's own V, fp32
    SeqTable seqs;
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    const int qd = p.Hq * p.hd, kvd = p.Hkv * p.hd;
    // the three matrix pointers are read as values first: a choice between
    // the fields' addresses (what the compiler would otherwise form from the
    // branches below) makes it copy the whole argument block to scratch
    const bf16_t* wq = p.wq;
    const bf16_t* wk = p.wk;
    const bf16_t* wv = p.wv;
    asm volatile("" : "+s"(wq), "+s"(wk), "+s"(wv));
    if (vc < qd) {
      int h = vc / p.hd, d = paired_dim(vc % p.hd, p.hd);
      return wq + (size_t)(h * p.hd + d) * p.D;
    }
    vc -= qd;
    if (vc < kvd) {
      int h = vc / p.hd, d = paired_dim(vc % p.hd, p.hd);
      return wk + (size_t)(h * p.hd + d) * p.D;
    }
    vc -= kvd;
    return wv + (size_t)vc * p.D;
  }
  // row r8 of the 8-column group starting at vc8 (a multiple of 8): the
  // matrix and head follow from vc8 alone
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    const int qd = p.Hq * p.hd, kvd = p.Hkv * p.hd;
    if (vc8 < qd + kvd) {
      const bool is_q = vc8 < qd;
      const int vcl = is_q ? vc8 : vc8 - qd;
      const int h = vcl / p.hd;
      const int d = paired_dim(vcl % p.hd + r8, p.hd);
      return (is_q ? p.wq : p.wk) + (size_t)(h * p.hd + d) * p.D;
    }
    return p.wv + (size_t)(vc8 - qd - kvd + r8) * p.D;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs,
                             int vc0, int m0, int M) {
    const int qd = p.Hq * p.hd, kvd = p.Hkv * p.hd;
    constexpr int NG = VC / 16;
    // each row's position once, through LDS (read per element it would be a
    // load that every iteration waits for behind the previous iteration's
    // stores)
    __shared__ int r_pos[ROWS];
    // the rotation frequencies (revolutions per position) once per call (an
    // fp64 exp2 per element would cost more than the tall path's whole k loop)
    __shared__ double inv_f[kMaxHeadDim / 2];
    // sequences walked with a uniform index: a per-lane index into the
    // sequence table would make the compiler copy the whole table (kernel
    // arguments) into per-lane scratch memory
    const int s_end = (min(M, m0 + ROWS) + p.Bl - 1) / p.Bl;
    for (int sq = m0 / p.Bl; sq < s_end; ++sq) {
      const int len = seq_len(p.seqs, sq);
      const int ml = sq * p.Bl - m0 + (int)threadIdx.x;
      if (threadIdx.x < (unsigned)p.Bl && ml >= 0 && ml < ROWS && m0 + ml < M)
        r_pos[ml] = len + (int)threadIdx.x;
    }
    for (int d = threadIdx.x; d < p.hd / 2; d += blockDim.x)
      inv_f[d] = rope_rev_freq(d, p.hd, p.log2_theta);
    __syncthreads();
    // one thread per (row, 16-column group): the group's 8 RoPE pairs (or
    // 16 V dims) are contiguous in the outputs, so each output is written
    // with 16-byte stores
    for (int e = threadIdx.x; e < ROWS * NG; e += blockDim.x) {
      const int ml = e / NG, c = e % NG;
      const int m = m0 + ml;
      if (m >= M) continue;
      const int vc = vc0 + c * 16;
      if (vc >= qd + 2 * kvd) continue;
      const float r = rs[ml];
      float x1[8], x2[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x1[j] = tile[ml][c * 16 + j] * r;
        x2[j] = tile[ml][c * 16 + j + 8] * r;
      }
      if (vc < qd + kvd) {
        const bool is_q = vc < qd;
        const int vcl = is_q ? vc : vc - qd;
        const int h = vcl / p.hd;
        const int d0 = (vcl % p.hd) >> 1;  // group t covers dims 8t .. 8t+7
        const int pos = r_pos[ml];
        float o1[8], o2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float cs, sn;
          rope_cs_rev(pos, inv_f[d0 + j], cs, sn);
          o1[j] = x1[j] * cs - x2[j] * sn;
          o2[j] = x2[j] * cs + x1[j] * sn;
        }
        if (is_q) {
          const size_t qi = (size_t)m * qd + h * p.hd + d0;
          bf16x8 hi, lo;
          pack_split_bf16x8(o1, hi, lo);
          *reinterpret_cast<bf16x8*>(p.q_out + qi) = hi;
          *reinterpret_cast<bf16x8*>(p.q_lo + qi) = lo;
          pack_split_bf16x8(o2, hi, lo);
          *reinterpret_cast<bf16x8*>(p.q_out + qi + p.hd / 2) = hi;
          *reinterpret_cast<bf16x8*>(p.q_lo + qi + p.hd / 2) = lo;
        } else {
          float* k = p.blk_k + (size_t)m * kvd + h * p.hd + d0;
          *reinterpret_cast<float4*>(k) = make_float4(o1[0], o1[1], o1[2], o1[3]);
          *reinterpret_cast<float4*>(k + 4) = make_float4(o1[4], o1[5], o1[6], o1[7]);
          *reinterpret_cast<float4*>(k + p.hd / 2) = make_float4(o2[0], o2[1], o2[2], o2[3]);
          *reinterpret_cast<float4*>(k + p.hd / 2 + 4) = make_float4(o2[4], o2[5], o2[6], o2[7]);
        }
      } else {
        float* v = p.blk_v + (size_t)m * kvd + (vc - qd - kvd);  // dims vi .. vi + 15
        *reinterpret_cast<float4*>(v) = make_float4(x1[0], x1[1], x1[2], x1[3]);
        *reinterpret_cast<float4*>(v + 4) = make_float4(x1[4], x1[5], x1[6], x1[7]);
        *reinterpret_cast<float4*>(v + 8) = make_float4(x2[0], x2[1], x2[2], x2[3]);
        *reinterpret_cast<float4*>(v + 12) = make_float4(x2[4], x2[5], x2[6], x2[7]);
      }
    }
  }
};

struct EpiResid {
  struct P {
    const bf16_t* w;     // [N=D][K]
    int K, D;
    float* x;            // [M][D] residual stream, updated in place
    bf16_t *xh, *xl;     // [M][D] next RMSNorm input x*gain, hi/lo
    const bf16_t* gain;  // [D]
    float* ssq;          // [M][D/32]
    float* hidden;       // optional [M][D]
    int n_vcols;         // D
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    return p.w + (size_t)vc * p.K;
  }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return p.w + (size_t)(vc8 + r8) * p.K;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float*,
                             int vc0, int m0, int M) {
    static_assert(VC % 32 == 0, "whole 32-column norm groups per workgroup");
    // one thread per (row, 8 consecutive columns): x and the gain read and x,
    // the hidden copy and the next norm's hi/lo input written as 16- and
    // 32-byte pieces; the four threads of a 32-column norm group are a DPP
    // quartet, which sums the group's x^2. U items per thread have their
    // loads in flight together (clamped addresses); the tall path's 64-row
    // slices (512 threads) take all of theirs in one batch. (D is a multiple
    // of 32, so an 8-column piece is wholly inside or outside the matrix.)
    constexpr int C8 = VC / 8;
    constexpr int U = ROWS >= 64 ? 4 : 1;
    const int ng = p.D / 32;
    for (int e0 = threadIdx.x; e0 < ROWS * C8; e0 += U * blockDim.x) {
      float4 xo[U][2];
      u32x4 go[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * blockDim.x;
        const int ml = e / C8, c8 = e % C8;
        int m = m0 + ml, n = vc0 + 8 * c8;
        m = m < M ? m : M - 1;
        n = n < p.n_vcols ? n : p.n_vcols - 8;
        const float4* xr = reinterpret_cast<const float4*>(p.x + (size_t)m * p.D + n);
        xo[u][0] = xr[0];
        xo[u][1] = xr[1];
        go[u] = *reinterpret_cast<const u32x4*>(p.gain + n);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * blockDim.x;
        const int ml = e / C8, c8 = e % C8;
        const int m = m0 + ml;
        const int n = vc0 + 8 * c8;
        const bool live = e < ROWS * C8 && m < M && n < p.n_vcols;
        const float x8[8] = {xo[u][0].x, xo[u][0].y, xo[u][0].z, xo[u][0].w,
                             xo[u][1].x, xo[u][1].y, xo[u][1].z, xo[u][1].w};
        float xn[8], xg[8], sq = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xn[j] = x8[j] + tile[live ? ml : 0][8 * c8 + j];
          const uint32_t gw = go[u][j >> 1];
          xg[j] = xn[j] * __uint_as_float(j & 1 ? gw & 0xffff0000u : gw << 16);
          sq += xn[j] * xn[j];
        }
        sq = quad_sum(sq);  // the row's 32-column group (all four lanes take part)
        if (!live) continue;
        const size_t i = (size_t)m * p.D + n;
        float4* xw = reinterpret_cast<float4*>(p.x + i);
        xw[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
        xw[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
        if (p.hidden) {
          float4* hw = reinterpret_cast<float4*>(p.hidden + i);
          hw[0] = make_float4(xn[0], xn[1], xn[2], xn[3]);
          hw[1] = make_float4(xn[4], xn[5], xn[6], xn[7]);
        }
        bf16x8 hi, lo;
        pack_split_bf16x8(xg, hi, lo);
        *reinterpret_cast<bf16x8*>(p.xh + i) = hi;
        *reinterpret_cast<bf16x8*>(p.xl + i) = lo;
        if ((c8 & 3) == 0) p.ssq[(size_t)m * ng + n / 32] = sq;
      }
    }
  }
};

struct EpiSwiglu {
  struct P {
    const bf16_t *wg, *wu;  // [F][D]
    int K, F;
    bf16_t *ah, *al;        // [M][F] activation hi/lo
    int n_vcols;            // 2F
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    const int t = vc >> 4, j = vc & 15;
    const int f = (t << 3) + (j & 7);
    return (j < 8 ? p.wg : p.wu) + (size_t)f * p.K;
  }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return ((vc8 & 8) ? p.wu : p.wg) + (size_t)((vc8 >> 4) * 8 + r8) * p.K;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs,
                             int vc0, int m0, int M) {
    constexpr int NG = VC / 16;
    // one thread per (row, 16-column group): its 8 gate/up pairs are 8
    // consecutive activation columns, written as 16-byte stores (F is a
    // multiple of 8 on every path that gets here: checked on the host)
    for (int e = threadIdx.x; e < ROWS * NG; e += blockDim.x) {
      const int ml = e / NG, c = e % NG;
      const int m = m0 + ml;
      if (m >= M || vc0 + c * 16 >= p.n_vcols) continue;
      const float r = rs[ml];
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float g = tile[ml][c * 16 + j] * r;
        const float u = tile[ml][c * 16 + j + 8] * r;
        // silu(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal
        // (each within about an ulp); -g past the exponent range gives 1/inf = 0
        a[j] = g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f)) * u;
      }
      const size_t i = (size_t)m * p.F + ((vc0 >> 4) + c) * 8;
      bf16x8 hi, lo;
      pack_split_bf16x8(a, hi, lo);
      *reinterpret_cast<bf16x8*>(p.ah + i) = hi;
      *reinterpret_cast<bf16x8*>(p.al + i) = lo;
    }
  }
};

struct EpiLM {
  struct P {
    const bf16_t* w;   // [V][K]
    int K, V;
    float* logits;     // optional [M][V]
    uint64_t* part;    // [n_tiles][M] argmax keys
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    return p.w + (size_t)(vc < p.V ? vc : p.V - 1) * p.K;
  }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return wrow(p, vc8 + r8);
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs,
                             int vc0, int m0, int M) {
    // one pass: the row scale applied as the keys are formed (and the
    // optional logits written); eight threads per row, thread q taking
    // columns q, q + 8, ... (the eight rows and eight column offsets of a
    // wave's reads fall in distinct banks for any row pitch of 8 mod 64
    // words), then a max over the eight
    constexpr int TPR = 8;
    static_assert(ROWS * TPR % 64 == 0 && VC % TPR == 0, "whole waves per pass, whole column strides");
    for (int e0 = 0; e0 < ROWS * TPR; e0 += blockDim.x) {
      const int e = e0 + threadIdx.x;
      const int ml = e / TPR, q = e % TPR;
      const bool live = e < ROWS * TPR && m0 + ml < M;
      uint64_t best = 0;
      if (live) {
        // every read of the row's columns issued before the first key
        constexpr int NC = VC / TPR;
        const float sc = rs[ml];
        float z[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) z[i] = tile[ml][q + i * TPR] * sc;
        if (p.logits) {
          float* lrow = p.logits + (size_t)(m0 + ml) * p.V;
#pragma unroll
          for (int i = 0; i < NC; ++i)
            if (vc0 + q + i * TPR < p.V) lrow[vc0 + q + i * TPR] = z[i];
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int v = vc0 + q + i * TPR;
          if (v < p.V) best = umax64(best, argmax_key(z[i], (uint32_t)v));
        }
      }
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        const uint64_t other = __shfl_xor(best, o, kWave);
        best = umax64(best, other);
      }
      if (live && q == 0) p.part[(size_t)(vc0 / VC) * M + m0 + ml] = best;
    }
  }
};

// Plain fp32 store of the product (the draft's sublayer outputs when a conv
// follows them: the residual add happens after the conv's finish call).
struct EpiStore {
  struct P {
    const bf16_t* w;   // [N][K]
    int K, N;
    float* out;        // [M][N]
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) { return p.w + (size_t)vc * p.K; }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return p.w + (size_t)(vc8 + r8) * p.K;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs, int vc0, int m0,
                             int M) {
    for (int e = threadIdx.x; e < ROWS * VC; e += blockDim.x) {
      const int ml = e / VC, c = e % VC;
      const int m = m0 + ml, n = vc0 + c;
      if (m < M && n < p.N) p.out[(size_t)m * p.N + n] = tile[ml][c] * rs[ml];
    }
  }
};

// Context fusion for a few rows (the accepted rows appended each round):
// y = [h_1 .. h_n] W_c^T in fp32 plus per-32-column sums of y^2; the RMSNorm
// pass runs afterwards and rounds to bf16 once.
struct EpiFuseRows {
  struct P {
    const bf16_t* w;  // W_c [D][K]
    int K, D;
    float* y;         // [M][D] (or, with yh: not written)
    float* ssq;       // [M][D/32]
    int n_vcols;      // D
    bf16_t *yh = nullptr, *yl = nullptr;  // optional: hi/lo of y * gain instead of y
    const bf16_t* gain = nullptr;
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) { return p.w + (size_t)vc * p.K; }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return p.w + (size_t)(vc8 + r8) * p.K;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float*, int vc0, int m0,
                             int M) {
    static_assert(VC % 32 == 0, "whole 32-column norm groups per workgroup");
    for (int e = threadIdx.x; e < ROWS * VC; e += blockDim.x) {
      const int ml = e / VC, c = e % VC;
      const int m = m0 + ml;
      if (m >= M || vc0 + c >= p.n_vcols) continue;
      const float y = tile[ml][c];
      const size_t i = (size_t)m * p.D + vc0 + c;
      if (p.yh)
        split_bf16(y * bf2f(p.gain[vc0 + c]), p.yh[i], p.yl[i]);
      else
        p.y[i] = y;
      tile[ml][c] = y * y;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ROWS * (VC / 32); e += blockDim.x) {
      const int ml = e / (VC / 32), g = e % (VC / 32);
      if (m0 + ml >= M || vc0 + g * 32 >= p.n_vcols) continue;
      float s = 0.f;
      for (int c = 0; c < 32; ++c) s += tile[ml][g * 32 + c];
      p.ssq[(size_t)(m0 + ml) * (p.D / 32) + vc0 / 32 + g] = s;
    }
  }
};

// KV injection for a few rows: virtual columns run over every layer's K and
// V; within K heads the RoPE pairs share a 16-column group as in EpiQKV.
struct EpiInjectRows {
  struct P {
    const bf16_t* wk[kMaxLayers];
    const bf16_t* wv[kMaxLayers];
    int D, Hkv, hd, pos0, cap;
    double log2_theta;
    bf16_t* kv;
    int n_vcols;     // L * 2 * Hkv * hd
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    const int kvd = p.Hkv * p.hd;
    const int i = vc / (2 * kvd), r = vc % (2 * kvd);
    if (r < kvd) {
      const int h = r / p.hd, d = paired_dim(r % p.hd, p.hd);
      return p.wk[i] + (size_t)(h * p.hd + d) * p.D;
    }
    return p.wv[i] + (size_t)(r - kvd) * p.D;
  }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    const int kvd = p.Hkv * p.hd;
    const int i = vc8 / (2 * kvd), r = vc8 % (2 * kvd);
    if (r < kvd) {
      const int h = r / p.hd, d = paired_dim(r % p.hd + r8, p.hd);
      return p.wk[i] + (size_t)(h * p.hd + d) * p.D;
    }
    return p.wv[i] + (size_t)(r - kvd + r8) * p.D;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float*, int vc0, int m0,
                             int M) {
    const int kvd = p.Hkv * p.hd;
    const size_t plane = (size_t)p.cap * p.hd;
    constexpr int NG = VC / 16;
    // the rotation frequencies (revolutions per position) once per call
    __shared__ double inv_f[kMaxHeadDim / 2];
    for (int d = threadIdx.x; d < p.hd / 2; d += blockDim.x) inv_f[d] = rope_rev_freq(d, p.hd, p.log2_theta);
    __syncthreads();
    for (int e = threadIdx.x; e < ROWS * NG * 8; e += blockDim.x) {
      const int ml = e / (NG * 8), c = (e / 8) % NG, j = e % 8;
      const int m = m0 + ml;
      if (m >= M) continue;
      const int pos = p.pos0 + m;
      const int vc = vc0 + c * 16;
      if (vc >= p.n_vcols) continue;
      const int i = vc / (2 * kvd), r = vc % (2 * kvd);
      const float x1 = tile[ml][c * 16 + j], x2 = tile[ml][c * 16 + j + 8];
      if (r < kvd) {
        const int h = r / p.hd, d = ((r % p.hd) >> 1) + j;
        float cs, sn;
        rope_cs_rev(pos, inv_f[d], cs, sn);
        bf16_t* k = p.kv + (size_t)((2 * i) * p.Hkv + h) * plane + (size_t)pos * p.hd;
        k[d] = f2bf(x1 * cs - x2 * sn);
        k[d + p.hd / 2] = f2bf(x2 * cs + x1 * sn);
      } else {
        const int h = (r - kvd) / p.hd, d0 = (r - kvd) % p.hd + j;
        bf16_t* v = p.kv + (size_t)((2 * i + 1) * p.Hkv + h) * plane;
        v[(size_t)d0 * p.cap + pos] = f2bf(x1);
        v[(size_t)(d0 + 8) * p.cap + pos] = f2bf(x2);
      }
    }
  }
};

// KV injection of the accepted rows of several sequences at their device
// lengths (device-resident rounds): output row m is row r = m % rps of
// sequence s = m / rps; it is written at position len[s] + r when
// r < tau[s] and that position lies inside the buffer, and dropped
// otherwise. Column order and RoPE pairing as in EpiInjectRows.
struct EpiAppendRows {
  struct P {
    const bf16_t* wk[kMaxLayers];
    const bf16_t* wv[kMaxLayers];
    int D, Hkv, hd, rps;
    double log2_theta;
    const int32_t* tau;   // [n_seqs] device
    SeqTable seqs;        // with len_dev
    int n_vcols;          // L * 2 * Hkv * hd
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    const int kvd = p.Hkv * p.hd;
    const int i = vc / (2 * kvd), r = vc % (2 * kvd);
    if (r < kvd) {
      const int h = r / p.hd, d = paired_dim(r % p.hd, p.hd);
      return p.wk[i] + (size_t)(h * p.hd + d) * p.D;
    }
    return p.wv[i] + (size_t)(r - kvd) * p.D;
  }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    const int kvd = p.Hkv * p.hd;
    const int i = vc8 / (2 * kvd), r = vc8 % (2 * kvd);
    if (r < kvd) {
      const int h = r / p.hd, d = paired_dim(r % p.hd + r8, p.hd);
      return p.wk[i] + (size_t)(h * p.hd + d) * p.D;
    }
    return p.wv[i] + (size_t)(r - kvd + r8) * p.D;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs, int vc0, int m0,
                             int M) {
    const int kvd = p.Hkv * p.hd;
    constexpr int NG = VC / 16;
    // each row's position (-1: not appended) and cache once, through LDS
    __shared__ int r_pos[ROWS], r_cap[ROWS];
    __shared__ bf16_t* r_kv[ROWS];
    // and the rotation frequencies (revolutions per position)
    __shared__ double inv_f[kMaxHeadDim / 2];
    for (int d = threadIdx.x; d < p.hd / 2; d += blockDim.x) inv_f[d] = rope_rev_freq(d, p.hd, p.log2_theta);
    for (int ml = threadIdx.x; ml < ROWS; ml += blockDim.x) {
      const int m = m0 + ml;
      int pos = -1;
      if (m < M) {
        const int s = m / p.rps, rr = m % p.rps;
        const int at = seq_len(p.seqs, s) + rr;
        if (rr < p.tau[s] && at < p.seqs.s[s].max_ctx) pos = at;
        r_cap[ml] = p.seqs.s[s].cap;
        r_kv[ml] = p.seqs.s[s].kv;
      }
      r_pos[ml] = pos;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ROWS * NG * 8; e += blockDim.x) {
      const int ml = e / (NG * 8), c = (e / 8) % NG, j = e % 8;
      const int m = m0 + ml;
      if (m >= M) continue;
      const int pos = r_pos[ml];
      if (pos < 0) continue;
      SeqDesc sd;
      sd.cap = r_cap[ml];
      sd.kv = r_kv[ml];
      const int vc = vc0 + c * 16;
      if (vc >= p.n_vcols) continue;
      const size_t plane = (size_t)sd.cap * p.hd;
      const int i = vc / (2 * kvd), r = vc % (2 * kvd);
      const float x1 = tile[ml][c * 16 + j] * rs[ml], x2 = tile[ml][c * 16 + j + 8] * rs[ml];
      if (r < kvd) {
        const int h = r / p.hd, d = ((r % p.hd) >> 1) + j;
        float cs, sn;
        rope_cs_rev(pos, inv_f[d], cs, sn);
        bf16_t* k = sd.kv + (size_t)((2 * i) * p.Hkv + h) * plane + (size_t)pos * p.hd;
        k[d] = f2bf(x1 * cs - x2 * sn);
        k[d + p.hd / 2] = f2bf(x2 * cs + x1 * sn);
      } else {
        const int h = (r - kvd) / p.hd, d0 = (r - kvd) % p.hd + j;
        bf16_t* v = sd.kv + (size_t)((2 * i + 1) * p.Hkv + h) * plane;
        v[(size_t)d0 * sd.cap + pos] = f2bf(x1);
        v[(size_t)(d0 + 8) * sd.cap + pos] = f2bf(x2);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// the streaming GEMM
// ---------------------------------------------------------------------------

// DFlash 2 grouped dynamic two-tap conv ([Code] sections 13-14): the
// projection of the hidden state to 2 x 2 x G corrections (call, tap, group;
// call 0 "prepare", call 1 "finish") runs as a streaming GEMM over the rows.
// Its virtual columns put both taps of 16 groups of one call in each
// 32-column pair: column 32p + j is tap j / 16 of group 16p + j % 16. A
// call-0 pair's epilogue applies the prepare conv to its 16 * gs channels,
//   y_t = (b0 + c_{t,0}) * x_t + (b1 + c_{t,1}) * x_{t-1},
// where a block's first row reads prev; a call-1 pair stores its
// corrections for the finish call.
struct EpiConv {
  struct P {
    const bf16_t* proj;  // [4G][D]
    const bf16_t* base;  // [2][2][D] (call, tap, channel)
    const float* x;      // [M][D] the conv input (also the GEMM's A, as hi/lo)
    const float* prev;   // [n_seqs][D]; null: a zero row
    float* y;            // [M][D]
    float* corr;         // [M][2G] finish corrections (tap, group)
    int D, G, gs, Bl;
    int n_vcols;         // 4G
    int parts;           // workgroups sharing a pair's channels (grid.y of the finisher), else 1
    // inside a draft layer (EpiConvNorm): x is the residual stream and the
    // conv input the normed row x * gain * rs (rs the GEMM's row scale, which
    // also scales the corrections); the output goes to yh / yl as the
    // sublayer GEMM's bf16 hi/lo input instead of y. All rows in one tile.
    const bf16_t* gain;  // null: x is the conv input itself
    bf16_t *yh, *yl;
  };
  __device__ static int prow(const P& p, int v) {
    const int call = v / (2 * p.G), w = v - call * 2 * p.G;
    return (call * 2 + ((w & 31) >> 4)) * p.G + (w >> 5) * 16 + (w & 15);
  }
  __device__ static const bf16_t* wrow(const P& p, int vc) {
    return p.proj + (size_t)prow(p, vc) * p.D;
  }
  // an 8-aligned group of virtual columns maps to 8 consecutive projection rows
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return p.proj + (size_t)(prow(p, vc8) + r8) * p.D;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs, int vc0, int m0,
                             int M) {
    static_assert(VC % 32 == 0, "whole column pairs per workgroup");
    for (int pl = 0; pl < VC / 32; ++pl) {
      const int v0 = vc0 + pl * 32;
      if (v0 >= p.n_vcols) break;
      const int call = v0 / (2 * p.G);
      const int g0 = ((v0 - call * 2 * p.G) >> 5) * 16;
      const int part = p.parts > 1 ? (int)blockIdx.y : 0;
      if (call == 1) {
        if (part) continue;
        for (int e = threadIdx.x; e < ROWS * 32; e += blockDim.x) {
          const int ml = e >> 5, j = e & 31, m = m0 + ml;
          if (m < M)
            p.corr[(size_t)m * 2 * p.G + (j >> 4) * p.G + g0 + (j & 15)] = tile[ml][pl * 32 + j] * rs[ml];
        }
        continue;
      }
      // eight elements per thread at a time: their loads (clamped
      // addresses) go out together before any use
      constexpr int U = 8;
      // this workgroup's share of the pair's 16 * gs channels
      const int nch = 16 * p.gs / p.parts, c0 = g0 * p.gs + part * nch;
      for (int e0 = threadIdx.x; e0 < ROWS * nch; e0 += U * blockDim.x) {
        float xv[U], xb[U];
        bf16_t b0[U], b1[U], gn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + u * blockDim.x;
          int ml = e / nch;
          const int c = c0 + (e - ml * nch);
          int m = m0 + ml;
          m = m < M ? m : M - 1;
          const int t = m % p.Bl;
          xv[u] = p.x[(size_t)m * p.D + c];
          xb[u] = t == 0 ? (p.prev ? p.prev[(size_t)(m / p.Bl) * p.D + c] : 0.f)
                         : p.x[(size_t)(m - 1) * p.D + c];
          b0[u] = p.base[c];
          b1[u] = p.base[p.D + c];
          gn[u] = p.gain ? p.gain[c] : (bf16_t)0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + u * blockDim.x;
          const int ml = e / nch, cl = e - ml * nch, m = m0 + ml;
          if (e >= ROWS * nch || m >= M) continue;
          const int gl = (c0 - g0 * p.gs + cl) / p.gs;
          const float k0 = bf2f(b0[u]) + tile[ml][pl * 32 + gl] * rs[ml];
          const float k1 = bf2f(b1[u]) + tile[ml][pl * 32 + 16 + gl] * rs[ml];
          const size_t i = (size_t)m * p.D + c0 + cl;
          if (p.gain) {  // normed rows: the previous row's scale is rs[ml - 1] (one tile)
            const float g = bf2f(gn[u]);
            const float ht = xv[u] * g * rs[ml];
            const float hp = m % p.Bl ? xb[u] * g * rs[ml - 1] : 0.f;
            split_bf16(k0 * ht + k1 * hp, p.yh[i], p.yl[i]);
          } else {
            p.y[i] = k0 * xv[u] + k1 * xb[u];
          }
        }
      }
    }
  }
};

// The prepare call inside a draft layer: EpiConv in its fused mode, with the
// GEMM's A operand staged as usual (the residual's next-norm input x * gain as
// a bf16 hi/lo pair and its row scale) instead of fp32 conv input rows.
struct EpiConvNorm : EpiConv {};

// The finish call of a layer's conv fused with the residual add (the
// sublayer's output product, one tile holding every row): per row m
// (position t of its block) and column c of the tile, z = the product,
//   y = (base[1][0][c] + corr[m][0][g]) z_t + (base[1][1][c] + corr[m][1][g]) z_{t-1},
// z_{-1} = 0, g = c / gs; then x += y, the optional hidden copy, the next
// RMSNorm's input x * gain as a bf16 hi/lo pair and per-32-column sums of
// x^2, as EpiResid leaves them.
struct EpiConvResid {
  struct P {
    const bf16_t* w;     // [N=D][K]
    int K, D;
    const bf16_t* base;  // [2][2][D]
    const float* corr;   // [M][2G]
    int G, gs, Bl;
    float* x;            // [M][D]
    bf16_t *xh, *xl;     // [M][D]
    const bf16_t* gain;  // [D] the next norm's gain
    float* ssq;          // [M][D/32]
    float* hidden;       // optional [M][D]
    int n_vcols;         // D
  };
  __device__ static const bf16_t* wrow(const P& p, int vc) { return p.w + (size_t)vc * p.K; }
  __device__ static const bf16_t* wrow8(const P& p, int vc8, int r8) {
    return p.w + (size_t)(vc8 + r8) * p.K;
  }
  template <int ROWS, int VC, int LD = VC + 1>
  __device__ static void run(const P& p, float (*tile)[LD], const float* rs, int vc0, int m0,
                             int M) {
    static_assert(VC % 32 == 0, "whole 32-column norm groups per workgroup");
    __shared__ float sq[ROWS][VC + 1];
    for (int e = threadIdx.x; e < ROWS * VC; e += blockDim.x) {
      const int ml = e / VC, c = e % VC;
      const int m = m0 + ml, n = vc0 + c;
      float v = 0.f;
      if (m < M && n < p.n_vcols) {
        const int t = m % p.Bl, g = n / p.gs;
        const float zt = tile[ml][c] * rs[ml];
        const float zp = t ? tile[ml - 1][c] * rs[ml - 1] : 0.f;
        const float k0 = bf2f(p.base[2 * p.D + n]) + p.corr[(size_t)m * 2 * p.G + g];
        const float k1 = bf2f(p.base[3 * p.D + n]) + p.corr[(size_t)m * 2 * p.G + p.G + g];
        const size_t i = (size_t)m * p.D + n;
        const float xn = p.x[i] + k0 * zt + k1 * zp;
        p.x[i] = xn;
        if (p.hidden) p.hidden[i] = xn;
        split_bf16(xn * bf2f(p.gain[n]), p.xh[i], p.xl[i]);
        v = xn * xn;
      }
      sq[ml][c] = v;
    }
    __syncthreads();
    const int ng = p.D / 32;
    for (int e = threadIdx.x; e < ROWS * (VC / 32); e += blockDim.x) {
      const int ml = e / (VC / 32), g = e % (VC / 32);
      if (m0 + ml >= M || vc0 + g * 32 >= p.n_vcols) continue;
      float sum = 0.f;
#pragma unroll 8
      for (int c = 0; c < 32; ++c) sum += sq[ml][g * 32 + c];
      p.ssq[(size_t)(m0 + ml) * ng + vc0 / 32 + g] = sum;
    }
  }
};

struct SplitK {
  int ksplit;        // workgroups sharing one column block's K range
  int steps;         // 32-wide k steps per split
  float* part;       // [col block][split][ROWS][VC] fp32 partial tiles
};

// RMSNorm row scale of the tile rows from the producer's per-32-column sums
// of x^2 (one wave per row); 1 when the GEMM has no input norm.
template <int ROWS>
__device__ __forceinline__ void row_scales(const SkinnyA& a, int m0, float* rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int row = w; row < ROWS; row += nw) {
    float s = 0.f;
    if (a.ssq && m0 + row < a.M) {
      const float* q = a.ssq + (size_t)in_row(a, m0 + row) * a.ssq_ld;
      s = strided_sum(q, a.ssq_ld, lane, 64);
      s = wave_sum(s);
    }
    if (lane == 0) rs[row] = a.ssq ? rsqrtf(s / (float)a.K + a.eps) : 1.f;
  }
}

template <int MT, int NCT, int NW, int U, bool LO, class Epi>
__global__ void __launch_bounds__(NW * 64)
skinny_gemm(SkinnyA a, typename Epi::P ep, int n_vcols, SplitK sk) {
  constexpr int VC = 16 * NCT;
  constexpr int ROWS = 16 * MT;
  __shared__ float red[NW][MT * NCT * 4][64];
  __shared__ float tile[ROWS][VC + 1];
  __shared__ float rs[ROWS];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cb = blockIdx.x / sk.ksplit, ksi = blockIdx.x % sk.ksplit;
  const int vc0 = cb * VC;
  const int m0 = blockIdx.y * ROWS;
  const int kq = 8 * (lane >> 4);

  const bf16_t* wr[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    int vc = vc0 + c * 16 + (lane & 15);
    vc = vc < n_vcols ? vc : n_vcols - 1;
    wr[c] = Epi::wrow(ep, vc) + kq;
  }
  size_t aoff[MT];
  bool av[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = m0 + m * 16 + (lane & 15);
    av[m] = row < a.M;
    aoff[m] = av[m] ? (size_t)in_row(a, row) * a.lda + kq : 0;
  }

  f32x4 acc[MT][NCT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KS = a.K >> 5;
  const int kbeg = ksi * sk.steps;
  const int kend = min(kbeg + sk.steps, KS);
  for (int ks0 = kbeg + w; ks0 < kend; ks0 += NW * U) {
    bf16x8 bq[U][NCT], xh[U][MT], xl[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * NW;
      if (ks < kend) {
        const int k = ks * 32;
        const int sg = k / a.seg_k;
        const bf16_t* hb = a.seg[sg] + (k - sg * a.seg_k);
#pragma unroll
        for (int c = 0; c < NCT; ++c) bq[u][c] = ld_bf16x8(wr[c] + k);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          xh[u][m] = av[m] ? ld_bf16x8(hb + aoff[m]) : zero_bf16x8();
          if (LO) xl[u][m] = av[m] ? ld_bf16x8(a.xl + aoff[m] + k) : zero_bf16x8();
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + u * NW < kend) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            acc[m][c] = mfma16x16x32(xh[u][m], bq[u][c], acc[m][c]);
            if (LO) acc[m][c] = mfma16x16x32(xl[u][m], bq[u][c], acc[m][c]);
          }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w][(m * NCT + c) * 4 + e][lane] = acc[m][c][e];
  __syncthreads();

  for (int e = threadIdx.x; e < MT * NCT * 256; e += NW * 64) {
    const int l = e & 63, q4 = (e >> 6) & 3, c = (e >> 8) % NCT, m = e / (256 * NCT);
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += red[ww][(m * NCT + c) * 4 + q4][l];
    tile[m * 16 + (l >> 4) * 4 + q4][c * 16 + (l & 15)] = s;
  }
  __syncthreads();

  if (sk.ksplit > 1) {  // publish this split's partial tile for the finisher
    float* mine = sk.part + ((size_t)cb * sk.ksplit + ksi) * ROWS * VC;
    for (int e = threadIdx.x; e < ROWS * VC; e += NW * 64) mine[e] = tile[e / VC][e % VC];
    return;
  }
  row_scales<ROWS>(a, m0, rs);
  __syncthreads();
  Epi::template run<ROWS, VC>(ep, tile, rs, vc0, m0, a.M);
}

// Sum of a column block's split partials, in split order, then the epilogue.
constexpr int kFinishBatch = 8;
template <int MT, int NCT, class Epi>
__global__ void __launch_bounds__(256)
skinny_finish(SkinnyA a, typename Epi::P ep, SplitK sk) {
  constexpr int VC = 16 * NCT;
  constexpr int ROWS = 16 * MT;
  __shared__ float tile[ROWS][VC + 1];
  __shared__ float rs[ROWS];
  const int cb = blockIdx.x;
  const float* __restrict__ all = sk.part + (size_t)cb * sk.ksplit * ROWS * VC;
  // every partial of this thread's elements is loaded before any is summed:
  // one memory round trip instead of one per split
  constexpr int EPT = ROWS * VC / 256;
  static_assert(ROWS * VC % 256 == 0, "whole elements per thread");
  for (int k0 = 0; k0 < sk.ksplit; k0 += kFinishBatch) {
    float v[kFinishBatch][EPT];
#pragma unroll
    for (int k = 0; k < kFinishBatch; ++k)
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        v[k][j] = k0 + k < sk.ksplit ? all[(size_t)(k0 + k) * ROWS * VC + threadIdx.x + 256 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = threadIdx.x + 256 * j;
      float acc = k0 ? tile[e / VC][e % VC] : 0.f;
#pragma unroll
      for (int k = 0; k < kFinishBatch; ++k) acc += v[k][j];  // split order
      tile[e / VC][e % VC] = acc;
    }
  }
  row_scales<ROWS>(a, 0, rs);
  __syncthreads();
  Epi::template run<ROWS, VC>(ep, tile, rs, cb * VC, 0, a.M);
}

// ---------------------------------------------------------------------------
// LDS-staged streaming GEMM for up to 16 activation rows
// ---------------------------------------------------------------------------
// The weights arrive by direct global->LDS loads into a ring of R slots per
// wave. A slot holds 16 weight rows x 256 k (8 KB); each load instruction
// fetches 512 contiguous bytes of two rows, so DRAM sees long row bursts
// (fewer, longer bursts measured faster than 128-byte pieces, and those
// faster than the MFMA operand layout loaded straight into registers). The
// rows are read back as MFMA B fragments through an XOR swizzle (16-byte
// chunk c of row r stored at chunk c ^ r) that keeps the lane reads free of
// bank conflicts. The workgroup's K slice of the activations sits in LDS in
// fragment order. Each wave owns whole units - one 16-column tile over the
// slice - so the loop has no barrier: a barrier would wait for every direct
// load in flight. Units go round-robin over the waves of the workgroups that
// share a slice; the grid is one workgroup per CU. Each unit leaves an fp32
// partial tile; the finisher sums the slices in order and runs the epilogue.

constexpr int kSW = 4;             // waves per workgroup
constexpr int kCUs = 256;          // the grid: at most one workgroup per CU
constexpr int kItemK = 256;        // k per ring slot
constexpr int kItem = 16 * kItemK * 2;  // ring slot bytes
constexpr int kItemLoads = kItem / 1024;  // direct-load instructions per slot
constexpr int kSliceMax = 1024;    // k per workgroup slice (LDS activation buffer)
#ifndef DFL_STREAM_RING
#define DFL_STREAM_RING 3
#endif
#ifndef DFL_STREAM_BATCH
#define DFL_STREAM_BATCH 4
#endif
constexpr int kStreamRing = DFL_STREAM_RING;    // ring slots per wave
constexpr int kStreamBatch = DFL_STREAM_BATCH;  // units per batch of partial stores

// s_waitcnt immediate for vmcnt <= n (0..63), expcnt and lgkmcnt left open
#define DFL_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | 0xF70)
#define DFL_LGKM0 0xC07F

// The eight 16-byte B-fragment reads of one ring slot (k steps 0..7 of row
// r = lane % 16: chunk 4s + lane / 16, stored at that chunk ^ r), complete on
// return. Inline assembly, so that the compiler's wait-count pass does not
// treat them as possibly aliasing the direct loads still in flight into the
// other ring slots (it would drain every outstanding load before each read);
// explicit vmcnt waits order the ring instead. Activation reads the compiler
// issued before this block are complete on return as well.
__device__ __forceinline__ void ring_read8(u32x4 (&b)[8], const uint8_t* row, int c0, int r) {
  const uint32_t base = (uint32_t)(uintptr_t)row;
  uint32_t ad[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) ad[s] = base + ((((4 * s) + c0) ^ r) << 4);
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]),
        "=&v"(b[6]), "=&v"(b[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7])
      : "memory");
}


// wait until at most n direct loads (whole slots) are in flight
__device__ __forceinline__ void wait_vm_slots(int slots_after) {
  switch (slots_after) {
    case 0: __builtin_amdgcn_s_waitcnt(DFL_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(DFL_VMCNT(kItemLoads)); break;
    case 2: __builtin_amdgcn_s_waitcnt(DFL_VMCNT(2 * kItemLoads)); break;
    default: __builtin_amdgcn_s_waitcnt(DFL_VMCNT(3 * kItemLoads)); break;
  }
}

// R ring slots per wave; KSL the largest K slice the activation buffer holds
// (the slices of the short products leave room for a deeper ring)
template <int R, int UB, bool LO, class Epi, int KSL = kSliceMax>
__global__ void __launch_bounds__(kSW * 64)
stream_gemm(SkinnyA a, typename Epi::P ep, int n_vcols, int ks, int kc, float* __restrict__ part) {
  static_assert(R >= 2 && R - 1 <= 3, "slots in flight handled by wait_vm_slots");
  static_assert(kItemK == 256, "ring_read8 covers 8 k steps per slot");
  static_assert(KSL * 64 + kSW * R * kItem <= 160 * 1024, "activation slice and ring fit in LDS");
  __shared__ __attribute__((aligned(16))) u32x4 As[KSL / 32][2][64];  // [k step][hi, lo][lane]
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSW][R][kItem];
  const int lane = threadIdx.x & 63;
  // wave-uniform in a scalar register: the matrix and segment choices below
  // then compile to scalar selects, never to per-lane loads of kernel
  // arguments (a vector load in the loop would wait for every direct load)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = blockIdx.x % ks;
  const int k0 = slice * kc;
  const int nsteps = kc >> 5;

  const int gw = (blockIdx.x / ks) * kSW + w;  // wave within the slice's group
  const int Wg = (gridDim.x / ks) * kSW;
  const int n_tiles = (n_vcols + 15) >> 4;
  const int units = gw < n_tiles ? (n_tiles - gw + Wg - 1) / Wg : 0;
  const int ipu = kc / kItemK;                  // ring slots per unit
  const int n_items = units * ipu;
  uint8_t* my_ring = &ring[w][0][0];

  // direct loads of slot t: instruction q covers rows 2q and 2q + 1 (lanes
  // 0-31 and 32-63), 512 bytes each; chunk position p of row r receives the
  // row's chunk p ^ r
  auto issue = [&](int t) {
    const int j = t / ipu, i = t - j * ipu;
    const int tile = gw + j * Wg;
    const int kk = k0 + i * kItemK;
    uint8_t* slot = my_ring + (t % R) * kItem;
    const int hi = lane >> 5, pos = lane & 31;
#pragma unroll
    for (int q = 0; q < kItemLoads; ++q) {
      const int r = 2 * q + hi;
      int vc8 = tile * 16 + ((2 * q) & ~7);              // uniform 8-row group
      vc8 = vc8 < n_vcols ? vc8 : ((n_vcols - 1) >> 3) << 3;
      int r8 = ((2 * q) & 7) + hi;
      r8 = vc8 + r8 < n_vcols ? r8 : n_vcols - 1 - vc8;  // ragged last group
      dma16_nt(Epi::wrow8(ep, vc8, r8) + kk + ((pos ^ r) << 3), slot + q * 1024);
    }
  };
  // the weight stream starts before the activations are in place
  const int pre = n_items < R - 1 ? n_items : R - 1;
  for (int t = 0; t < pre; ++t) issue(t);

  // the slice of the activations, in MFMA A-fragment order: wave w fills
  // fragments w, w + kSW, ... (each one k step, hi or lo); every load is
  // issued before the first store
  {
    constexpr int PER = KSL / 32 * 2 / kSW;
    u32x4 v[PER];
    const int m = lane & 15;
    const bool mv = m < a.M;
    const size_t row = (size_t)in_row(a, mv ? m : 0) * a.lda;
    // unconditional loads from clamped addresses, zeroed at the store, so
    // that all of them are in flight together; the dynamic conv reads its
    // fp32 rows and splits them into bf16 high and low halves here
    constexpr bool kF32A = std::is_same<Epi, EpiConv>::value;
    float4 fv[kF32A ? PER : 1][2];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int fr = w + u * kSW, hl = fr & 1;
      const int st = min(fr >> 1, nsteps - 1);
      const int kst = k0 + st * 32;
      const int k = kst + 8 * (lane >> 4);
      if constexpr (kF32A) {
        const float4* src = reinterpret_cast<const float4*>(ep.x + row + k);
        fv[u][0] = src[0];
        fv[u][1] = src[1];
      } else if (LO && hl) {
        v[u] = *reinterpret_cast<const u32x4*>(a.xl + row + k);
      } else {
        const int sg = kst / a.seg_k;
        v[u] = *reinterpret_cast<const u32x4*>(a.seg[sg] + row + (k - sg * a.seg_k));
      }
    }
    // steps past the slice land in unused slots (fr / 2 < KSL / 32)
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int fr = w + u * kSW, hl = fr & 1;
      const bool keep = mv && (hl == 0 || LO);
      if constexpr (kF32A) {
        const float f[8] = {fv[u][0].x, fv[u][0].y, fv[u][0].z, fv[u][0].w,
                            fv[u][1].x, fv[u][1].y, fv[u][1].z, fv[u][1].w};
        bf16x8 h, l;
        pack_split_bf16x8(f, h, l);
        v[u] = __builtin_bit_cast(u32x4, hl ? l : h);
      }
      As[fr >> 1][hl][lane] = keep ? v[u] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  const int br = lane & 15;
  const int c0 = lane >> 4;
  auto step = [&](int t, int i, f32x4& acc) {
    // the slot refilled below was read in the previous step
    __builtin_amdgcn_s_waitcnt(DFL_LGKM0);
    if (t + R - 1 < n_items) {
      issue(t + R - 1);
      __builtin_amdgcn_s_waitcnt(DFL_VMCNT((R - 1) * kItemLoads));
    } else {
      wait_vm_slots(n_items - 1 - t);
    }
    const uint8_t* row = my_ring + (t % R) * kItem + br * (kItemK * 2);
    // activation fragments of the slot's 8 k steps, then its weight
    // fragments: one LDS round trip for all of them
    u32x4 ah[8], al[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      ah[s8] = As[i * 8 + s8][0][lane];
      if (LO) al[s8] = As[i * 8 + s8][1][lane];
    }
    u32x4 b[8];
    ring_read8(b, row, c0, br);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      const bf16x8 bb = __builtin_bit_cast(bf16x8, b[s8]);
      acc = mfma16x16x32(__builtin_bit_cast(bf16x8, ah[s8]), bb, acc);
      if (LO) acc = mfma16x16x32(__builtin_bit_cast(bf16x8, al[s8]), bb, acc);
    }
  };
  // units in batches of UB whose partial tiles are stored together, each as
  // one contiguous kilobyte in MFMA lane order (layout [tile][split][lane][4]:
  // lane l, item e holds row 4 (l / 16) + e, column l % 16), written through
  // the L2 (the finisher, a separate launch, reads them): a store makes the
  // following ring waits wait for it as well, so fewer, larger batches keep
  // the stream flowing
  for (int jb = 0; jb < units; jb += UB) {
    f32x4 acc[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jb + u < units)
        for (int i = 0; i < ipu; ++i) step((jb + u) * ipu + i, i, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (jb + u < units) {
        const int tile = gw + (jb + u) * Wg;
        store16_wt(part, (uint32_t)(((tile * ks + slice) * 256 + lane * 4) * 4), acc[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// embedding of the block and the drafted-token reduction
// ---------------------------------------------------------------------------

// One workgroup per (row, 1024 columns); every thread owns 4 adjacent columns
// and makes a single round trip. 8 threads cover one 32-column norm group.
__global__ void __launch_bounds__(256)
embed_block(const bf16_t* __restrict__ E, int V, int D, const int32_t* __restrict__ anchors,
            int mask_id, int Bl, const bf16_t* __restrict__ gain, float* __restrict__ x,
            bf16_t* __restrict__ xh, bf16_t* __restrict__ xl, float* __restrict__ ssq,
            int32_t* __restrict__ block_out) {
  const int m = blockIdx.y, s = m / Bl, r = m % Bl;
  int id = r == 0 ? anchors[s] : mask_id;
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);  // keep the gather in bounds
  if (r == 0 && blockIdx.x == 0 && threadIdx.x == 0) block_out[s * Bl] = id;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  float sq = 0.f;
  if (n < D) {
    const uint2 ev = *reinterpret_cast<const uint2*>(E + (size_t)id * D + n);
    const uint2 gv = *reinterpret_cast<const uint2*>(gain + n);
    const bf16_t e4[4] = {(bf16_t)(ev.x & 0xffff), (bf16_t)(ev.x >> 16), (bf16_t)(ev.y & 0xffff),
                          (bf16_t)(ev.y >> 16)};
    const bf16_t g4[4] = {(bf16_t)(gv.x & 0xffff), (bf16_t)(gv.x >> 16), (bf16_t)(gv.y & 0xffff),
                          (bf16_t)(gv.y >> 16)};
    float4 xv;
    bf16_t hi[4], lo[4];
    float* xp = reinterpret_cast<float*>(&xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xp[i] = bf2f(e4[i]);
      split_bf16(xp[i] * bf2f(g4[i]), hi[i], lo[i]);
      sq += xp[i] * xp[i];
    }
    const size_t o = (size_t)m * D + n;
    *reinterpret_cast<float4*>(x + o) = xv;
    *reinterpret_cast<uint2*>(xh + o) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *reinterpret_cast<uint2*>(xl + o) = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
  sq = row8_sum(sq);
  if (n < D && (threadIdx.x & 7) == 0) ssq[(size_t)m * (D / 32) + n / 32] = sq;
}

__global__ void __launch_bounds__(256)
lm_argmax_reduce(const uint64_t* __restrict__ part, int n_tiles, int M_lm, int Bl,
                 int32_t* __restrict__ block_out) {
  const int m = blockIdx.x;
  uint64_t best = 0;
#pragma unroll 8
  for (int t = threadIdx.x; t < n_tiles; t += 256) best = umax64(best, part[(size_t)t * M_lm + m]);
  best = wave_max_u64(best);
  __shared__ uint64_t wbest[4];
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    best = umax64(umax64(wbest[0], wbest[1]), umax64(wbest[2], wbest[3]));
    const int g = Bl - 1;
    block_out[(m / g) * Bl + 1 + (m % g)] = (int32_t)argmax_key_index(best);
  }
}

// Sum of a 32-column pair's slice partials of the LDS-staged kernel, in slice
// order, then the epilogue. The row norms' sums of squares are fetched
// together with the partials. FB: partials requested per batch (16 where
// the slices are that many: one round trip instead of two).
template <class Epi, int FB = kFinishBatch>
__global__ void __launch_bounds__(256)
stream_finish(SkinnyA a, typename Epi::P ep, int ks, const float* __restrict__ part) {
  __shared__ float tile[16][33];
  __shared__ float rs[16];
  // device-resident lengths: request them before the partials, so the
  // epilogue's reads of them hit this CU's cache instead of waiting on a
  // round trip of their own (the value is kept live to the end)
  int warm = 0;
  if constexpr (std::is_same<Epi, EpiQKV>::value)
    if (ep.seqs.len_dev && (int)threadIdx.x < a.M / ep.Bl) warm = ep.seqs.len_dev[threadIdx.x];
  // the residual epilogue reads x and the norm gain of the pair's columns:
  // request their cache lines now as well, two elements per thread (loaded
  // into registers that are only named at the very end, so that no
  // instruction waits for them before the epilogue)
  float warm_x[2] = {0.f, 0.f};
  uint32_t warm_g[2] = {0u, 0u};
  if constexpr (std::is_same<Epi, EpiResid>::value) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = threadIdx.x + 256 * k, ml = e / 32, n = blockIdx.x * 32 + e % 32;
      const int mc = ml < a.M ? ml : a.M - 1, nc = n < ep.n_vcols ? n : ep.n_vcols - 1;
      warm_x[k] = ep.x[(size_t)mc * ep.D + nc];
      warm_g[k] = ep.gain[nc];
    }
  }
  const int t = threadIdx.x, pair = blockIdx.x;
  // thread t: element t of both tiles of the pair ([lane][4] order)
  const int ln = t >> 2, e = t & 3;
  const int m = 4 * (ln >> 4) + e, n = ln & 15;
  // row scales: wave w sums rows 4w..4w+3 (16 lanes each)
  const int lane = t & 63, w = t >> 6;
  const int srow = 4 * w + (lane >> 4);
  const float* p0 = part + ((size_t)(2 * pair) * ks) * 256 + t;
  const float* p1 = p0 + (size_t)ks * 256;
  // the first batch of slice partials and the row sums of x^2 are requested
  // together (clamped addresses: no branch around any load)
  float f0[FB], f1[FB];
#pragma unroll
  for (int k = 0; k < FB; ++k) {
    const int kk = k < ks ? k : ks - 1;
    f0[k] = p0[(size_t)kk * 256];
    f1[k] = p1[(size_t)kk * 256];
  }
  float sq = 0.f;
  if (a.ssq && srow < a.M) {
    const float* q = a.ssq + (size_t)in_row(a, srow) * a.ssq_ld;
    sq = strided_sum(q, a.ssq_ld, lane & 15, 16);
  }
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < FB; ++k)
    if (k < ks) { s0 += f0[k]; s1 += f1[k]; }  // slice order
  for (int k0 = FB; k0 < ks; k0 += FB) {
    float v0[FB], v1[FB];
#pragma unroll
    for (int k = 0; k < FB; ++k) {
      v0[k] = k0 + k < ks ? p0[(size_t)(k0 + k) * 256] : 0.f;
      v1[k] = k0 + k < ks ? p1[(size_t)(k0 + k) * 256] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < FB; ++k) { s0 += v0[k]; s1 += v1[k]; }  // slice order
  }
  tile[m][n] = s0;
  tile[m][16 + n] = s1;
  sq = row16_sum(sq);
  if ((lane & 15) == 0 && srow < 16) rs[srow] = a.ssq ? rsqrtf(sq / (float)a.K + a.eps) : 1.f;
  __syncthreads();
  Epi::template run<16, 32>(ep, tile, rs, pair * 32, 0, a.M);
  asm volatile("" ::"v"(warm), "v"(warm_x[0]), "v"(warm_x[1]), "v"(warm_g[0]), "v"(warm_g[1]));
}

// LM-head finisher: 256 vocabulary columns per workgroup, one per thread.
// Sums the slice partials (16-byte loads of four rows each), applies the
// final RMSNorm row scale, optionally writes the logits, and reduces each
// row's argmax key over the workgroup's columns into part[block][row].
__global__ void __launch_bounds__(256)
lm_stream_finish(SkinnyA a, EpiLM::P ep, int ks, const float* __restrict__ part) {
  __shared__ float rs[16];
  __shared__ uint64_t keys[16][256 + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int col = blockIdx.x * 256 + t;
  const int tile = col >> 4, n = col & 15;
  // row scales: wave w sums rows 4w..4w+3 (16 lanes each)
  const int srow = 4 * w + (lane >> 4);
  const int tiles = (ep.V + 15) >> 4;
  const int tl = tile < tiles ? tile : tiles - 1;
  // element (row 4g + e, column n) of a tile sits at [lane 16g + n][e]
  const float* src = part + (size_t)tl * ks * 256 + n * 4;
  // the first four slices' partials and the row sums of x^2 are requested
  // together (clamped addresses: no branch around any load)
  f32x4 f[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      f[k][g] = *reinterpret_cast<const f32x4*>(src + (size_t)(k < ks ? k : ks - 1) * 256 + g * 64);
  float sq = 0.f;
  if (a.ssq && srow < a.M) {
    const float* q = a.ssq + (size_t)in_row(a, srow) * a.ssq_ld;
    sq = strided_sum(q, a.ssq_ld, lane & 15, 16);
  }
  f32x4 z[4] = {};
#pragma unroll
  for (int k = 0; k < 4; ++k)  // slice order
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (k < ks) z[g] += f[k][g];
  for (int k0 = 4; k0 < ks; k0 += 4) {
    f32x4 v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        v[k][g] = k0 + k < ks ? *reinterpret_cast<const f32x4*>(src + (size_t)(k0 + k) * 256 + g * 64)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)  // slice order
#pragma unroll
      for (int g = 0; g < 4; ++g) z[g] += v[k][g];
  }
  sq = row16_sum(sq);
  if ((lane & 15) == 0) rs[srow] = a.ssq ? rsqrtf(sq / (float)a.K + a.eps) : 1.f;
  __syncthreads();
  const bool valid = col < ep.V;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float zm = z[m >> 2][m & 3] * rs[m];
    if (ep.logits && valid && m < a.M) ep.logits[(size_t)m * ep.V + col] = zm;
    keys[m][t] = valid ? argmax_key(zm, (uint32_t)col) : 0;
  }
  __syncthreads();
  // thread t: row t / 16 over columns 16 (t % 16) .. +15, then the 16 lanes
  // of the row
  {
    const int m = t >> 4, j = t & 15;
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) best = umax64(best, keys[m][16 * j + c]);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) best = umax64(best, (uint64_t)__shfl_xor(best, o, kWave));
    if (j == 0 && m < a.M) ep.part[(size_t)blockIdx.x * a.M + m] = best;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {
constexpr int kNW = 8;

// Column tiles per wave and the K split: few rows take wide tiles (the
// activation fragments are reused across NCT weight tiles) and narrow
// matrices split K so that the grid holds ~512-1024 workgroups.
template <class Epi, bool LO, int MT, int NCT, int U>
hipError_t launch_cfg(const SkinnyA& a, const typename Epi::P& ep, int n_vcols, const SplitWs& ws,
                      hipStream_t st) {
  constexpr int VC = 16 * NCT, ROWS = 16 * MT;
  const int blocks = (n_vcols + VC - 1) / VC;
  const int row_blocks = (a.M + ROWS - 1) / ROWS;
  const int KS = a.K / 32;
  int ks = 1;
  if (row_blocks == 1 && ws.part)
    while (blocks * ks * 2 <= kSplitTargetWG && KS / (ks * 2) >= 2 * kNW &&
           (size_t)blocks * ks * 2 * ROWS * VC <= ws.part_floats)
      ks *= 2;
  SplitK sk;
  sk.ksplit = ks;
  sk.steps = (KS + ks - 1) / ks;
  sk.part = ws.part;
  hipLaunchKernelGGL((skinny_gemm<MT, NCT, kNW, U, LO, Epi>), dim3(blocks * ks, row_blocks),
                     dim3(kNW * 64), 0, st, a, ep, n_vcols, sk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  hipLaunchKernelGGL((skinny_finish<MT, NCT, Epi>), dim3(blocks), dim3(256), 0, st, a, ep, sk);
  return hipGetLastError();
}

// Split of K for the LDS-staged kernel: slices of whole ring slots and at
// most kSliceMax (the LDS activation buffer), chosen so the units (16-column
// tiles x slices) spread evenly over the waves of the grid, which holds
// ks * floor(kCUs / ks) workgroups.
int stream_grid(int ks) { return ks * (kCUs / ks); }

bool stream_plan(int M, int n_vcols, int K, int& ks_out) {
  if (M < 1 || M > 16 || K % kItemK) return false;
  const int tiles = (n_vcols + 15) / 16;
  int best = 0;
  double best_eff = 0.0;
  for (int ks = 1; ks <= kCUs; ++ks) {
    if (K % ks || (K / ks) % kItemK || K / ks > kSliceMax) continue;
    const double waves = (double)stream_grid(ks) * kSW;
    const double units = (double)tiles * ks;
    const double per = std::ceil(units / waves);
    // time ~ per-wave units x slice length; fewer slices also mean less
    // partial traffic, so ties go to the smaller split
    const double eff = units / (waves * per) * ((double)stream_grid(ks) / kCUs);
    if (eff > best_eff + 0.02) { best_eff = eff; best = ks; }
    if (eff >= 0.9) break;
  }
  if (!best) return false;
  ks_out = best;
  return true;
}

template <class Epi, bool LO>
hipError_t launch_stream(const SkinnyA& a, const typename Epi::P& ep, int n_vcols, int ks,
                         const SplitWs& ws, hipStream_t st) {
  const int kc = a.K / ks;
  // slices of at most 512 k (the short products) leave LDS for a fourth ring
  // slot per wave: three slots in flight instead of two
  if (kc <= kSliceMax / 2)
    hipLaunchKernelGGL((stream_gemm<kStreamRing + 1, kStreamBatch, LO, Epi, kSliceMax / 2>),
                       dim3(stream_grid(ks)), dim3(kSW * 64), 0, st, a, ep, n_vcols, ks, kc, ws.part);
  else
    hipLaunchKernelGGL((stream_gemm<kStreamRing, kStreamBatch, LO, Epi>), dim3(stream_grid(ks)),
                       dim3(kSW * 64), 0, st, a, ep, n_vcols, ks, kc, ws.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ks > kFinishBatch)
    hipLaunchKernelGGL((stream_finish<Epi, 2 * kFinishBatch>), dim3((n_vcols + 31) / 32), dim3(256), 0,
                       st, a, ep, ks, ws.part);
  else
    hipLaunchKernelGGL((stream_finish<Epi>), dim3((n_vcols + 31) / 32), dim3(256), 0, st, a, ep, ks,
                       ws.part);
  return hipGetLastError();
}

// true when launch_skinny takes the LDS-staged kernel for this shape
bool uses_stream(const SkinnyA& a, int n_vcols, const SplitWs& ws, int& ks) {
  if (!ws.part || !stream_plan(a.M, n_vcols, a.K, ks)) return false;
  const size_t floats = (size_t)((n_vcols + 31) / 32) * 2 * ks * 256;
  // partial stores take 32-bit byte offsets
  return floats <= ws.part_floats && floats * 4 < ((size_t)1 << 31);
}

// A draft epilogue on the tiled MFMA GEMM, for batches of more than 64
// rows: the weights are read once per 128-row tile instead of once per
// 64-row block. The activations' bf16 hi and lo halves are stacked in the
// tile's A rows (hi.W + lo.W summed in the epilogue). The RMSNorm row
// scales of the tile's rows come from the producer's per-32-column sums of
// x^2, read in the GEMM's prologue; the epilogue runs on each 64-row slice
// in place.
template <class E>
struct EpiTiled {
  static constexpr bool kStack = true;  // the draft's hi/lo activations
  struct P {
    typename E::P ep;
    const float* ssq;  // optional: per-row partial sums of x^2 [rows_in][ssq_ld]
    int ssq_ld, K;
    float eps;
    int a_group, a_stride, a_off;  // output row -> input row (as SkinnyA)
  };
  __device__ static const bf16_t* wrow(const P& p, int n) { return E::wrow(p.ep, n); }
  // the RMSNorm row scales of every row of the tile, indexed by row % 256
  __device__ static float* rs_buf() {
    __shared__ float rs[256];
    return rs;
  }
  // Row scales of the tile's rows, computed once per workgroup before its
  // main loop: eight threads per row, each summing every eighth pair of the
  // row's partial sums (all requested before any is added), then three lane
  // exchanges. (Per 64-row slice in the epilogue, with a wave reduction per
  // row, this cost more than the rest of the epilogue: the loads wait behind
  // the other workgroups' operand streams.)
  __device__ static void prologue(const P& p, int m0, int rows, int M) {
    float* rs = rs_buf();
    constexpr int TPR = 8;
    for (int e0 = 0; e0 < rows * TPR; e0 += blockDim.x) {
      const int e = e0 + threadIdx.x;
      const int r = e / TPR, q = e % TPR, m = m0 + r;
      const bool ok = p.ssq && e < rows * TPR && m < M;
      float s = 0.f;
      if (ok) {
        const int mi = (m / p.a_group) * p.a_stride + p.a_off + m % p.a_group;
        const float2* row = reinterpret_cast<const float2*>(p.ssq + (size_t)mi * p.ssq_ld);
        const int n2 = p.ssq_ld >> 1;  // the row holds D / 32 sums, D a multiple of 64
        for (int c0 = q; c0 < n2; c0 += 8 * TPR) {
          float2 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int c = c0 + u * TPR;
            v[u] = row[c < n2 ? c : n2 - 1];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (c0 + u * TPR < n2) s += v[u].x + v[u].y;
        }
      }
      static_assert(TPR == 8, "eight-lane groups");
      s = row8_sum(s);
      if (q == 0 && e < rows * TPR) rs[m & 255] = p.ssq ? rsqrtf(s / (float)p.K + p.eps) : 1.f;
    }
  }
  // C: the slice, row pitch BN + 8 (the tiled kernel's)
  template <int BN>
  __device__ static void run(const P& p, const float* C, int ld, int m0, int n0, int M) {
    float* tile = const_cast<float*>(C);
    const float* rs = rs_buf() + (m0 & 255);  // slices start at multiples of 64
    E::template run<kSlice, BN, BN + 8>(p.ep, reinterpret_cast<float (*)[BN + 8]>(tile), rs, n0, m0, M);
  }
};

constexpr int kTallBN = 256;

// Products whose epilogue works on 16-column groups of any tile width take
// 192-wide tiles where that fills the CUs better: at 512 draft rows qkv's
// 96 tiles of 256 (x 2 splits) leave a quarter of the CUs idle and gate/up's
// 384 tiles take two rounds of which the second is half empty, while 192-wide
// tiles give 128 x 2 and 512 (two full rounds).
template <class E>
struct TallNarrow {
  static constexpr bool ok = false;
};
template <>
struct TallNarrow<EpiQKV> {
  static constexpr bool ok = true;
};
template <>
struct TallNarrow<EpiSwiglu> {
  static constexpr bool ok = true;
};

// rounds of workgroups x work per workgroup, for a tile width (stacked hi/lo
// tiles: 128 output rows)
double tall_cost(int M, int N, int K, int BN) {
  const int tiles = ((M + 127) / 128) * ((N + BN - 1) / BN);
  const int S = choose_split(tiles, K, 8, 512);
  const int rounds = (((tiles + 7) & ~7) * S + kCUs - 1) / kCUs;
  return (double)rounds * BN * ((double)K / S);
}

template <class Epi>
hipError_t launch_tall(const SkinnyA& a, const typename Epi::P& ep, int n_vcols, const GemmWs& gw,
                       hipStream_t st) {
  GemmA g;
  for (int i = 0; i < kMaxFeat; ++i) g.seg[i] = a.xh;
  g.ld = a.lda; g.seg_k = a.K; g.M = a.M; g.K = a.K; g.b_k = a.K;
  g.stack = 1;
  // both halves have the same row pitch; the offset between the two buffers
  // in elements (both are 2-byte aligned)
  g.lo_off = ((intptr_t)a.xl - (intptr_t)a.xh) / (intptr_t)sizeof(bf16_t);
  g.a_group = a.a_group; g.a_stride = a.a_stride; g.a_off = a.a_off;
  typename EpiTiled<Epi>::P p;
  p.ep = ep; p.ssq = a.ssq; p.ssq_ld = a.ssq_ld; p.K = a.K; p.eps = a.eps;
  p.a_group = a.a_group; p.a_stride = a.a_stride; p.a_off = a.a_off;
  // the draft's few-tile products (o_proj, down at 512 rows: 64 tiles) split
  // K up to 8 ways, down to 512 k per split
  if constexpr (TallNarrow<Epi>::ok) {
    if (tall_cost(a.M, n_vcols, a.K, 192) < tall_cost(a.M, n_vcols, a.K, kTallBN))
      return launch_tiled<192, EpiTiled<Epi>>(g, p, n_vcols, gw, st, 8, 512);
  }
  return launch_tiled<kTallBN, EpiTiled<Epi>>(g, p, n_vcols, gw, st, 8, 512);
}

// true when launch_skinny takes the tiled GEMM for this shape: more rows
// than one register-streaming block of 64 (which would stream the weights
// once per block)
bool uses_tall(const SkinnyA& a, const GemmWs* tall) {
  return tall && a.M > 64 && a.xl && a.K % kTiledK == 0 && a.seg_k == a.K;
}

template <class Epi, bool LO = true>
hipError_t launch_skinny(const SkinnyA& a, const typename Epi::P& ep, int n_vcols,
                         const SplitWs& ws, hipStream_t st, const GemmWs* tall = nullptr) {
  int ks;
  if (uses_stream(a, n_vcols, ws, ks)) return launch_stream<Epi, LO>(a, ep, n_vcols, ks, ws, st);
  if (LO && uses_tall(a, tall)) return launch_tall<Epi>(a, ep, n_vcols, *tall, st);
  if (a.M <= 16) return launch_cfg<Epi, LO, 1, 4, 4>(a, ep, n_vcols, ws, st);
  if (a.M <= 32) return launch_cfg<Epi, LO, 2, 4, 2>(a, ep, n_vcols, ws, st);
  // more rows: 64-row blocks over grid.y, each streaming the weights again
  return launch_cfg<Epi, LO, 4, 2, 2>(a, ep, n_vcols, ws, st);
}

SkinnyA make_a(const bf16_t* xh, const bf16_t* xl, int lda, int M, int K,
               const float* ssq, int ssq_ld, float eps) {
  SkinnyA a;
  a.xh = xh; a.xl = xl; a.lda = lda; a.M = M; a.K = K;
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = xh;
  a.seg_k = K;
  a.a_group = M > 0 ? M : 1; a.a_stride = 0; a.a_off = 0;
  a.ssq = ssq; a.ssq_ld = ssq_ld; a.eps = eps;
  return a;
}
}  // namespace

int skinny_tile_cols() { return 32; }  // narrowest column block of any configuration
int skinny_max_rows() { return 64; }

size_t stream_part_floats(int n_vcols, int K) {
  int ks;
  if (!stream_plan(16, n_vcols, K, ks)) return 0;
  return (size_t)((n_vcols + 31) / 32) * 2 * ks * 256;
}

// fp32 rows -> bf16 hi/lo (the streaming GEMM's A operand); 4 elements per thread
__global__ void __launch_bounds__(256)
conv_split(const float* __restrict__ x, int D, bf16_t* __restrict__ xh, bf16_t* __restrict__ xl) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= D) return;
  const size_t i = (size_t)blockIdx.y * D + c;
  const float4 v = *reinterpret_cast<const float4*>(x + i);
  const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) split_bf16(a[k], xh[i + k], xl[i + k]);
}

// The finish call of the dynamic conv: base[1] plus the corrections the
// prepare call stored, applied to z; one element per thread, every load
// issued before any use.
__global__ void __launch_bounds__(256)
conv_finish(const float* __restrict__ z, const float* __restrict__ prev,
            const bf16_t* __restrict__ base, const float* __restrict__ corr, int D, int G, int gs,
            int Bl, float* __restrict__ y) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  if (c >= D) return;
  const int t = m % Bl, g = c / gs;
  const float zv = z[(size_t)m * D + c];
  const float zb = t == 0 ? (prev ? prev[(size_t)(m / Bl) * D + c] : 0.f) : z[(size_t)(m - 1) * D + c];
  const float k0 = bf2f(base[2 * D + c]) + corr[(size_t)m * 2 * G + g];
  const float k1 = bf2f(base[3 * D + c]) + corr[(size_t)m * 2 * G + G + g];
  y[(size_t)m * D + c] = k0 * zv + k1 * zb;
}

// RMSNorm of the residual rows in fp32: h = x * gain * rsqrt(mean(x^2) + eps),
// the mean from the producer's per-32-column sums of x^2. One workgroup per
// (row, 1024 columns), four columns per thread.
__global__ void __launch_bounds__(256)
norm_rows(const float* __restrict__ x, const bf16_t* __restrict__ gain,
          const float* __restrict__ ssq, int D, float eps, float* __restrict__ h) {
  const int m = blockIdx.y;
  __shared__ float rs;
  if (threadIdx.x < 64) {
    float s = strided_sum(ssq + (size_t)m * (D / 32), D / 32, threadIdx.x, 64);
    s = wave_sum(s);
    if (threadIdx.x == 0) rs = rsqrtf(s / (float)D + eps);
  }
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
  uint2 gv = make_uint2(0u, 0u);
  if (n < D) {
    xv = *reinterpret_cast<const float4*>(x + (size_t)m * D + n);
    gv = *reinterpret_cast<const uint2*>(gain + n);
  }
  __syncthreads();
  if (n >= D) return;
  const float r = rs;
  float4 o;
  o.x = xv.x * bf2f((bf16_t)(gv.x & 0xffff)) * r;
  o.y = xv.y * bf2f((bf16_t)(gv.x >> 16)) * r;
  o.z = xv.z * bf2f((bf16_t)(gv.y & 0xffff)) * r;
  o.w = xv.w * bf2f((bf16_t)(gv.y >> 16)) * r;
  *reinterpret_cast<float4*>(h + (size_t)m * D + n) = o;
}

// The finish call of a layer's conv followed by the residual add: for row m
// (position t of its block) and channel c,
//   y = (b1[0][c] + corr[m][0][g]) z_t[c] + (b1[1][c] + corr[m][1][g]) z_{t-1}[c],
// z_{-1} = 0, g = c / gs; then x += y, the optional hidden copy, the next
// RMSNorm's input x * gain as a bf16 hi/lo pair and per-32-column sums of
// x^2 (as the residual epilogue of the GEMMs leaves them). One workgroup per
// (row, 1024 columns), four columns per thread, eight threads per 32-column
// group.
__global__ void __launch_bounds__(256)
conv_finish_resid(const float* __restrict__ z, const bf16_t* __restrict__ base,
                  const float* __restrict__ corr, int D, int G, int gs, int Bl,
                  const bf16_t* __restrict__ gain, float* __restrict__ x,
                  float* __restrict__ hidden, bf16_t* __restrict__ xh, bf16_t* __restrict__ xl,
                  float* __restrict__ ssq) {
  const int m = blockIdx.y, t = m % Bl;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  float sq = 0.f;
  if (n < D) {
    const size_t i = (size_t)m * D + n;
    const float4 zv = *reinterpret_cast<const float4*>(z + i);
    const float4 zp = t > 0 ? *reinterpret_cast<const float4*>(z + i - D) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 xv = *reinterpret_cast<const float4*>(x + i);
    const uint2 b0 = *reinterpret_cast<const uint2*>(base + 2 * D + n);  // base[1][0]
    const uint2 b1 = *reinterpret_cast<const uint2*>(base + 3 * D + n);  // base[1][1]
    const uint2 gv = *reinterpret_cast<const uint2*>(gain + n);
    const float* cr = corr + (size_t)m * 2 * G;
    const float zc[4] = {zv.x, zv.y, zv.z, zv.w}, zq[4] = {zp.x, zp.y, zp.z, zp.w};
    const uint32_t bb0[2] = {b0.x, b0.y}, bb1[2] = {b1.x, b1.y}, gg[2] = {gv.x, gv.y};
    float* xp = reinterpret_cast<float*>(&xv);
    bf16_t hi[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int gk = (n + k) / gs;
      const float k0 = bf2f((bf16_t)(k & 1 ? bb0[k >> 1] >> 16 : bb0[k >> 1] & 0xffff)) + cr[gk];
      const float k1 = bf2f((bf16_t)(k & 1 ? bb1[k >> 1] >> 16 : bb1[k >> 1] & 0xffff)) + cr[G + gk];
      const float gn = bf2f((bf16_t)(k & 1 ? gg[k >> 1] >> 16 : gg[k >> 1] & 0xffff));
      xp[k] += k0 * zc[k] + k1 * zq[k];
      split_bf16(xp[k] * gn, hi[k], lo[k]);
      sq += xp[k] * xp[k];
    }
    *reinterpret_cast<float4*>(x + i) = xv;
    if (hidden) *reinterpret_cast<float4*>(hidden + i) = xv;
    *reinterpret_cast<uint2*>(xh + i) =
        make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *reinterpret_cast<uint2*>(xl + i) =
        make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
  sq = row8_sum(sq);
  if (n < D && (threadIdx.x & 7) == 0) ssq[(size_t)m * (D / 32) + n / 32] = sq;
}

hipError_t launch_conv_prepare(const ConvLaunch& C, hipStream_t st) {
  const int M = C.n_seqs * C.Bl;
  SkinnyA a = make_a(C.xh, C.xl, C.D, M, C.D, nullptr, 0, 0.f);
  EpiConv::P p;
  p.proj = C.proj; p.base = C.base; p.x = C.x; p.prev = C.prev; p.y = C.y; p.corr = C.corr;
  p.D = C.D; p.G = C.D / C.gs; p.gs = C.gs; p.Bl = C.Bl; p.n_vcols = 4 * p.G; p.parts = 1;
  p.gain = nullptr; p.yh = nullptr; p.yl = nullptr;
  int ks;
  hipError_t e;
  if (!uses_stream(a, p.n_vcols, C.split, ks)) {
    // the register-streaming kernel reads bf16 hi/lo rows from the workspace
    hipLaunchKernelGGL(conv_split, dim3((C.D / 4 + 255) / 256, M), dim3(256), 0, st, C.x, C.D,
                       C.xh, C.xl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_skinny<EpiConv>(a, p, p.n_vcols, C.split, st);
  }
  // the LDS-staged kernel splits the fp32 rows itself as it stages them
  // the LDS-staged GEMM, then a finisher whose pairs each spread their conv
  // over 8 workgroups (a pair re-reads its 32 KB of partials per workgroup):
  // the finisher grid grows from n_vcols / 32 to 8x that
  p.parts = 8;
  hipLaunchKernelGGL((stream_gemm<kStreamRing, kStreamBatch, true, EpiConv>), dim3(stream_grid(ks)),
                     dim3(kSW * 64), 0, st, a, p, p.n_vcols, ks, C.D / ks, C.split.part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stream_finish<EpiConv>), dim3(p.n_vcols / 32, p.parts), dim3(256), 0, st, a, p,
                     ks, C.split.part);
  return hipGetLastError();
}

hipError_t launch_conv_finish(const ConvLaunch& C, hipStream_t st) {
  hipLaunchKernelGGL(conv_finish, dim3((C.D + 255) / 256, C.n_seqs * C.Bl), dim3(256), 0, st,
                     C.x, C.prev, C.base, C.corr, C.D, C.D / C.gs, C.gs, C.Bl, C.y);
  return hipGetLastError();
}

hipError_t launch_fuse_rows(const FuseLaunch& F, hipStream_t st) {
  SkinnyA a = make_a(F.feats[0], nullptr, (int)F.ld, F.T, F.n_feat * F.D, nullptr, 0, F.eps);
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = i < F.n_feat ? F.feats[i] : F.feats[0];
  a.seg_k = F.D;
  EpiFuseRows::P p;
  p.w = F.w_c; p.K = F.n_feat * F.D; p.D = F.D; p.y = F.y; p.ssq = F.ssq; p.n_vcols = F.D;
  if (F.norm_in_consumer) {
    p.yh = F.out; p.yl = F.out_lo; p.gain = F.gain;
  }
  hipError_t e = launch_skinny<EpiFuseRows, false>(a, p, F.D, F.split, st);
  if (e != hipSuccess || F.norm_in_consumer) return e;
  return launch_fuse_normalize(F.out, F.out_lo, F.y, F.ssq, F.D / 32, F.T, F.D, F.gain, F.eps, st);
}

hipError_t launch_inject_rows(const InjectLaunch& I, hipStream_t st) {
  SkinnyA a = make_a(I.ctx, nullptr, I.D, I.T, I.D, nullptr, 0, 0.f);
  EpiInjectRows::P p;
  for (int i = 0; i < kMaxLayers; ++i) {
    p.wk[i] = i < I.L ? I.wk[i] : I.wk[0];
    p.wv[i] = i < I.L ? I.wv[i] : I.wv[0];
  }
  p.D = I.D; p.Hkv = I.Hkv; p.hd = I.hd; p.pos0 = I.pos0; p.cap = I.cap;
  p.log2_theta = I.log2_theta; p.kv = I.kv; p.n_vcols = I.L * 2 * I.Hkv * I.hd;
  return launch_skinny<EpiInjectRows, false>(a, p, I.L * 2 * I.Hkv * I.hd, I.split, st);
}

hipError_t launch_append_inject(const AppendLaunch& A, hipStream_t st) {
  // with ssq the fused rows are y * gain and the RMSNorm's row scale is
  // applied to the products (it commutes with them)
  SkinnyA a = make_a(A.ctx, A.ctx_lo, A.D, A.T, A.D, A.ssq, A.D / 32, A.eps);
  EpiAppendRows::P p;
  for (int i = 0; i < kMaxLayers; ++i) {
    p.wk[i] = i < A.L ? A.wk[i] : A.wk[0];
    p.wv[i] = i < A.L ? A.wv[i] : A.wv[0];
  }
  p.D = A.D; p.Hkv = A.Hkv; p.hd = A.hd; p.rps = A.rps; p.log2_theta = A.log2_theta;
  p.tau = A.tau; p.seqs = *A.seqs; p.n_vcols = A.L * 2 * A.Hkv * A.hd;
  return launch_skinny<EpiAppendRows, true>(a, p, p.n_vcols, A.split, st);
}

hipError_t launch_embed(const DraftLaunch& L, hipStream_t st) {
  hipLaunchKernelGGL(embed_block, dim3((L.D + 1023) / 1024, L.M), dim3(256), 0, st, L.embed, L.V, L.D,
                     L.anchors, L.mask_id, L.Bl, L.gain0, L.x, L.xh, L.xl, L.ssq,
                     L.block_out);
  return hipGetLastError();
}

hipError_t launch_qkv(const DraftLaunch& L, int layer, const bf16_t* wq,
                      const bf16_t* wk, const bf16_t* wv, hipStream_t st, const bf16_t* ah,
                      const bf16_t* al) {
  // the residual's next-norm input with the norm's row scale, or (ah/al) rows
  // that are already the layer's input
  SkinnyA a = ah ? make_a(ah, al, L.D, L.M, L.D, nullptr, 0, L.eps)
                 : make_a(L.xh, L.xl, L.D, L.M, L.D, L.ssq, L.D / 32, L.eps);
  EpiQKV::P p;
  p.wq = wq; p.wk = wk; p.wv = wv; p.D = L.D; p.Hq = L.Hq; p.Hkv = L.Hkv;
  p.hd = L.hd; p.Bl = L.Bl; p.layer = layer; p.log2_theta = L.log2_theta;
  p.q_out = L.q; p.q_lo = L.q_lo; p.blk_k = L.blk_k; p.blk_v = L.blk_v; p.seqs = *L.seqs;
  return launch_skinny<EpiQKV>(a, p, (L.Hq + 2 * L.Hkv) * L.hd, L.split, st, &L.gemm);
}

hipError_t launch_resid(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah,
                        const bf16_t* al, int K, const bf16_t* gain_next,
                        float* hidden, hipStream_t st) {
  SkinnyA a = make_a(ah, al, K, L.M, K, nullptr, 0, L.eps);
  EpiResid::P p;
  p.w = w; p.K = K; p.D = L.D; p.x = L.x; p.xh = L.xh; p.xl = L.xl;
  p.gain = gain_next; p.ssq = L.ssq; p.hidden = hidden; p.n_vcols = L.D;
  return launch_skinny<EpiResid>(a, p, L.D, L.split, st, &L.gemm);
}

hipError_t launch_swiglu(const DraftLaunch& L, const bf16_t* wg, const bf16_t* wu,
                         hipStream_t st, const bf16_t* ah, const bf16_t* al) {
  SkinnyA a = ah ? make_a(ah, al, L.D, L.M, L.D, nullptr, 0, L.eps)
                 : make_a(L.xh, L.xl, L.D, L.M, L.D, L.ssq, L.D / 32, L.eps);
  EpiSwiglu::P p;
  p.wg = wg; p.wu = wu; p.K = L.D; p.F = L.F; p.ah = L.act_h; p.al = L.act_l; p.n_vcols = 2 * L.F;
  return launch_skinny<EpiSwiglu>(a, p, 2 * L.F, L.split, st, &L.gemm);
}

hipError_t launch_store(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah, const bf16_t* al,
                        int K, float* out, hipStream_t st) {
  SkinnyA a = make_a(ah, al, K, L.M, K, nullptr, 0, L.eps);
  EpiStore::P p;
  p.w = w; p.K = K; p.N = L.D; p.out = out;
  return launch_skinny<EpiStore>(a, p, L.D, L.split, st, &L.gemm);
}

hipError_t launch_norm_rows(const DraftLaunch& L, const bf16_t* gain, hipStream_t st) {
  hipLaunchKernelGGL(norm_rows, dim3((L.D + 1023) / 1024, L.M), dim3(256), 0, st, L.x, gain, L.ssq, L.D,
                     L.eps, L.conv_h);
  return hipGetLastError();
}

hipError_t launch_conv_prepare_draft(const DraftLaunch& L, const bf16_t* base, const bf16_t* proj,
                                     float* corr, hipStream_t st) {
  ConvLaunch C{};
  C.n_seqs = L.n_seqs; C.Bl = L.Bl; C.D = L.D; C.gs = L.conv_gs;
  C.base = base; C.proj = proj; C.x = L.conv_h; C.prev = nullptr; C.y = L.conv_y; C.corr = corr;
  C.xh = L.conv_xh; C.xl = L.conv_xl; C.split = L.split;
  hipError_t e = launch_conv_prepare(C, st);
  if (e != hipSuccess) return e;
  // the conv's output as the sublayer GEMM's bf16 hi/lo input
  hipLaunchKernelGGL(conv_split, dim3((L.D / 4 + 255) / 256, L.M), dim3(256), 0, st, L.conv_y, L.D,
                     L.conv_ah, L.conv_al);
  return hipGetLastError();
}

bool conv_fused(const DraftLaunch& L) {
  // one tile holds every row (the finishers read the previous row of a block
  // from their own tile) and the projection takes the LDS-staged kernel
  if (L.M > 16) return false;
  SkinnyA a = make_a(L.xh, L.xl, L.D, L.M, L.D, L.ssq, L.D / 32, L.eps);
  int ks;
  return uses_stream(a, 4 * (L.D / L.conv_gs), L.split, ks);
}

hipError_t launch_conv_prepare_fused(const DraftLaunch& L, const bf16_t* gain, const bf16_t* base,
                                     const bf16_t* proj, float* corr, hipStream_t st) {
  SkinnyA a = make_a(L.xh, L.xl, L.D, L.M, L.D, L.ssq, L.D / 32, L.eps);
  EpiConvNorm::P p;
  p.proj = proj; p.base = base; p.x = L.x; p.prev = nullptr; p.y = nullptr; p.corr = corr;
  p.D = L.D; p.G = L.D / L.conv_gs; p.gs = L.conv_gs; p.Bl = L.Bl; p.n_vcols = 4 * p.G;
  p.parts = 8; p.gain = gain; p.yh = L.conv_ah; p.yl = L.conv_al;
  int ks;
  if (!uses_stream(a, p.n_vcols, L.split, ks)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((stream_gemm<kStreamRing, kStreamBatch, true, EpiConvNorm>), dim3(stream_grid(ks)),
                     dim3(kSW * 64), 0, st, a, p, p.n_vcols, ks, L.D / ks, L.split.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stream_finish<EpiConvNorm>), dim3(p.n_vcols / 32, p.parts), dim3(256), 0, st, a,
                     p, ks, L.split.part);
  return hipGetLastError();
}

hipError_t launch_conv_resid_fused(const DraftLaunch& L, const bf16_t* w, const bf16_t* ah,
                                   const bf16_t* al, int K, const bf16_t* base, const float* corr,
                                   const bf16_t* gain_next, float* hidden, hipStream_t st) {
  SkinnyA a = make_a(ah, al, K, L.M, K, nullptr, 0, L.eps);
  EpiConvResid::P p;
  p.w = w; p.K = K; p.D = L.D; p.base = base; p.corr = corr;
  p.G = L.D / L.conv_gs; p.gs = L.conv_gs; p.Bl = L.Bl;
  p.x = L.x; p.xh = L.xh; p.xl = L.xl; p.gain = gain_next; p.ssq = L.ssq; p.hidden = hidden;
  p.n_vcols = L.D;
  int ks;
  if (uses_stream(a, L.D, L.split, ks)) return launch_stream<EpiConvResid, true>(a, p, L.D, ks, L.split, st);
  return launch_cfg<EpiConvResid, true, 1, 4, 4>(a, p, L.D, L.split, st);
}

hipError_t launch_conv_finish_resid(const DraftLaunch& L, const bf16_t* base, const float* corr,
                                    const bf16_t* gain_next, float* hidden, hipStream_t st) {
  hipLaunchKernelGGL(conv_finish_resid, dim3((L.D + 1023) / 1024, L.M), dim3(256), 0, st, L.conv_o,
                     base, corr, L.D, L.D / L.conv_gs, L.conv_gs, L.Bl, gain_next, L.x, hidden, L.xh,
                     L.xl, L.ssq);
  return hipGetLastError();
}

namespace {
struct LmPlan {
  SkinnyA a;
  EpiLM::P p;
  int M_lm;
  bool stream;
  bool tall;  // the tiled GEMM (more than 64 rows)
  int ks;   // K slices of the LDS-staged kernel
  int vc;   // vocabulary columns per argmax key
};

LmPlan lm_plan(const DraftLaunch& L, const bf16_t* w_lm, float* logits) {
  LmPlan q;
  const int g = L.Bl - 1;
  q.M_lm = L.n_seqs * g;
  q.a = make_a(L.xh, L.xl, L.D, q.M_lm, L.D, L.ssq, L.D / 32, L.eps);
  q.a.a_group = g; q.a.a_stride = L.Bl; q.a.a_off = 1;
  q.p.w = w_lm; q.p.K = L.D; q.p.V = L.V; q.p.logits = logits; q.p.part = L.lm_part;
  q.ks = 0;
  q.stream = uses_stream(q.a, L.V, L.split, q.ks);
  q.tall = !q.stream && uses_tall(q.a, &L.gemm);
  q.vc = q.stream ? 256 : q.tall ? kTallBN : q.M_lm <= 16 ? 128 : q.M_lm <= 32 ? 64 : 32;
  return q;
}
}  // namespace

hipError_t launch_lm(const DraftLaunch& L, const bf16_t* w_lm, float* logits,
                     hipStream_t st) {
  const LmPlan q = lm_plan(L, w_lm, logits);
  if (q.stream) {  // partial logits; the argmax launch finishes them
    hipLaunchKernelGGL((stream_gemm<kStreamRing, kStreamBatch, true, EpiLM>),
                       dim3(stream_grid(q.ks)), dim3(kSW * 64), 0, st, q.a, q.p, L.V, q.ks,
                       L.D / q.ks, L.split.part);
    return hipGetLastError();
  }
  if (q.tall) return launch_tall<EpiLM>(q.a, q.p, L.V, L.gemm, st);
  // the register-streaming kernel never splits the LM head's K (its vocab
  // gives thousands of column blocks); its epilogue leaves one argmax key per
  // column block and row
  const SplitWs none{};
  if (q.M_lm <= 16) return launch_cfg<EpiLM, true, 1, 8, 2>(q.a, q.p, L.V, none, st);
  if (q.M_lm <= 32) return launch_cfg<EpiLM, true, 2, 4, 2>(q.a, q.p, L.V, none, st);
  return launch_cfg<EpiLM, true, 4, 2, 2>(q.a, q.p, L.V, none, st);
}

hipError_t launch_lm_argmax(const DraftLaunch& L, const bf16_t* w_lm, float* logits,
                            hipStream_t st) {
  const LmPlan q = lm_plan(L, w_lm, logits);
  if (q.stream) {  // slice sums, row scale, logits, one key per 256 columns
    hipLaunchKernelGGL(lm_stream_finish, dim3((L.V + q.vc - 1) / q.vc), dim3(256), 0, st, q.a, q.p,
                       q.ks, L.split.part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tiles = (L.V + q.vc - 1) / q.vc;
  hipLaunchKernelGGL(lm_argmax_reduce, dim3(q.M_lm), dim3(256), 0, st, L.lm_part, tiles, q.M_lm,
                     L.Bl, L.block_out);
  return hipGetLastError();
}

}  // namespace dfl
