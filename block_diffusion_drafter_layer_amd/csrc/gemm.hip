// Dense context-side GEMMs on bf16 MFMA: C[m][n] = sum_k A[m][k] B[n][k] with
// both operands K-contiguous. Output tiles of BM x 128 (BM = 256 or 128),
// BK = 64, LDS double buffering, four waves in a 2x2 arrangement each owning
// a (BM/2) x 64 block of 32x32x16 MFMA tiles: a 128x64 wave block reads
// 6 KB of LDS per 262 kFLOP, which keeps the LDS under its bandwidth at full
// MFMA rate. LDS rows are padded to 72 elements (144 bytes). The output tile
// goes through LDS in 128-row halves for the epilogue.
//
// A is read through a segmented loader so the fusion GEMM never materialises
// the concatenation of the target layers (A3-dflash tutorial section 2.1.1:
// concat along the hidden axis): k in [j*D, (j+1)*D) reads layer j's array.
//
// Epilogues (the output tile is staged through LDS as fp32):
//   fuse   - y as bf16 plus per-(row, 128-column tile) sums of y^2; a second
//            kernel applies RMSNorm and the gain (tutorial section 2.1.2);
//   inject - every draft layer's K (RoPE at position pos0 + row) and V,
//            written into the KV-cache layout (txtmix article section 5).
#include "common.h"
#include "launch.h"

namespace dfl {

namespace {
constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;
constexpr int kThreads = 256;
}

struct GemmA {
  const bf16_t* seg[kMaxFeat];
  int64_t ld;      // row stride of every segment (elements)
  int seg_k;       // k extent of one segment
  int M, K;
};

struct EpiFuse {
  struct P {
    const bf16_t* w;  // [N][K]
    int K, N;
    bf16_t* out;      // [M][N]
    float* ssq;       // [M][n_tiles]
    int n_tiles;
  };
  __device__ static const bf16_t* wrow(const P& p, int n) { return p.w + (size_t)n * p.K; }
  __device__ static void run(const P& p, float (*C)[BN + 1], int m0, int n0, int M) {
    for (int e = threadIdx.x; e < BM * BN; e += kThreads) {
      const int r = e / BN, c = e % BN;
      const int m = m0 + r, n = n0 + c;
      if (m < M && n < p.N) p.out[(size_t)m * p.N + n] = f2bf(C[r][c]);
    }
    for (int r = threadIdx.x; r < BM && n0 < p.N; r += kThreads) {
      const int m = m0 + r;
      if (m >= M) continue;
      float s = 0.f;
      for (int c = 0; c < BN && n0 + c < p.N; ++c) s += C[r][c] * C[r][c];
      p.ssq[(size_t)m * p.n_tiles + n0 / BN] = s;
    }
  }
};

struct EpiInject {
  struct P {
    const bf16_t* wk[kMaxLayers];
    const bf16_t* wv[kMaxLayers];
    int K, N;        // N = L * 2 * Hkv * hd
    int Hkv, hd, pos0, cap;
    double log2_theta;
    bf16_t* kv;
  };
  __device__ static const bf16_t* wrow(const P& p, int n) {
    const int kvd = p.Hkv * p.hd;
    const int i = n / (2 * kvd), r = n % (2 * kvd);
    return (r < kvd ? p.wk[i] + (size_t)r * p.K : p.wv[i] + (size_t)(r - kvd) * p.K);
  }
  __device__ static void run(const P& p, float (*C)[BN + 1], int m0, int n0, int M) {
    const int kvd = p.Hkv * p.hd, half = p.hd / 2;
    const size_t plane = (size_t)p.cap * p.hd;
    // K columns: RoPE pairs (d, d + hd/2), consecutive threads along d
    for (int e = threadIdx.x; e < BM * (BN / 2); e += kThreads) {
      const int r = e / (BN / 2), cp = e % (BN / 2);
      const int head_in_tile = cp / half, d = cp % half;
      const int c = head_in_tile * p.hd + d;  // column of the pair's first half
      const int n = n0 + c, m = m0 + r;
      if (m >= M || n >= p.N || c + half >= BN) continue;
      const int i = n / (2 * kvd), rr = n % (2 * kvd);
      if (rr >= kvd) continue;  // V column
      const int h = rr / p.hd;
      const int pos = p.pos0 + m;
      float cs, sn;
      rope_cs(pos, d, p.hd, p.log2_theta, cs, sn);
      const float x1 = C[r][c], x2 = C[r][c + half];
      bf16_t* k = p.kv + (size_t)((2 * i) * p.Hkv + h) * plane + (size_t)pos * p.hd;
      k[d] = f2bf(x1 * cs - x2 * sn);
      k[d + half] = f2bf(x2 * cs + x1 * sn);
    }
    // V columns: dim-major plane, consecutive threads along positions
    for (int e = threadIdx.x; e < BM * BN; e += kThreads) {
      const int c = e / BM, r = e % BM;
      const int n = n0 + c, m = m0 + r;
      if (m >= M || n >= p.N) continue;
      const int i = n / (2 * kvd), rr = n % (2 * kvd);
      if (rr < kvd) continue;
      const int h = (rr - kvd) / p.hd, d = (rr - kvd) % p.hd;
      bf16_t* v = p.kv + (size_t)((2 * i + 1) * p.Hkv + h) * plane;
      v[(size_t)d * p.cap + p.pos0 + m] = f2bf(C[r][c]);
    }
  }
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D[i][j] += sum_k A[i][k] B[k][j], 32x32x16, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32] and
// holds D[8*(v/4) + 4*(l/32) + v%4][l%32] in item v.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int TBM, class Epi>
__global__ void __launch_bounds__(kThreads)
gemm_tile(GemmA a, typename Epi::P p, int N) {
  constexpr int WM = TBM / 2;          // rows per wave
  constexpr int TI = WM / 32, TJ = 2;  // 32x32 tiles per wave
  constexpr int ALD = TBM * BK / 8 / kThreads;  // 16-byte chunks per thread
  constexpr int BLD = BN * BK / 8 / kThreads;
  constexpr int STAGE = (TBM + BN) * LDK;        // bf16 elements per stage
  static_assert(128 * (BN + 1) * 4 <= 2 * STAGE * 2, "epilogue half tile fits");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * TBM, n0 = blockIdx.x * BN;
  const int KT = a.K / BK;
  auto As = [&](int st, int r, int k) -> bf16_t* { return smem + st * STAGE + r * LDK + k; };
  auto Bs = [&](int st, int r, int k) -> bf16_t* { return smem + st * STAGE + (TBM + r) * LDK + k; };

  int arow[ALD], acol[ALD], brow_i[BLD], bcol[BLD];
  int64_t aoff[ALD];
  const bf16_t* bptr[BLD];
#pragma unroll
  for (int i = 0; i < ALD; ++i) {
    const int c = tid + i * kThreads;
    arow[i] = c >> 3;
    acol[i] = (c & 7) * 8;
    int m = m0 + arow[i];
    m = m < a.M ? m : a.M - 1;
    aoff[i] = (int64_t)m * a.ld + acol[i];
  }
#pragma unroll
  for (int i = 0; i < BLD; ++i) {
    const int c = tid + i * kThreads;
    brow_i[i] = c >> 3;
    bcol[i] = (c & 7) * 8;
    int n = n0 + brow_i[i];
    n = n < N ? n : N - 1;
    bptr[i] = Epi::wrow(p, n) + bcol[i];
  }

  u32x4 ra[ALD], rb[BLD];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    const int sgi = k0 / a.seg_k, kin = k0 - sgi * a.seg_k;
    const bf16_t* base = a.seg[sgi] + kin;
#pragma unroll
    for (int i = 0; i < ALD; ++i) ra[i] = *reinterpret_cast<const u32x4*>(base + aoff[i]);
#pragma unroll
    for (int i = 0; i < BLD; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + k0);
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < ALD; ++i) *reinterpret_cast<u32x4*>(As(st, arow[i], acol[i])) = ra[i];
#pragma unroll
    for (int i = 0; i < BLD; ++i) *reinterpret_cast<u32x4*>(Bs(st, brow_i[i], bcol[i])) = rb[i];
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();
  const int lr = lane & 31, lk = 8 * (lane >> 5);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As(cur, wm * WM + i * 32 + lr, ks * 16 + lk)));
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs(cur, wn * 64 + j * 32 + lr, ks * 16 + lk)));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue in 128-row halves of the tile
  float (*C)[BN + 1] = reinterpret_cast<float (*)[BN + 1]>(smem);
#pragma unroll
  for (int half = 0; half < TBM / 128; ++half) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r0 = wm * WM + i * 32;  // tile row of this 32x32 block
      if (r0 / 128 != half) continue;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          C[r0 % 128 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3)][wn * 64 + j * 32 + lr] = acc[i][j][v];
    }
    __syncthreads();
    Epi::run(p, C, m0 + half * 128, n0, a.M);
    __syncthreads();
  }
}


// 256-row tiles when the grid still fills the chip evenly, else 128-row tiles
template <class Epi>
static hipError_t launch_tiled(const GemmA& a, const typename Epi::P& p, int N, int M,
                               hipStream_t st) {
  const int nb = (N + BN - 1) / BN;
  const int t256 = nb * ((M + 255) / 256);
  if (t256 >= 1024 || (t256 >= 256 && t256 % 256 == 0))
    hipLaunchKernelGGL((gemm_tile<256, Epi>), dim3(nb, (M + 255) / 256), dim3(kThreads), 0, st, a, p, N);
  else
    hipLaunchKernelGGL((gemm_tile<128, Epi>), dim3(nb, (M + 127) / 128), dim3(kThreads), 0, st, a, p, N);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256)
fuse_normalize(bf16_t* __restrict__ out, const float* __restrict__ ssq, int n_tiles, int D,
               const bf16_t* __restrict__ gain, float eps) {
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
#pragma unroll 4
  for (int n = threadIdx.x; n < D; n += 256) {
    bf16_t* o = out + (size_t)m * D + n;
    *o = f2bf(bf2f(*o) * r * bf2f(gain[n]));
  }
}

hipError_t launch_fuse(const FuseLaunch& F, hipStream_t st) {
  GemmA a;
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = i < F.n_feat ? F.feats[i] : F.feats[0];
  a.ld = F.ld; a.seg_k = F.D; a.M = F.T; a.K = F.n_feat * F.D;
  EpiFuse::P p;
  p.w = F.w_c; p.K = a.K; p.N = F.D; p.out = F.out; p.ssq = F.ssq;
  p.n_tiles = (F.D + BN - 1) / BN;
  hipError_t e = launch_tiled<EpiFuse>(a, p, F.D, F.T, st);
  if (e != hipSuccess) return e;
  return launch_fuse_normalize(F.out, F.ssq, p.n_tiles, F.T, F.D, F.gain, F.eps, st);
}

hipError_t launch_fuse_normalize(bf16_t* out, const float* ssq, int n_parts, int T, int D,
                                 const bf16_t* gain, float eps, hipStream_t st) {
  hipLaunchKernelGGL(fuse_normalize, dim3(T), dim3(256), 0, st, out, ssq, n_parts, D, gain, eps);
  return hipGetLastError();
}

hipError_t launch_inject(const InjectLaunch& I, hipStream_t st) {
  GemmA a;
  for (int i = 0; i < kMaxFeat; ++i) a.seg[i] = I.ctx;
  a.ld = I.D; a.seg_k = I.D; a.M = I.T; a.K = I.D;
  EpiInject::P p;
  for (int i = 0; i < kMaxLayers; ++i) {
    p.wk[i] = i < I.L ? I.wk[i] : I.wk[0];
    p.wv[i] = i < I.L ? I.wv[i] : I.wv[0];
  }
  p.K = I.D; p.N = I.L * 2 * I.Hkv * I.hd; p.Hkv = I.Hkv; p.hd = I.hd; p.pos0 = I.pos0;
  p.cap = I.cap; p.log2_theta = I.log2_theta; p.kv = I.kv;
  return launch_tiled<EpiInject>(a, p, p.N, I.T, st);
}

}  // namespace dfl
