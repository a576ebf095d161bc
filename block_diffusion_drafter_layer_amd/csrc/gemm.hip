// Dense context-side GEMMs on bf16 MFMA: C[m][n] = sum_k A[m][k] B[n][k] with
// both operands K-contiguous, 128x128 output tiles, BK = 64, LDS double
// buffering, four waves each owning a 64x64 quarter (4x4 tiles of
// 16x16x32 MFMAs). Rows of LDS tiles are padded to 72 elements (144 bytes) so
// the 16 rows read by one MFMA operand fall in distinct bank groups.
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
    for (int r = threadIdx.x; r < BM; r += kThreads) {
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

template <class Epi>
__global__ void __launch_bounds__(kThreads)
gemm_tile(GemmA a, typename Epi::P p, int N) {
  // two stages of A and B tiles; reused as the fp32 output tile at the end
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * BM * LDK * 2];
  bf16_t (*As)[BM][LDK] = reinterpret_cast<bf16_t (*)[BM][LDK]>(smem);
  bf16_t (*Bs)[BN][LDK] = reinterpret_cast<bf16_t (*)[BN][LDK]>(smem + 2 * BM * LDK * 2);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int KT = a.K / BK;

  // this thread's four 16-byte chunks of each tile: row = c / 8, k = (c % 8) * 8
  const bf16_t* brow[4];
  int arow_off[4];
  int crow[4], ck[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    crow[i] = c >> 3;
    ck[i] = (c & 7) * 8;
    int m = m0 + crow[i];
    m = m < a.M ? m : a.M - 1;
    arow_off[i] = m;
    int n = n0 + crow[i];
    n = n < N ? n : N - 1;
    brow[i] = Epi::wrow(p, n) + ck[i];
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    const int sgi = k0 / a.seg_k, kin = k0 - sgi * a.seg_k;
    const bf16_t* base = a.seg[sgi];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(base + (size_t)arow_off[i] * a.ld + kin + ck[i]);
      rb[i] = *reinterpret_cast<const u32x4*>(brow[i] + k0);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&As[st][crow[i]][ck[i]]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[st][crow[i]][ck[i]]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
      const int kk = ks * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&As[cur][wm * 64 + i * 16 + (lane & 15)][kk]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Bs[cur][wn * 64 + j * 16 + (lane & 15)][kk]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  float (*C)[BN + 1] = reinterpret_cast<float (*)[BN + 1]>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        C[wm * 64 + i * 16 + 4 * (lane >> 4) + e][wn * 64 + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  Epi::run(p, C, m0, n0, a.M);
}

static_assert(BM * (BN + 1) * 4 <= 2 * 2 * BM * LDK * 2, "output tile fits the stage buffers");

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
  dim3 grid(p.n_tiles, (F.T + BM - 1) / BM);
  hipLaunchKernelGGL(gemm_tile<EpiFuse>, grid, dim3(kThreads), 0, st, a, p, F.D);
  hipError_t e = hipGetLastError();
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
  dim3 grid((p.N + BN - 1) / BN, (I.T + BM - 1) / BM);
  hipLaunchKernelGGL(gemm_tile<EpiInject>, grid, dim3(kThreads), 0, st, a, p, p.N);
  return hipGetLastError();
}

}  // namespace dfl
