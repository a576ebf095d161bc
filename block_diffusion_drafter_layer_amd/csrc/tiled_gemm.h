// Dense GEMMs on bf16 MFMA: C[m][n] = sum_k A[m][k] B[n][k] with both operands
// K-contiguous.
//
// Output tiles of 256 x BN (BN = 256 for the fusion, 320 for the injection,
// 192 or 256 for the draft's tall products), eight waves (two per SIMD), each
// owning a block of 32x32x16 MFMA tiles: 128 x 64 for BN = 256, 64 x 160 for
// BN = 320, 64 x 96 for BN = 192. Large tiles keep the global
// load traffic at ~30 B/clk per CU at full MFMA rate, half of what the
// CU's load path sustains (a 256 x 128 tile needs ~47 B/clk and is bound by
// it). Operands go straight from global memory into LDS
// (global_load_lds_dwordx4, no register staging) in 64-wide k stages, two of
// them (64 or 72 KB each): while one is multiplied the next one loads. Each
// 1 KB load instruction covers eight 128-byte tile rows: the load path keeps
// a bounded number of requests in flight per CU, and 128-byte row pieces move
// more bytes per request than 64-byte ones. 16-byte chunk c of row r is
// stored at chunk c ^ ((r >> 1) & 7), so a fragment read (sixteen
// consecutive lanes on sixteen rows, same chunk) touches 64 distinct banks.
// Fragment reads for the next 16-wide k step are issued before the MFMAs of
// the current one.
//
// Split K: when the tiles alone would leave CUs idle, S workgroups share a
// tile, each over K/S. Each writes its fp32 partial and counts itself in on
// the tile's counter with an agent-scope release (its partial is written back
// past its XCD's L2 before the count); the last to arrive takes an
// agent-scope acquire (stale lines of its L1 and L2 dropped) before it adds
// the others' partials in split order and runs the epilogue. The splits may
// therefore run on any XCDs. Workgroup ids are still laid out so that the S
// of a tile are consecutive on one XCD (ids 8 apart), where their partials
// meet in one L2. Nobody waits for anybody, so there is no co-residency
// requirement.
//
// Epi supplies kStack (whether its tiles are stacked hi/lo pairs, below),
// wrow(p, n) (B row n), prologue(p, m0, rows, M) (run by every
// workgroup after its first loads are issued; it may read memory and write
// LDS of its own for the epilogue) and run<BN>(p, C, ld, m0, n0, M) (a
// 64-row slice of the tile in LDS).
//
// Users: the prefill fusion and injection (gemm.hip) and the draft GEMMs of
// batches too tall for the weight-streaming kernels (skinny.hip). The A
// operand may be read through segments (k in [j*seg_k, (j+1)*seg_k) reads
// seg[j]) and a row map; B rows are Epi::wrow(p, n) and their k index wraps
// at b_k. A bf16 hi/lo pair of activations is multiplied "stacked": the
// tile's A rows 2j and 2j + 1 are the hi and lo halves of output row j (128
// output rows per tile), against one B tile; the two products land in
// adjacent items of one lane, and the epilogue adds them in registers. Each B tile is then read once per 128 output rows
// (the alternative, [hi | lo] x [W | W] over 2K, reads it twice per 256 rows
// with the two reads K apart, which no cache keeps).
#pragma once
#include "common.h"
#include "launch.h"

namespace dfl {

namespace {
constexpr int BM = 256, BK = kTiledK;
constexpr int kRow = BK * 2;         // bytes per tile row and stage
constexpr int NS = 2;                // stages in LDS
constexpr int kLds = 160 * 1024;
constexpr int kSlice = 64;           // epilogue rows per LDS pass

template <int BN>
struct TileCfg;
template <>
struct TileCfg<256> {
  static constexpr int W = 8, WGM = 2;  // waves, waves along M
};
template <>
struct TileCfg<320> {
  static constexpr int W = 8, WGM = 4;
};
template <>
struct TileCfg<192> {
  static constexpr int W = 8, WGM = 4;  // 64 x 96 per wave
};
}  // namespace

struct GemmA {
  const bf16_t* seg[kMaxFeat];
  int64_t ld;      // row stride of every segment (elements)
  int seg_k;       // k extent of one segment
  int M, K;
  int b_k;         // B's k extent: B's k index is k for k < b_k, k - b_k above (K <= 2 b_k)
  // output row m reads A row (m / a_group) * a_stride + a_off + m % a_group
  int a_group, a_stride, a_off;
  // stacked hi/lo (stack = 1): the tile holds BM / 2 output rows; its A rows
  // BM / 2 .. BM - 1 repeat rows 0 .. BM / 2 - 1 at element offset lo_off
  // (the lo halves' buffer minus the hi halves')
  int stack = 0;
  int64_t lo_off = 0;
};

// A read in place: row m is row m, B's k index is k
__device__ __host__ inline void gemm_a_plain(GemmA& a) {
  a.b_k = a.K;
  a.a_group = a.M > 0 ? a.M : 1;
  a.a_stride = 0;
  a.a_off = 0;
}

// split-K bookkeeping of one launch
struct GemmSplit {
  int S;           // workgroups per tile
  float* part;     // [tile][S][BM * BN] fp32 partials in MFMA register order
  int32_t* ctr;    // [tile] arrival counters, zero between launches
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D[i][j] += sum_k A[i][k] B[k][j], 32x32x16, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32] and
// holds D[8*(v/4) + 4*(l/32) + v%4][l%32] in item v.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte fragment read at addr + OFF, issued without waiting. Inline
// assembly: the compiler's wait-count pass would otherwise treat it as
// aliasing the direct loads in flight into the other stages and drain those
// first. Reads are ordered among themselves (volatile) and complete in order.
template <int OFF>
__device__ __forceinline__ void ds_frag(u32x4& f, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "n"(OFF) : "memory");
}

// Wait until at most N LDS reads are outstanding; the fragments passed through
// become usable only after this point.
template <int N>
__device__ __forceinline__ void frag_wait(u32x4 (&f)[6]) {
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5])
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void frag_wait(u32x4 (&f)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                 "+v"(f[6]), "+v"(f[7])
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void frag_wait(u32x4 (&f)[5]) {
  asm volatile("s_waitcnt lgkmcnt(%5)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4])
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void frag_wait(u32x4 (&f)[7]) {
  asm volatile("s_waitcnt lgkmcnt(%7)"
               : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                 "+v"(f[6])
               : "n"(N));
}

// the TI A fragments (32-row blocks 32 * kRow = 4 KB apart) then the TJ B
// fragments
template <int TI, int TJ>
__device__ __forceinline__ void frag_issue(u32x4 (&f)[TI + TJ], uint32_t a, uint32_t b) {
  static_assert(32 * kRow == 4096, "fragment block stride");
  ds_frag<0>(f[0], a);
  ds_frag<4096>(f[1], a);
  if constexpr (TI > 2) {
    ds_frag<8192>(f[2], a);
    ds_frag<12288>(f[3], a);
  }
  ds_frag<0>(f[TI], b);
  ds_frag<4096>(f[TI + 1], b);
  if constexpr (TJ > 2) ds_frag<8192>(f[TI + 2], b);
  if constexpr (TJ > 3) ds_frag<12288>(f[TI + 3], b);
  if constexpr (TJ > 4) ds_frag<16384>(f[TI + 4], b);
}


// s_waitcnt immediate: vmcnt <= n with the other counters open
#define DFL_VM(n) ((((n) & 15) | (((n) >> 4) << 14)) | 0xF70)

template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(DFL_VM(N)); }

// Workgroup -> (tile, split). The tile count is padded to a multiple of 8
// (the launch's grid covers the padding; those workgroups return at once).
// XCD x (workgroup id % 8) takes a contiguous chunk of tiles, walked in
// groups of 4 tile rows column by column, so the workgroups an XCD runs at
// one time share A row blocks and B column blocks through its L2; the S
// splits of a tile are consecutive on that XCD. Returns false for padding.
__device__ __forceinline__ bool tile_of(int id, int tm, int tn, int S, int& rt, int& ct, int& s) {
  const int nt = tm * tn;
  const int nt8 = (nt + 7) & ~7;
  const int local = id >> 3;
  s = local % S;
  const int t = (id & 7) * (nt8 >> 3) + local / S;
  if (t >= nt) return false;
  constexpr int GR = 4;
  const int g = t / (GR * tn);
  const int rows = min(GR, tm - g * GR);
  const int i = t - g * GR * tn;
  rt = g * GR + i % rows;
  ct = i / rows;
  return true;
}

template <int BN, class Epi>
__global__ void __launch_bounds__(TileCfg<BN>::W * 64)
ctx_gemm(GemmA a, typename Epi::P p, int N, GemmSplit sp) {
  using Cfg = TileCfg<BN>;
  constexpr int kWaves = Cfg::W;
  constexpr int WGM = Cfg::WGM, WGN = kWaves / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int kStage = (BM + BN) * kRow;
  constexpr int kLoadsA = BM / 8 / kWaves;            // A loads per wave and stage
  constexpr int kLoadsBTot = BN / 8;                  // B loads per stage
  constexpr int kLoadsBMax = (kLoadsBTot + kWaves - 1) / kWaves;
  static_assert(NS * kStage <= kLds, "ring fits in LDS");
  static_assert(kSlice * (BN + 8) * 4 + 16 * BN <= NS * kStage,
                "epilogue slice and column table fit in the ring");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;
  constexpr int BMH = BM / 2;
  // stacked hi/lo tiles are a property of the epilogue type, so that each
  // instantiation holds one layout's code (both in one kernel spilled)
  constexpr bool ST = Epi::kStack;
  const int bm_out = ST ? BMH : BM;  // output rows per tile
  const int tm = (a.M + bm_out - 1) / bm_out, tn = (N + BN - 1) / BN;
  int rt, ct, sidx;
  if (!tile_of(blockIdx.x, tm, tn, sp.S, rt, ct, sidx)) return;
  const int m0 = rt * bm_out, n0 = ct * BN;
  const int KT_all = a.K / BK;
  const int kt_per = (KT_all + sp.S - 1) / sp.S;
  const int kt0 = sidx * kt_per;
  const int KT = max(0, min(KT_all - kt0, kt_per));

  // Loads: instruction b covers tile rows 8b .. 8b+7 (of A, then of B);
  // wave w issues A instructions w, w + 8, ... and B instructions w, w + 8,
  // ... Lane l fetches row r = 8b + l/8, chunk (l%8) ^ ((r >> 1) & 7), and
  // lands at byte 16 l of the instruction's kilobyte.
  const int lrow = lane >> 3;
  auto lchunk = [&](int b) { return ((lane & 7) ^ (((8 * b + lrow) >> 1) & 7)) * 8; };
  const int nb = (kLoadsBTot % kWaves == 0 || w < kLoadsBTot % kWaves) ? kLoadsBMax : kLoadsBMax - 1;
  int64_t aoff[kLoadsA];
  const bf16_t* bptr[kLoadsBMax];
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q) {
    const int b = w + kWaves * q;
    const int r = 8 * b + lrow;
    const bool lo = ST && (r & 1);
    int m = m0 + (ST ? r >> 1 : r);
    m = m < a.M ? m : a.M - 1;
    m = (m / a.a_group) * a.a_stride + a.a_off + m % a.a_group;
    aoff[q] = (int64_t)m * a.ld + lchunk(b) + (lo ? a.lo_off : 0);
  }
#pragma unroll
  for (int q = 0; q < kLoadsBMax; ++q) {
    const int b = w + kWaves * q;
    int n = n0 + 8 * b + lrow;
    n = n < N ? n : N - 1;
    bptr[q] = Epi::wrow(p, n) + lchunk(b);
  }
  // the current A segment: its pointer is loaded only when a stage enters a
  // new segment (a load of it every stage would come with a wait that also
  // drains the fragment reads in flight)
  int seg_cur = -1;
  const bf16_t* seg_base = nullptr;
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NS) * kStage;
    const int k0 = (kt0 + kt) * BK;
    const int sg = k0 / a.seg_k;
    if (sg != seg_cur) {
      seg_cur = sg;
      seg_base = a.seg[sg];
      asm volatile("" : "+s"(seg_base));  // complete here, not at every stage's join
    }
    const bf16_t* base = seg_base + (k0 - sg * a.seg_k);
    const int kb = k0 < a.b_k ? k0 : k0 - a.b_k;
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) dma16(base + aoff[q], st + (w + kWaves * q) * 1024);
#pragma unroll
    for (int q = 0; q < kLoadsBMax; ++q)
      if (q < nb) dma16(bptr[q] + kb, st + BM * kRow + (w + kWaves * q) * 1024);
  };
  // fragment addresses: lane l reads row l % 32 of a 32-row block at chunk
  // (2 kk + l / 32) ^ (((l % 32) >> 1) & 7), kk the 16-wide step within the
  // stage (32-row blocks start at multiples of 32, so the swizzle of a row
  // depends on l % 32 alone)
  constexpr int KK = BK / 16;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  const int fr = lane & 31;
  uint32_t foff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    foff[kk] = fr * kRow + (((2 * kk + (lane >> 5)) ^ ((fr >> 1) & 7)) << 4);
  const uint32_t a_f = sbase + (uint32_t)(wm * WM) * kRow;
  const uint32_t b_f = sbase + (uint32_t)(BM * kRow) + (uint32_t)(wn * WN) * kRow;

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stage t sits in slot t % 2 and is multiplied in four 16-wide k steps;
  // each step issues the next step's fragment reads before its own MFMAs.
  // Stage t + 1 is loaded into the other slot from the start of stage t: its
  // previous contents (stage t - 1) were read by every wave before the
  // barrier that opened stage t. The last step waits for this wave's loads
  // of stage t + 1 and meets the other waves at a barrier; past it stage
  // t + 1 is in LDS, and its first fragments are read under the MFMAs of
  // stage t's last step. (A plain barrier: a fence would also wait for loads
  // still in flight.)
  // the epilogue's own inputs (e.g. row scales) are requested here, so that
  // their latency overlaps the first stage's loads instead of the end
  if (KT > 0) issue(0);
  Epi::prologue(p, m0, bm_out, a.M);
  if (KT > 0) {
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    u32x4 f[2][TI + TJ];
    frag_issue<TI, TJ>(f[0], a_f + foff[0], b_f + foff[0]);
    for (int kt = 0; kt < KT; ++kt) {
      const uint32_t st = (uint32_t)((kt & 1) * kStage);
      if (kt + 1 < KT) issue(kt + 1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          frag_issue<TI, TJ>(f[(kk + 1) & 1], a_f + st + foff[kk + 1], b_f + st + foff[kk + 1]);
          frag_wait<TI + TJ>(f[kk & 1]);
        } else {
          frag_wait<0>(f[kk & 1]);
          if (kt + 1 < KT) {
            wait_vm<0>();
            __builtin_amdgcn_s_barrier();
            const uint32_t sn = (uint32_t)(((kt + 1) & 1) * kStage);
            frag_issue<TI, TJ>(f[0], a_f + sn + foff[0], b_f + sn + foff[0]);
          }
        }
        // the MFMAs go out at raised priority, so that the other wave on the
        // SIMD issues its reads and loads around them rather than the two
        // waves' MFMA bursts queueing behind each other
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = mfma32x32x16(__builtin_bit_cast(bf16x8, f[kk & 1][i]),
                                     __builtin_bit_cast(bf16x8, f[kk & 1][TI + j]), acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
        // keep this step's MFMAs ahead of the next step's reads and waits
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (sp.S > 1) {
    // publish this split's partial (lane-major: 1 KB per store instruction),
    // then count in; the last to arrive sums every partial in split order
    // (stacked tiles: the hi + lo sums only, items 2k + 1 left at zero by the
    // last arriver, so half the partial bytes)
    const int tile = rt * tn + ct;
    float* mine = sp.part + ((size_t)tile * sp.S + sidx) * (BM * BN);
    constexpr int NQ = ST ? 2 : 4;  // 16-byte pieces per lane and 32x32 block
    if constexpr (ST) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int b = 8 * q;
            f32x4 v = {acc[i][j][b] + acc[i][j][b + 1], acc[i][j][b + 2] + acc[i][j][b + 3],
                       acc[i][j][b + 4] + acc[i][j][b + 5], acc[i][j][b + 6] + acc[i][j][b + 7]};
            store16_wt(mine, (uint32_t)(((((w * TI + i) * TJ + j) * 2 + q) * 64 + lane) * 16), v);
          }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            store16_wt(mine, (uint32_t)(((((w * TI + i) * TJ + j) * 4 + q) * 64 + lane) * 16), v);
          }
    }
    // this wave's partial is written (through the L2: the release below then
    // has little to write back)
    __builtin_amdgcn_s_waitcnt(DFL_VM(0));
    __syncthreads();  // every wave's has (also: every wave is done with the ring)
    int32_t* arrived = reinterpret_cast<int32_t*>(smem);
    // agent-scope release: the workgroup's partial (all waves' stores, ordered
    // before this point by the barrier) is visible on every XCD before the
    // count; the last arriver's acquire makes the others' partials visible
    // to it
    if (tid == 0)
      *arrived = __hip_atomic_fetch_add(sp.ctr + tile, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*arrived != sp.S - 1) return;
    if (tid == 0) __hip_atomic_store(sp.ctr + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // split by split, a row block's loads of a split's partial all issued
    // before its adds (the loop over splits outermost, so that the loads of
    // the next blocks can go out under the adds of this one)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    for (int s = 0; s < sp.S; ++s) {
      const float* src = sp.part + ((size_t)tile * sp.S + s) * (BM * BN);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        f32x4 v[TJ][4];
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < NQ)
              v[j][q] = *reinterpret_cast<const f32x4*>(
                  src + ((((w * TI + i) * TJ + j) * NQ + q) * 64 + lane) * 4);
        if constexpr (ST) {
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][j][8 * q + 2 * e] += v[j][q][e];
        } else {
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += v[j][q][e];
        }
      }
    }
  }

  // epilogue: 64-row slices through LDS
  constexpr int CLD = BN + 8;
  float* C = reinterpret_cast<float*>(smem);
  __syncthreads();  // every wave is done with the ring
  if constexpr (ST) {
    // tile rows 2j and 2j + 1 (the hi and lo halves of output row j) sit in
    // items v and v + 1 of one lane: their sum is stored once per slice
#pragma unroll
    for (int sl = 0; sl < BMH / kSlice; ++sl) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r0 = wm * WM + i * 32;
        if ((r0 >> 1) / kSlice != sl) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const int r = r0 % (2 * kSlice) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            C[(r >> 1) * CLD + wn * WN + j * 32 + fr] = acc[i][j][v] + acc[i][j][v + 1];
          }
      }
      __syncthreads();
      Epi::template run<BN>(p, C, CLD, m0 + sl * kSlice, n0, a.M);
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int sl = 0; sl < BM / kSlice; ++sl) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r0 = wm * WM + i * 32;
      if (r0 / kSlice != sl) continue;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = r0 % kSlice + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          C[r * CLD + wn * WN + j * 32 + fr] = acc[i][j][v];
        }
    }
    __syncthreads();
    Epi::template run<BN>(p, C, CLD, m0 + sl * kSlice, n0, a.M);
    __syncthreads();
  }
}

// Split count: K is split while the doubled grid still fits one workgroup
// per CU and each split keeps at least min_k of K (its prologue and epilogue
// are then a small part of it). The splits of a tile run on one XCD
// (tile_of), which keeps their partials in one L2; the counter's
// release/acquire does not depend on that placement.
static int choose_split(int tiles, int K, int max_split, int min_k) {
  int S = 1;
  while (2 * S <= max_split && tiles * 2 * S <= 256 && K / (2 * S) >= min_k) S *= 2;
  return S;
}

template <int BN, class Epi>
static hipError_t launch_tiled(const GemmA& a, const typename Epi::P& p, int N, const GemmWs& ws,
                               hipStream_t st, int max_split = kGemmMaxSplit, int min_k = 1024) {
  // whole 64-wide k stages, none straddling an A segment or B's wrap
  if (a.K % BK || a.seg_k % BK || a.b_k % BK) return hipErrorInvalidValue;
  if ((a.stack != 0) != Epi::kStack) return hipErrorInvalidValue;
  const int bm_out = a.stack ? BM / 2 : BM;
  const int tiles = ((a.M + bm_out - 1) / bm_out) * ((N + BN - 1) / BN);
  GemmSplit sp;
  sp.S = choose_split(tiles, a.K, max_split, min_k);
  if (sp.S > 1 && (!ws.part || !ws.ctr || (size_t)tiles * sp.S * BM * BN > ws.part_floats ||
                   tiles > ws.n_ctr))
    sp.S = 1;
  sp.part = ws.part;
  sp.ctr = ws.ctr;
  const int grid = ((tiles + 7) & ~7) * sp.S;  // tile_of's padding to whole XCD chunks
  hipLaunchKernelGGL((ctx_gemm<BN, Epi>), dim3(grid), dim3(TileCfg<BN>::W * 64), 0, st, a, p, N,
                     sp);
  return hipGetLastError();
}

}  // namespace dfl
