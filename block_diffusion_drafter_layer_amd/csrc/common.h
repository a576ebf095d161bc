// Shared device helpers for the gfx950 kernels of the DFlash hot path:
// bf16 storage conversions, the 16x16x32 bf16 MFMA, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16_t;  // storage type: raw bf16 bits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxSeqs = 64;
constexpr int kMaxHeadDim = 128;  // the largest head size the library accepts

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (low half = a), one conversion instruction
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi): the pair carries ~16
// significant bits, so a product against exact bf16 weights through two
// MFMAs is close to fp32 accurate.
__device__ __forceinline__ void split_bf16(float v, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

// 16 bytes (8 bf16) from global memory as an MFMA operand.
__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = f2bf2(v[2 * i], v[2 * i + 1]);
  return __builtin_bit_cast(bf16x8, r);
}

// hi/lo pair of 8 values packed as two MFMA operands
__device__ __forceinline__ void pack_split_bf16x8(const float* v, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2bf2(v[2 * i], v[2 * i + 1]);
    const float h0 = __uint_as_float(h[i] << 16), h1 = __uint_as_float(h[i] & 0xffff0000u);
    l[i] = f2bf2(v[2 * i] - h0, v[2 * i + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// D[i][j] += sum_k A[i][k] B[k][j], 16x16x32, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] and
// holds D[4*(l/16) + e][l%16], e = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x of another lane of the same 16-lane row, by a DPP lane pattern
// (quad_perm 0xB1: lane ^ 1; quad_perm 0x4E: lane ^ 2; 0x141: mirror within
// 8 lanes; 0x140: mirror within 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_lane(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over lanes l, l ^ 1, l ^ 2, l ^ 3 (each lane pairs with a partner
// that computes the same sum in the other operand order: the quartet agrees)
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_lane<0xB1>(v);
  return v + dpp_lane<0x4E>(v);
}

// Max and sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48),
// with gfx950's row-swap instructions: each returns the pair {x_l, x_l^16}
// (resp. {x_l, x_l^32}) in some order, so every lane of a quartet ends with
// the same bits. VALU only: no LDS round trip as with a lane shuffle.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// sums over aligned groups of 8 and of 16 lanes (the quartets, then the
// mirrored halves), every lane of a group with the same bits
__device__ __forceinline__ float row8_sum(float v) {
  v = quad_sum(v);
  return v + dpp_lane<0x141>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v = row8_sum(v);
  return v + dpp_lane<0x140>(v);
}

// Whole-wave sum and max: DPP steps inside each 16-lane row (the pairs at
// distance 1 and 2, then the mirrored halves of 8 and of 16 lanes), then the
// row swaps; VALU only, and every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) { return rows4_sum(row16_sum(v)); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_lane<0xB1>(v));
  v = fmaxf(v, dpp_lane<0x4E>(v));
  v = fmaxf(v, dpp_lane<0x141>(v));
  v = fmaxf(v, dpp_lane<0x140>(v));
  return rows4_max(v);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// q[start] + q[start + stride] + ... over indices below n, added in that
// order, with the loads of eight terms in flight together (a plain loop
// would wait for each load before the next one is issued)
__device__ __forceinline__ float strided_sum(const float* q, int n, int start, int stride) {
  float s = 0.f;
  for (int g0 = start; g0 < n; g0 += 8 * stride) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = g0 + u * stride;
      v[u] = q[g < n ? g : n - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + u * stride < n) s += v[u];
  }
  return s;
}

// Order-preserving key for (value, index) argmax with the lowest index
// winning ties: larger key <=> larger value, or equal value and lower index.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t k) {
  return 0xffffffffu - (uint32_t)(k & 0xffffffffu);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) {
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = umax64(v, w);
  }
  return v;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 from the Random123 paper's round function
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t row, uint64_t seq,
                                                 uint64_t purpose) {
  uint64_t c[4] = {row, seq, purpose, 0ull};
  philox4x64_10(c, seed, 0ull);
  return (double)(c[0] >> 11) * 0x1.0p-53;
}

// RoPE angle for position `pos` and pair index d of a head of size hd:
// pos * theta^(-2d/hd) radians. The rotation is formed from the frequency in
// revolutions per position (theta^(-2d/hd) / 2 pi): the angle pos * f is
// formed and reduced to [-1/2, 1/2] revolution in fp64, then the hardware
// sine and cosine, which take revolutions (max abs error ~1.2e-7 on that
// range, measured against fp64), in place of a library sincosf of the
// reduced angle.
__device__ __forceinline__ double rope_inv_freq(int d, int hd, double log2_theta) {
  return exp2(-2.0 * (double)d / (double)hd * log2_theta);
}
__device__ __forceinline__ double rope_rev_freq(int d, int hd, double log2_theta) {
  return rope_inv_freq(d, hd, log2_theta) * 0.15915494309189533577;  // 1 / (2 pi)
}
__device__ __forceinline__ void rope_cs_rev(int pos, double f_rev, float& c, float& s) {
  double r = (double)pos * f_rev;
  r -= rint(r);
  const float x = (float)r;
  s = __builtin_amdgcn_sinf(x);
  c = __builtin_amdgcn_cosf(x);
}

// One sequence of a draft call: its KV buffer and the context length.
struct SeqDesc {
  bf16_t* kv;       // base of the sequence's KV buffer
  int32_t cap;      // row capacity of each head plane
  int32_t len;      // context positions (the anchor sits at position len)
  int32_t max_ctx;  // context positions the buffer holds
};
struct SeqTable {
  SeqDesc s[kMaxSeqs];
  // device-resident rounds: the lengths live in device memory (int32 per
  // sequence) and override s[i].len
  const int32_t* len_dev;
};

// 16 bytes per lane from global memory to LDS at lds + 16 * lane (lds is
// wave-uniform): a direct load, no register staging.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
// the same with the non-temporal hint (nt): for data read exactly once, such
// as streamed weights, so that it does not displace reused lines from the
// caches
__device__ __forceinline__ void dma16_nt(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 2);
}

// 16-byte store with the system-coherent cache policy (sc0 sc1): written
// through the L2, so partial results that a later kernel reads leave no dirty
// lines behind for the write-back at the kernel's end. byte_off < 2^31.
__device__ __forceinline__ void store16_wt(float* base, uint32_t byte_off, f32x4 v) {
  // raw buffer, 32-bit elements (descriptor word 3 of this GPU family)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, 17);
}

// context length of sequence s: the host value, or the device one clamped to
// the buffer (a length past max_ctx would put the block's rows out of it)
__device__ __forceinline__ int seq_len(const SeqTable& t, int s) {
  if (!t.len_dev) return t.s[s].len;
  const int l = t.len_dev[s];
  return l < 0 ? 0 : (l > t.s[s].max_ctx ? t.s[s].max_ctx : l);
}

}  // namespace dfl
