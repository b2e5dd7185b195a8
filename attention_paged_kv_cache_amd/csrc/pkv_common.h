// Device-side helpers shared by the paged-KV kernels (gfx950 / CDNA4 only).
//
// Vector types are the operand types of the MFMA builtins; small helpers
// convert and pack elements. Nothing here knows about pages or attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element tags: storage type of one element and the MFMA family it feeds.
struct F16Tag {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct BF16Tag {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct E4M3Tag {
  using storage = uint8_t;
  static constexpr int bytes = 1;
};

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 ld8(const void *p) {
  return *reinterpret_cast<const u32x2 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}
__device__ __forceinline__ void st8(void *p, u32x2 v) {
  *reinterpret_cast<u32x2 *>(p) = v;
}

// Two fp32 -> packed pair of 16-bit floats (round to nearest even).
__device__ __forceinline__ uint32_t pack2(float a, float b, BF16Tag) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack2(float a, float b, F16Tag) {
  _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// fp32 -> e4m3fn code (low 8 bits): nearest value, ties to the even
// mantissa; magnitudes above 448 saturate to +-448 (the format has no
// infinity); NaN gives the NaN code of its sign. Written out in integer
// arithmetic so the rounding is exactly this rule.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return sign | 0x7Fu;
  if (a > 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes m * 2^-9, m = 0..8
    return sign | (uint32_t)rintf(a * 512.0f);  // exact scaling, rint is RNE
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;  // -6 .. 8
  uint32_t keep = (u >> 20) & 0x7u;        // top 3 mantissa bits
  const uint32_t rest = u & 0xFFFFFu;      // the 20 bits rounded away
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}

// Four e4m3fn codes (one dword) -> four bf16 (two dwords). Exact: every
// e4m3fn value is representable in bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 16-bit lane of a packed dword pair: byte-select masks for v_perm_b32.
// perm(hi, lo, sel) picks bytes of {hi:lo}; lo bytes are 0..3, hi 4..7.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  // {b.lo16 : a.lo16}
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  // {b.hi16 : a.hi16}
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Transpose an 8x8 block of 16-bit elements held by one lane.
// in[r] holds row r (8 elements, element c in dword c/2, half c%2).
// out[c] holds column c: element r of column c = in[r] element c.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      const uint32_t a = in[2 * rp][w], b = in[2 * rp + 1][w];
      out[c][rp] = (c & 1) ? pack_hi16(a, b) : pack_lo16(a, b);
    }
  }
}

// Combine a value across the two 32-lane halves of a wave (lane l with lane
// l ^ 32) with v_permlane32_swap, which swaps the high half of its first
// operand with the low half of its second. Given two copies of x, the two
// results hold x's low half twice and x's high half twice; no LDS traffic.
// (The vector elements are copied to scalars before the bit casts: a bit
// cast applied to a subscripted vector element has been seen to read
// element 0.)
__device__ __forceinline__ void halves_of(float x, float &lo, float &hi) {
  const uint32_t a = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float wave_max_xor32(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float wave_sum_xor32(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return lo + hi;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace pkv
