// Internal helpers shared by the libmla HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kNope = 128;
constexpr int kRope = 64;
constexpr int kQDepth = 192;
constexpr int kV = 128;
constexpr int kLora = 512;
constexpr int kCache = 576;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// ---- bf16 ----------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

// Round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- float8 e4m3fn (OCP: bias 7, max 448, no infinities) -------------------

// Exact decode of one e4m3fn code to fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
  }
  if ((c & 0x7Fu) == 0x7Fu) mag = __uint_as_float(0x7FC00000u);
  return __uint_as_float(__float_as_uint(mag) | s);
}

// fp32 -> e4m3fn, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float f) {
  uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  float a = fminf(fabsf(f), 448.0f);
  if (!(a == a)) return sign | 0x7Fu;  // NaN
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9
    // rint rounds half to even in the default mode
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8 (8 == 2^-6, the first normal)
  } else {
    uint32_t b = __float_as_uint(a);
    // keep 3 mantissa bits: round at bit 20 (nearest even)
    b += 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t e = (b >> 23) - 120u;  // biased e4m3 exponent, >= 1
    const uint32_t m = (b >> 20) & 0x7u;
    code = (e << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// ---- wave helpers -----------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Reductions of a value with the lane 32 away (v_permlane32_swap, gfx950): the
// swap leaves lanes l < 32 holding (x[l], x[l+32]) and lanes l >= 32 holding
// (x[l-32], x[l]) in its two results, so combining them pairs every lane with
// its partner without a round trip through LDS.
__device__ __forceinline__ float max_with_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_lane32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same with the lane 16 away inside each 32-lane half
// (v_permlane16_swap, gfx950).
__device__ __forceinline__ float max_with_lane16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_lane16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mla
