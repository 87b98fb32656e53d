// Device-side helpers shared by the NVFP4 kernels (gfx950 only).
//
// Element and scale formats: two e2m1 codes per byte (element 2j in the low
// nibble) and one e4m3fn byte per 16-element block; pages "When a Benchmark
// Crashes: The Elusive FP4 GEMM Comparison on Blackwell SM120", section
// "Input Knowledge Required", item 3, and "The Art of Reading the Manual",
// section "The Message" (block_size=16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// Two e2m1 codes (byte SEL of w) -> two f16 values.  The hardware conversion
// applies only the exponent of its fp32 scale, so with scale 1.0 it is the
// exact code-to-value map (every e2m1 value is an f16 value).
template <int SEL>
__device__ __forceinline__ h2_t fp4x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two e4m3fn bytes (bits 0-15 of w) -> two f16 values, exact: every finite
// e4m3fn value (subnormals included) is a normal f16 value; 0x7F/0xFF give
// NaN.
__device__ __forceinline__ h2_t e4m3x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// Dequantise the 8 codes of one dword (elements 8t..8t+7 of a lane's chunk)
// with block scale pair s = (scale, scale): the MFMA operand, exact in f16
// (a code times a scale needs at most 6 significant bits and lies in
// [2^-10, 2688] when non-zero).
__device__ __forceinline__ h8_t dequant8(uint32_t w, h2_t s) {
  h2_t p0 = fp4x2_to_h2<0>(w) * s;
  h2_t p1 = fp4x2_to_h2<1>(w) * s;
  h2_t p2 = fp4x2_to_h2<2>(w) * s;
  h2_t p3 = fp4x2_to_h2<3>(w) * s;
  h8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Quantiser steps shared by the quantise kernel and the grouped GEMM that
// quantises its activations on load.  Every file that includes this header
// is built without fast-math and without fp contraction, so each step
// rounds exactly once.
// fp32 t (finite, >= 0) -> e4m3fn code, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float t) {
  t = fminf(t, 448.0f);
  if (t < 0.015625f) {
    // subnormal range: grid 2^-9; a result of 8 is code 0x08 = 2^-6
    return (uint32_t)__builtin_rintf(t * 512.0f);
  }
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  return (u >> 20) - 960u;           // rebias exponent 127 -> 7 (120 * 8 = 960)
}

// e4m3fn code in [0x00, 0x7E] -> its fp32 value (exact).
__device__ __forceinline__ float e4m3_value_pos(uint32_t code) {
  const int e = (int)(code >> 3), m = (int)(code & 7u);
  return e ? __builtin_ldexpf((float)(8 + m), e - 10) : __builtin_ldexpf((float)m, -9);
}

// Codes of 8 consecutive scaled elements, 2 per byte (element 2j in the low
// nibble of byte j).  The hardware f32 -> e2m1 conversion (scale 1.0: no
// extra scaling) rounds to nearest even, saturates at +-6 and keeps the sign
// of values that round to zero.
__device__ __forceinline__ uint32_t e2m1x8(f4_t lo, f4_t hi, float r) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo[0] * r, lo[1] * r, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo[2] * r, lo[3] * r, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hi[0] * r, hi[1] * r, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hi[2] * r, hi[3] * r, 1.0f, 3);
  return w;
}

// Quantise one 16-element block (v[0..3] hold elements 0..15 in fp32) with
// encode scale gs, in this order, each step rounding once:
//   t = (amax / 6) * gs;  sf = e4m3 RNE, saturating;  r = gs / E4M3(sf) (0 if
//   the scale is 0);  codes = e2m1 RNE of x * r.
// Returns the scale code; w[0] holds the codes of elements 0..7, w[1] those
// of elements 8..15.
__device__ __forceinline__ uint32_t quantize_block16(const f4_t (&v)[4], float gs, uint32_t (&w)[2]) {
  float a = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v[c][0]), fabsf(v[c][1])), fmaxf(fabsf(v[c][2]), fabsf(v[c][3]))));
  const float t = (a / 6.0f) * gs;
  const uint32_t code = e4m3_encode_pos(t);
  const float sv = e4m3_value_pos(code);
  const float r = sv == 0.0f ? 0.0f : gs / sv;
  w[0] = e2m1x8(v[0], v[1], r);
  w[1] = e2m1x8(v[2], v[3], r);
  return code;
}

// The same steps for a block whose 16 elements are split over the lane pair
// (l, l ^ 1): this lane holds 8 of them (lo, hi).  The block amax is the max
// over the pair (one DPP swap), so both lanes compute the same scale; w gets
// the codes of this lane's 8 elements.
__device__ __forceinline__ uint32_t quantize_half_block16(f4_t lo, f4_t hi, float gs, uint32_t& w) {
  float a = fmaxf(fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])), fmaxf(fabsf(lo[2]), fabsf(lo[3]))),
                  fmaxf(fmaxf(fabsf(hi[0]), fabsf(hi[1])), fmaxf(fabsf(hi[2]), fabsf(hi[3]))));
  // quad_perm [1, 0, 3, 2]: the value of lane l ^ 1
  a = fmaxf(a, __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(a), 0xB1, 0xF, 0xF, false)));
  const float t = (a / 6.0f) * gs;
  const uint32_t code = e4m3_encode_pos(t);
  const float sv = e4m3_value_pos(code);
  const float r = sv == 0.0f ? 0.0f : gs / sv;
  w = e2m1x8(lo, hi, r);
  return code;
}

// Eight bf16 values (one 16-byte chunk, element 2i in the low half of word i)
// -> two f4 of their exact fp32 values.
__device__ __forceinline__ void bf16x8_to_f32(u4_t c, f4_t& lo, f4_t& hi) {
  lo = f4_t{__uint_as_float(c[0] << 16), __uint_as_float(c[0] & 0xFFFF0000u), __uint_as_float(c[1] << 16),
            __uint_as_float(c[1] & 0xFFFF0000u)};
  hi = f4_t{__uint_as_float(c[2] << 16), __uint_as_float(c[2] & 0xFFFF0000u), __uint_as_float(c[3] << 16),
            __uint_as_float(c[3] & 0xFFFF0000u)};
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  bf2_t v = {(__bf16)lo, (__bf16)hi};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

}  // namespace nvfp4
