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
