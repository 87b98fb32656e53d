// NVFP4 quantisation and tensor-scale kernels for gfx950.
//
// The pages never quantise (their kernel test used random code bytes and
// random scale bytes: "The Moment the Zeros Disappeared: A Pivotal FP4 Kernel
// Test on Blackwell SM120", section "The Results: A Correction"); they fix the
// target format: block_size 16 ("The Art of Reading the Manual: Debugging FP4
// GEMM Kernels on Blackwell SM120", section "Assumptions and Their
// Consequences") with float8_e4m3fn block scales and two 4-bit codes per byte
// ("When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on Blackwell
// SM120", section "Input Knowledge Required", item 3).  The arithmetic below
// is fp32 with round-to-nearest-even, in this order, per 16-element block:
//   t = (amax / 6) * gs;  sf = e4m3 RNE, saturating at 448
//   r = gs / E4M3(sf) (correctly rounded; 0 when the scale is 0)
//   code = e2m1 RNE of x * r, saturating at 6, sign bit kept
// This translation unit must be built without fast-math and without fp
// contraction so that every step rounds exactly once.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

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

// fp32 y -> e2m1 code, round to nearest even, saturating at 6, sign kept.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// One thread per 4 consecutive elements; 4 consecutive lanes form a block.
__global__ __launch_bounds__(256) void k_quantize(const f4_t* __restrict__ x, int64_t n4,
                                                  const float* __restrict__ gs_p, uint16_t* __restrict__ q,
                                                  uint8_t* __restrict__ sf) {
  const float gs = gs_p ? *gs_p : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // n4 is a multiple of 4 and the stride a multiple of 64, so the 4 lanes of
  // a block are always active together.
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f4_t v = x[i];
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    const float t = (a / 6.0f) * gs;
    const uint32_t code = e4m3_encode_pos(t);
    const float sv = e4m3_value_pos(code);
    const float r = sv == 0.0f ? 0.0f : gs / sv;
    const uint32_t c0 = e2m1_encode(v[0] * r), c1 = e2m1_encode(v[1] * r);
    const uint32_t c2 = e2m1_encode(v[2] * r), c3 = e2m1_encode(v[3] * r);
    q[i] = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
    if ((i & 3) == 0) sf[i >> 2] = (uint8_t)code;
  }
}

__global__ void k_zero_word(uint32_t* w) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *w = 0u;
}

// max |x| as fp32 bits (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void k_amax(const float* __restrict__ x, int64_t n, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  float a = 0.0f;
  const f4_t* x4 = (const f4_t*)x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f4_t v = x4[i];
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    a = fmaxf(a, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(a));
}

__global__ void k_finish_scale(float* gs) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const float a = *gs;
  *gs = a > 0.0f ? 2688.0f / a : 1.0f;  // (6 * 448) / amax
}

__global__ void k_alpha(const float* __restrict__ gs_a, const float* __restrict__ gs_b, float* __restrict__ alpha,
                        int32_t count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) alpha[i] = 1.0f / (gs_a[0] * gs_b[i]);
}

hipError_t launch_quantize(const float* x, int64_t R, int64_t K, const float* gs, uint8_t* q, uint8_t* sf,
                           hipStream_t stream) {
  const int64_t n4 = R * K / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, (const f4_t*)x, n4, gs,
                     (uint16_t*)q, sf);
  return hipGetLastError();
}

hipError_t launch_global_scale(const float* x, int64_t n, float* gs, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(64), 0, stream, (uint32_t*)gs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (n > 0) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_amax, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, (uint32_t*)gs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_finish_scale, dim3(1), dim3(64), 0, stream, gs);
  return hipGetLastError();
}

hipError_t launch_alpha(const float* gs_a, const float* gs_b, float* alpha, int32_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_alpha, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, gs_a, gs_b, alpha,
                     count);
  return hipGetLastError();
}

}  // namespace nvfp4
