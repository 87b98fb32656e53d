// NVFP4 quantisation and tensor-scale kernels for gfx950.
//
// The pages never quantise (their kernel test used random code bytes and
// random scale bytes: "The Moment the Zeros Disappeared: A Pivotal FP4 Kernel
// Test on Blackwell SM120", section "The Results: A Correction"); they fix the
// target format: block_size 16 ("The Art of Reading the Manual: Debugging FP4
// GEMM Kernels on Blackwell SM120", section "Assumptions and Their
// Consequences") with float8_e4m3fn block scales and two 4-bit codes per byte
// ("When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on Blackwell
// SM120", section "Input Knowledge Required", item 3).  The arithmetic
// (quantize_block16 in device.h, shared with the kernels that quantise on
// load) is fp32 with round-to-nearest-even, in this order, per 16-element
// block:
//   t = (amax / 6) * gs;  sf = e4m3 RNE, saturating at 448
//   r = gs / E4M3(sf) (correctly rounded; 0 when the scale is 0)
//   code = e2m1 RNE of x * r, saturating at 6, sign bit kept
// This translation unit must be built without fast-math and without fp
// contraction so that every step rounds exactly once.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

// One thread per 16-element block (4 loads of 16 bytes, 8 code bytes and one
// scale byte out); the block's scale is computed once.  Each thread handles
// kQB blocks, one grid width apart, with all their loads issued first.
constexpr int kQB = 2;

__global__ __launch_bounds__(256) void k_quantize(const f4_t* __restrict__ x, int64_t nb,
                                                  const float* __restrict__ gs_p, u2_t* __restrict__ q,
                                                  uint8_t* __restrict__ sf) {
  const float gs = gs_p ? *gs_p : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b0 < nb; b0 += kQB * stride) {
    f4_t v[kQB][4];
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const int64_t b = b0 + j * stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[j][c] = b < nb ? x[4 * b + c] : f4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const int64_t b = b0 + j * stride;
      uint32_t w[2];
      const uint32_t code = quantize_block16(v[j], gs, w);
      if (b < nb) {
        q[b] = u2_t{w[0], w[1]};
        sf[b] = (uint8_t)code;
      }
    }
  }
}

// Rows gathered from bf16 activations and quantised: row i of (q, sf) is
// the quantisation of x[row_token[i]] (x[i] when row_token is NULL; a token
// outside [0, T) gives a zero row).  One thread per 16-element block; bf16
// values are exact fp32 values, so the codes are those k_quantize gives the
// fp32 copy of the gathered rows.
__global__ __launch_bounds__(256) void k_quantize_rows_bf16(const u4_t* __restrict__ x, const int32_t* __restrict__ tok,
                                                            int64_t rows, int64_t T, int64_t K,
                                                            const float* __restrict__ gs_p, u2_t* __restrict__ q,
                                                            uint8_t* __restrict__ sf) {
  const int64_t kb = K / 16;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows * kb) return;
  const float gs = gs_p ? *gs_p : 1.0f;
  const int64_t i = b / kb, j = b % kb;
  const int64_t t = tok ? (int64_t)tok[i] : i;
  f4_t v[4] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f},
               f4_t{0.f, 0.f, 0.f, 0.f}};
  if (t >= 0 && t < T) {
    const u4_t* src = x + t * (K / 8) + 2 * j;
    bf16x8_to_f32(src[0], v[0], v[1]);
    bf16x8_to_f32(src[1], v[2], v[3]);
  }
  uint32_t w[2];
  const uint32_t code = quantize_block16(v, gs, w);
  q[b] = u2_t{w[0], w[1]};
  sf[b] = (uint8_t)code;
}

__global__ void k_zero_word(uint32_t* w) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *w = 0u;
}

// max |x| as fp32 bits (non-negative floats order like their bit patterns).
// Reduced per wave, then per work-group through LDS: one atomic per
// work-group (atomics on one word serialise in L2).
__global__ __launch_bounds__(256) void k_amax(const float* __restrict__ x, int64_t n, uint32_t* __restrict__ out) {
  __shared__ float wmax[4];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  float a = 0.0f;
  const f4_t* x4 = (const f4_t*)x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {  // four 1 KB loads in flight per wave
    const f4_t v0 = x4[i], v1 = x4[i + stride], v2 = x4[i + 2 * stride], v3 = x4[i + 3 * stride];
    const f4_t m = {fmaxf(fmaxf(fabsf(v0[0]), fabsf(v1[0])), fmaxf(fabsf(v2[0]), fabsf(v3[0]))),
                    fmaxf(fmaxf(fabsf(v0[1]), fabsf(v1[1])), fmaxf(fabsf(v2[1]), fabsf(v3[1]))),
                    fmaxf(fmaxf(fabsf(v0[2]), fabsf(v1[2])), fmaxf(fabsf(v2[2]), fabsf(v3[2]))),
                    fmaxf(fmaxf(fabsf(v0[3]), fabsf(v1[3])), fmaxf(fabsf(v2[3]), fabsf(v3[3])))};
    a = fmaxf(a, fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])));
  }
  for (; i < n4; i += stride) {
    const f4_t v = x4[i];
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  for (int64_t j = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    a = fmaxf(a, fabsf(x[j]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(out, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
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
  const int64_t nb = R * K / 16;
  if (nb == 0) return hipSuccess;
  // about 8 work-groups (32 waves) per CU
  int64_t blocks = (nb + 256 * kQB - 1) / (256 * kQB);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, (const f4_t*)x, nb, gs, (u2_t*)q,
                     sf);
  return hipGetLastError();
}

hipError_t launch_quantize_rows_bf16(const uint16_t* x, const int32_t* row_token, int64_t rows, int64_t T,
                                    int64_t K, const float* gs, uint8_t* q, uint8_t* sf, hipStream_t stream) {
  const int64_t nb = rows * (K / 16);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_rows_bf16, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream,
                     (const u4_t*)x, row_token, rows, T, K, gs, (u2_t*)q, sf);
  return hipGetLastError();
}

hipError_t launch_global_scale(const float* x, int64_t n, float* gs, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(64), 0, stream, (uint32_t*)gs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (n > 0) {
    int64_t blocks = (n / 4 + 1023) / 1024;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
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
