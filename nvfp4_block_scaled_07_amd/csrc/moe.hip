// The MoE expert FFN around the grouped NVFP4 GEMM: the SwiGLU activation
// quantised to NVFP4 between the gate/up and down GEMMs, and the weighted
// combine of each token's expert rows.  The pages run these FFNs through a
// fused MoE kernel (cutlass_moe) on 256 experts with 8 active per token,
// hidden size 6144 and expert intermediate size 2048 ("When a Benchmark
// Crashes: The Elusive FP4 GEMM Comparison on Blackwell SM120", sections "Why
// This Message Was Written" and "The Thinking Process Visible in Reasoning
// Parts"); the activation is not named there: it is read as SwiGLU,
// h = silu(gate) * up with silu(g) = g / (1 + exp(-g)), gate and up being the
// first and second halves of the gate/up GEMM's output columns.
//
// Built, like the other kernel files, without fast-math and without fp
// contraction: every fp32 step rounds once.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

// One thread per 16-element block of h (row r, columns 16 j .. 16 j + 15):
// gate and up are read as bf16 (two 16-byte chunks each), h is formed in
// fp32 and quantised with the encode scale *gs_p by the quantiser's steps.
__global__ __launch_bounds__(256) void k_swiglu_quantize(const u4_t* __restrict__ gu, int64_t rows, int64_t I,
                                                         const float* __restrict__ gs_p, u2_t* __restrict__ q,
                                                         uint8_t* __restrict__ sf) {
  const int64_t nb = rows * (I / 16);
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const float gs = gs_p ? *gs_p : 1.0f;
  const int64_t r = b / (I / 16), j = b % (I / 16);
  // 16-byte chunks of one row of gate/up: 2 I bf16 = I / 4 chunks
  const u4_t* row = gu + r * (I / 4);
  const u4_t g0 = row[2 * j], g1 = row[2 * j + 1];
  const u4_t u0 = row[I / 8 + 2 * j], u1 = row[I / 8 + 2 * j + 1];
  f4_t g[4], u[4], h[4];
  bf16x8_to_f32(g0, g[0], g[1]);
  bf16x8_to_f32(g1, g[2], g[3]);
  bf16x8_to_f32(u0, u[0], u[1]);
  bf16x8_to_f32(u1, u[2], u[3]);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = g[c][e];
      const float s = x / (1.0f + expf(-x));
      h[c][e] = s * u[c][e];
    }
  uint32_t w[2];
  const uint32_t code = quantize_block16(h, gs, w);
  q[b] = u2_t{w[0], w[1]};
  sf[b] = (uint8_t)code;
}

// out[t][c .. c + 7] = bf16( sum_j w[t][j] * down[rows_of[t][j]][c .. c + 7] ),
// summed in fp32 in j order (one multiply and one add per term, each rounded
// once); a row index outside [0, rows) contributes nothing.  One thread per
// 8 output columns of one token.  The token's rows are taken kCB at a time:
// all their indices, then all their row loads, are issued before the sums,
// so a thread waits for two memory round trips per kCB rows, not two per row.
constexpr int kCB = 8;

__global__ __launch_bounds__(256) void k_moe_combine(const u4_t* __restrict__ down, const int32_t* __restrict__ rows_of,
                                                     const float* __restrict__ wt, u4_t* __restrict__ out, int64_t T,
                                                     int64_t H, int32_t top_k, int64_t rows) {
  const int64_t n8 = T * (H / 8);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int64_t t = i / (H / 8), c8 = i % (H / 8);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int j0 = 0; j0 < top_k; j0 += kCB) {
    int32_t r[kCB];
    float w[kCB];
    bool ok[kCB];
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
      const bool in = j0 + j < top_k;
      r[j] = in ? rows_of[t * top_k + j0 + j] : -1;
      w[j] = in ? wt[t * top_k + j0 + j] : 0.0f;
    }
    u4_t v[kCB];
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
      ok[j] = r[j] >= 0 && r[j] < rows;
      v[j] = ok[j] ? down[(int64_t)r[j] * (H / 8) + c8] : u4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
      if (!ok[j]) continue;
      f4_t lo, hi;
      bf16x8_to_f32(v[j], lo, hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w[j] * lo[e];
        acc[4 + e] += w[j] * hi[e];
      }
    }
  }
  out[i] = u4_t{f32x2_to_bf16x2_bits(acc[0], acc[1]), f32x2_to_bf16x2_bits(acc[2], acc[3]),
                f32x2_to_bf16x2_bits(acc[4], acc[5]), f32x2_to_bf16x2_bits(acc[6], acc[7])};
}

hipError_t launch_swiglu_quantize(const uint16_t* gu, int64_t rows, int64_t I, const float* gs, uint8_t* q,
                                  uint8_t* sf, hipStream_t stream) {
  const int64_t nb = rows * (I / 16);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_quantize, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, (const u4_t*)gu,
                     rows, I, gs, (u2_t*)q, sf);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* down, const int32_t* rows_of, const float* wt, uint16_t* out,
                              int64_t T, int64_t H, int32_t top_k, int64_t rows, hipStream_t stream) {
  const int64_t n8 = T * (H / 8);
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, (const u4_t*)down,
                     rows_of, wt, (u4_t*)out, T, H, top_k, rows);
  return hipGetLastError();
}

}  // namespace nvfp4
