// Internal interfaces between the host API (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

struct GemmLaunch {
  const uint8_t* a;
  const uint8_t* a_sf;
  const uint8_t* b;
  const uint8_t* b_sf;
  const float* alpha;
  uint16_t* d;
  float* ws;
  int64_t M, N, K;
  int64_t tiles_m, tiles_n;
  int splits;
  int group_m;
  // Scale layout of a_sf and b_sf: 0 linear [rows][K/16]; 1 and 2 the 128 x 4
  // and 8 x 4 tiled layouts, for the plans that read them in place
  // (plan_reads_tiled_scales).
  int sf_layout;
};

struct GroupedLaunch {
  const uint8_t* a;
  const uint8_t* a_sf;
  const uint8_t* b;
  const uint8_t* b_sf;
  const int32_t* offsets;
  const float* alpha;
  uint16_t* d;
  int64_t rows, N, K;
  int E;
  // Activations quantised on load (the fused variant; a and a_sf unused):
  // bf16 x[T][K], A row i = x[row_token[i]] (x[i] when row_token is NULL),
  // quantised with the encode scale *a_gs (1.0 when NULL).
  const uint16_t* x;
  const int32_t* row_token;
  const float* a_gs;
  int64_t T;
  // Scale layout of a_sf ([rows][K/16]) and b_sf (one [E * N][K/16] matrix):
  // 0 linear, 1 the 128 x 4 and 2 the 8 x 4 tiled layout (register kernels
  // only, K % 512 == 0)
  int sf_layout;
};

struct GemmPlan {
  const char* name;
  int kind;
  int64_t tiles_m, tiles_n;
  int splits;
  int group_m;
  size_t workspace;
};

// Plan families that nvfp4_force_plan can force (tuning sweeps and tests).
constexpr int kForceGemm = 0, kForceMx = 1, kForceGrouped = 2, kForceFamilies = 3;
void set_forced_plan(int family, int kind, int splits);

GemmPlan choose_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const GemmPlan& plan, GemmLaunch p, hipStream_t stream);
// Whether an NVFP4 plan reads scales in tiled layout sf_layout in place: the
// register tiles read both layouts, the automatic LDS tiles the 8 x 4 one;
// the others need linear scales.
bool plan_reads_tiled_scales(const GemmPlan& plan, int sf_layout);
// The unsplit 256x256 (plan kind 14) and 256x192 (kind 16) NVFP4 tiles, built
// in their own source with another instruction schedule; p carries the plan's
// tile counts, grid = their product.
void launch_large_tile(int kind, const GemmLaunch& p, unsigned grid, hipStream_t stream);
// MXFP4 (E8M0 scales per 32 elements): GemmLaunch with a_sf / b_sf of K/32 bytes per row.
GemmPlan choose_mx_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_mx_gemm(const GemmPlan& plan, GemmLaunch p, hipStream_t stream);
hipError_t launch_grouped(GroupedLaunch p, int32_t* status, hipStream_t stream, bool compute);
// Grouped GEMM on weights pre-packed by launch_pack_b (K % 512 == 0).
hipError_t launch_grouped_packed(GroupedLaunch p, int32_t* status, hipStream_t stream, bool compute);
// Grouped GEMM quantising its bf16 activations on load (K % 512 == 0), on
// [E][N][K/2] weights or (packed) on weights written by launch_pack_b.
hipError_t launch_grouped_fused(GroupedLaunch p, bool packed, int32_t* status, hipStream_t stream, bool compute);
size_t packed_b_bytes(int64_t N, int64_t K, int32_t E, size_t* sf_bytes);
hipError_t launch_pack_b(const uint8_t* b, const uint8_t* b_sf, int64_t N, int64_t K, int32_t E, uint8_t* pb,
                         uint8_t* psf, hipStream_t stream);
size_t grouped_workspace(int64_t rows, int64_t N, int64_t K, int32_t E);

// Scratch of nvfp4_gemm_noalloc: a fixed device array per GPU (this many
// bytes), whose address is looked up, and whose counters are cleared on
// `stream`, at the first call on each device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream);

// MoE expert FFN pieces (moe.hip): SwiGLU of a [rows][2I] bf16 gate/up
// output quantised to NVFP4 ([rows][I/2] codes, [rows][I/16] scales), and
// the weighted combine of each token's top_k expert rows of a [rows][H] bf16
// output into [T][H] bf16.
hipError_t launch_swiglu_quantize(const uint16_t* gu, int64_t rows, int64_t I, const float* gs, uint8_t* q,
                                  uint8_t* sf, hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* down, const int32_t* rows_of, const float* wt, uint16_t* out,
                              int64_t T, int64_t H, int32_t top_k, int64_t rows, hipStream_t stream);

// Scale layout interop (layout.hip): linear [rows][K/16] <-> 128 x 4 tiles.
size_t tiled128x4_bytes(int64_t rows, int64_t K);
hipError_t launch_scales_to_128x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, hipStream_t stream);
hipError_t launch_scales_from_128x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, hipStream_t stream);
// ... and the 8 x 4 tiles
size_t tiled8x4_bytes(int64_t rows, int64_t K);
hipError_t launch_scales_to_8x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, hipStream_t stream);
hipError_t launch_scales_from_8x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, hipStream_t stream);

hipError_t launch_quantize(const float* x, int64_t R, int64_t K, const float* gs, uint8_t* q, uint8_t* sf,
                           hipStream_t stream);
// bf16 rows x[row_token[i]] (x[i] if row_token is NULL) -> NVFP4 [rows][K/2], [rows][K/16].
hipError_t launch_quantize_rows_bf16(const uint16_t* x, const int32_t* row_token, int64_t rows, int64_t T,
                                    int64_t K, const float* gs, uint8_t* q, uint8_t* sf, hipStream_t stream);
hipError_t launch_global_scale(const float* x, int64_t n, float* gs, hipStream_t stream);
hipError_t launch_alpha(const float* gs_a, const float* gs_b, float* alpha, int32_t count, hipStream_t stream);

}  // namespace nvfp4
