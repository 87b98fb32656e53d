// C ABI of the NVFP4 library: host-side validation, plan choice and launch.
// Every check runs on the host before anything is enqueued, so a rejected
// call touches no device memory.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/nvfp4.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

nvfp4_status fail(nvfp4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

nvfp4_status ok() {
  g_err[0] = '\0';
  return NVFP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

nvfp4_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape rules shared by the GEMM entry points.
nvfp4_status check_k(int64_t K) {
  if (K < 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is negative", (long long)K);
  if (K % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of the block size 16", (long long)K);
  if (K % 256 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "K = %lld: the library needs K %% 256 == 0", (long long)K);
  if (K == 0) return fail(NVFP4_ERR_UNSUPPORTED, "K = 0 is not supported");
  // buffer offsets inside one 256-row operand tile stay below 2^31
  if (K > (int64_t(1) << 22))
    return fail(NVFP4_ERR_UNSUPPORTED, "K = %lld: the library needs K <= 4194304", (long long)K);
  return NVFP4_OK;
}

// nvfp4_gemm and nvfp4_gemm_noalloc: the same checks, plans and kernels; the
// second takes its split-K scratch from the library's fixed per-device array
// instead of a caller workspace.
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Whether nvfp4_gemm_sf converts the tiled scales of this plan into linear
// copies first (the plans that cannot read the layout in place).
bool converts_scales(const nvfp4::GemmPlan& plan, int32_t sf_layout) {
  return sf_layout != 0 && !nvfp4::plan_reads_tiled_scales(plan, sf_layout);
}

// Workspace of a GEMM call: the plan's own (split-K counters and partial
// tiles), then, when the scales are converted, linear copies of a_sf and b_sf.
size_t gemm_workspace(const nvfp4::GemmPlan& plan, int64_t M, int64_t N, int64_t K, int32_t sf_layout) {
  if (!converts_scales(plan, sf_layout)) return plan.workspace;
  return align256(plan.workspace) + align256((size_t)M * (size_t)(K / 16)) + align256((size_t)N * (size_t)(K / 16));
}

nvfp4_status gemm_call(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                       const float* alpha, uint16_t* d, int64_t M, int64_t N, int64_t K, void* workspace,
                       size_t workspace_bytes, void* stream, bool noalloc, int32_t sf_layout = 0) {
  const char* fn = noalloc ? "nvfp4_gemm_noalloc launch" : (sf_layout ? "nvfp4_gemm_sf launch" : "nvfp4_gemm launch");
  if (sf_layout < 0 || sf_layout > 2 || (noalloc && sf_layout != 0))
    return fail(NVFP4_ERR_SHAPE, "sf_layout = %d: 0 (linear), 1 (128 x 4) or 2 (8 x 4)", sf_layout);
  if (M < 0 || N < 0) return fail(NVFP4_ERR_SHAPE, "M = %lld, N = %lld must be >= 0", (long long)M, (long long)N);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (M == 0 || N == 0) return ok();
  if (!a || !a_sf || !b || !b_sf || !d)
    return fail(NVFP4_ERR_NULL, "a, a_sf, b, b_sf and d must be non-NULL (alpha may be NULL)");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_sf, 16) || !aligned(b_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "a, b, a_sf and b_sf must be 16-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4)) return fail(NVFP4_ERR_ALIGN, "d and alpha must be 4-byte aligned");
  if (M > (1ll << 30) || N > (1ll << 30) || K > (1ll << 30))
    return fail(NVFP4_ERR_UNSUPPORTED, "dimensions above 2^30 are not supported");
  const nvfp4::GemmPlan plan = nvfp4::choose_plan(M, N, K);
  const size_t need = gemm_workspace(plan, M, N, K, sf_layout);
  if (need > 0) {
    if (noalloc) {
      if (plan.workspace > nvfp4::kNoAllocScratchBytes)
        return fail(NVFP4_ERR_WORKSPACE, "plan %s needs %zu scratch bytes; nvfp4_gemm_noalloc holds at most %zu",
                    plan.name, plan.workspace, nvfp4::kNoAllocScratchBytes);
      hipError_t e = nvfp4::noalloc_scratch((hipStream_t)stream, &workspace);
      if (e != hipSuccess) return hip_status(e, "nvfp4_gemm_noalloc scratch set-up");
    } else {
      if (!workspace || workspace_bytes < need)
        return fail(NVFP4_ERR_WORKSPACE, "plan %s needs %zu workspace bytes, got %zu", plan.name, need,
                    workspace ? workspace_bytes : (size_t)0);
      if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
  }
  nvfp4::GemmLaunch p{a, a_sf, b, b_sf, alpha, d, (float*)workspace, M, N, K, 0, 0, 1, 1, sf_layout};
  if (converts_scales(plan, sf_layout)) {
    uint8_t* lin_a = (uint8_t*)workspace + align256(plan.workspace);
    uint8_t* lin_b = lin_a + align256((size_t)M * (size_t)(K / 16));
    hipError_t e = sf_layout == 1 ? nvfp4::launch_scales_from_128x4(a_sf, lin_a, M, K, (hipStream_t)stream)
                                  : nvfp4::launch_scales_from_8x4(a_sf, lin_a, M, K, (hipStream_t)stream);
    if (e == hipSuccess)
      e = sf_layout == 1 ? nvfp4::launch_scales_from_128x4(b_sf, lin_b, N, K, (hipStream_t)stream)
                         : nvfp4::launch_scales_from_8x4(b_sf, lin_b, N, K, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "nvfp4_gemm_sf scale conversion");
    p.a_sf = lin_a;
    p.b_sf = lin_b;
    p.sf_layout = 0;
  }
  return hip_status(nvfp4::launch_gemm(plan, p, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_err; }

nvfp4_status nvfp4_force_plan(int32_t family, int32_t kind, int32_t splits) {
  if (family < 0 || family >= nvfp4::kForceFamilies)
    return fail(NVFP4_ERR_SHAPE, "family = %d: 0 (nvfp4_gemm), 1 (nvfp4_mx_gemm) or 2 (grouped)", family);
  if (kind > 0xFFFE || splits > 16)
    return fail(NVFP4_ERR_SHAPE, "kind = %d, splits = %d out of range", kind, splits);
  nvfp4::set_forced_plan(family, kind, splits);
  return ok();
}

size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 256 || K > (int64_t(1) << 22)) return 0;
  return nvfp4::choose_plan(M, N, K).workspace;
}

const char* nvfp4_gemm_plan(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 256 || K > (int64_t(1) << 22)) return "none";
  return nvfp4::choose_plan(M, N, K).name;
}

nvfp4_status nvfp4_gemm(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                        const float* alpha, uint16_t* d, int64_t M, int64_t N, int64_t K, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return gemm_call(a, a_sf, b, b_sf, alpha, d, M, N, K, workspace, workspace_bytes, stream, false);
}

nvfp4_status nvfp4_gemm_noalloc(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                                const float* alpha, uint16_t* d, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_call(a, a_sf, b, b_sf, alpha, d, M, N, K, nullptr, 0, stream, true);
}

size_t nvfp4_gemm_sf_workspace_size(int64_t M, int64_t N, int64_t K, int32_t sf_layout) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 256 || K > (int64_t(1) << 22) || sf_layout < 0 || sf_layout > 2) return 0;
  return gemm_workspace(nvfp4::choose_plan(M, N, K), M, N, K, sf_layout);
}

nvfp4_status nvfp4_gemm_sf(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                           const float* alpha, uint16_t* d, int64_t M, int64_t N, int64_t K, int32_t sf_layout,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_call(a, a_sf, b, b_sf, alpha, d, M, N, K, workspace, workspace_bytes, stream, false, sf_layout);
}

size_t nvfp4_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 256 || K > (int64_t(1) << 22)) return 0;
  return nvfp4::choose_mx_plan(M, N, K).workspace;
}

const char* nvfp4_mx_gemm_plan(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 256 || K > (int64_t(1) << 22)) return "none";
  return nvfp4::choose_mx_plan(M, N, K).name;
}

nvfp4_status nvfp4_mx_gemm(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                           const float* alpha, uint16_t* d, int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return fail(NVFP4_ERR_SHAPE, "M = %lld, N = %lld must be >= 0", (long long)M, (long long)N);
  if (K < 0 || K % 32 != 0)
    return fail(NVFP4_ERR_SHAPE, "K = %lld is not a non-negative multiple of the MX block size 32", (long long)K);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (M == 0 || N == 0) return ok();
  if (!a || !a_sf || !b || !b_sf || !d)
    return fail(NVFP4_ERR_NULL, "a, a_sf, b, b_sf and d must be non-NULL (alpha may be NULL)");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_sf, 4) || !aligned(b_sf, 4))
    return fail(NVFP4_ERR_ALIGN, "a and b must be 16-byte aligned, a_sf and b_sf 4-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4)) return fail(NVFP4_ERR_ALIGN, "d and alpha must be 4-byte aligned");
  if (M > (1ll << 30) || N > (1ll << 30))
    return fail(NVFP4_ERR_UNSUPPORTED, "dimensions above 2^30 are not supported");
  const nvfp4::GemmPlan plan = nvfp4::choose_mx_plan(M, N, K);
  if (plan.workspace > 0) {
    if (!workspace || workspace_bytes < plan.workspace)
      return fail(NVFP4_ERR_WORKSPACE, "plan %s needs %zu workspace bytes, got %zu", plan.name, plan.workspace,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  nvfp4::GemmLaunch p{a, a_sf, b, b_sf, alpha, d, (float*)workspace, M, N, K, 0, 0, 1, 1};
  return hip_status(nvfp4::launch_mx_gemm(plan, p, (hipStream_t)stream), "nvfp4_mx_gemm launch");
}

nvfp4_status nvfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return ok();
  if (!workspace) return fail(NVFP4_ERR_NULL, "workspace must be non-NULL");
  if (!aligned(workspace, 4)) return fail(NVFP4_ERR_ALIGN, "workspace must be 4-byte aligned");
  return hip_status(nvfp4::launch_workspace_init(workspace, workspace_bytes, (hipStream_t)stream),
                    "nvfp4_workspace_init launch");
}

size_t nvfp4_grouped_workspace_size(int64_t rows, int64_t N, int64_t K, int32_t E) {
  return nvfp4::grouped_workspace(rows, N, K, E);
}

nvfp4_status nvfp4_grouped_gemm(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                                const int32_t* offsets, const float* alpha, uint16_t* d, int64_t rows, int64_t N,
                                int64_t K, int32_t E, void* workspace, size_t workspace_bytes, int32_t* status,
                                void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (rows < 0 || N < 0 || E < 0)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld, N = %lld, E = %d must be >= 0", (long long)rows, (long long)N, E);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (!offsets && E > 0) return fail(NVFP4_ERR_NULL, "offsets must be non-NULL");
  if (!aligned(offsets, 4) || !aligned(status, 4))
    return fail(NVFP4_ERR_ALIGN, "offsets and status must be 4-byte aligned");
  if (E == 0 || N == 0 || rows == 0) {
    // nothing to multiply; the offsets are still checked when status is asked for
    nvfp4::GroupedLaunch p{a, a_sf, b, b_sf, offsets, alpha, d, rows, N, K, E};
    return hip_status(nvfp4::launch_grouped(p, status, (hipStream_t)stream, false), "nvfp4_grouped_gemm status");
  }
  if (!a || !a_sf || !b || !b_sf || !d)
    return fail(NVFP4_ERR_NULL, "a, a_sf, b, b_sf and d must be non-NULL (alpha and status may be NULL)");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_sf, 16) || !aligned(b_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "a, b, a_sf and b_sf must be 16-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4)) return fail(NVFP4_ERR_ALIGN, "d and alpha must be 4-byte aligned");
  if (rows > (1ll << 30) || N > (1ll << 30) || K > (1ll << 30) || E > 65535)
    return fail(NVFP4_ERR_UNSUPPORTED, "dimensions above 2^30 (or E > 65535) are not supported");
  nvfp4::GroupedLaunch p{a, a_sf, b, b_sf, offsets, alpha, d, rows, N, K, E};
  return hip_status(nvfp4::launch_grouped(p, status, (hipStream_t)stream, true), "nvfp4_grouped_gemm launch");
}

nvfp4_status nvfp4_grouped_gemm_sf(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                                   const int32_t* offsets, const float* alpha, uint16_t* d, int64_t rows, int64_t N,
                                   int64_t K, int32_t E, int32_t sf_layout, int32_t* status, void* stream) {
  if (sf_layout < 0 || sf_layout > 2)
    return fail(NVFP4_ERR_SHAPE, "sf_layout = %d: 0 (linear), 1 (128 x 4) or 2 (8 x 4)", sf_layout);
  if (sf_layout == 0)
    return nvfp4_grouped_gemm(a, a_sf, b, b_sf, offsets, alpha, d, rows, N, K, E, nullptr, 0, status, stream);
  if (rows < 0 || N < 0 || E < 0)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld, N = %lld, E = %d must be >= 0", (long long)rows, (long long)N, E);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (K % 512 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "K = %lld: tiled scales need K %% 512 == 0", (long long)K);
  if (!offsets && E > 0) return fail(NVFP4_ERR_NULL, "offsets must be non-NULL");
  if (!aligned(offsets, 4) || !aligned(status, 4))
    return fail(NVFP4_ERR_ALIGN, "offsets and status must be 4-byte aligned");
  if (E == 0 || N == 0 || rows == 0) {
    nvfp4::GroupedLaunch p{a, a_sf, b, b_sf, offsets, alpha, d, rows, N, K, E};
    return hip_status(nvfp4::launch_grouped(p, status, (hipStream_t)stream, false), "nvfp4_grouped_gemm_sf status");
  }
  if (!a || !a_sf || !b || !b_sf || !d)
    return fail(NVFP4_ERR_NULL, "a, a_sf, b, b_sf and d must be non-NULL (alpha and status may be NULL)");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_sf, 16) || !aligned(b_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "a, b, a_sf and b_sf must be 16-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4)) return fail(NVFP4_ERR_ALIGN, "d and alpha must be 4-byte aligned");
  if (rows > (1ll << 30) || N > (1ll << 30) || K > (1ll << 30) || E > 65535 || (int64_t)E * N > (1ll << 30))
    return fail(NVFP4_ERR_UNSUPPORTED, "dimensions above 2^30 (or E > 65535) are not supported");
  nvfp4::GroupedLaunch p{a, a_sf, b, b_sf, offsets, alpha, d, rows, N, K, E};
  p.sf_layout = sf_layout;
  return hip_status(nvfp4::launch_grouped(p, status, (hipStream_t)stream, true), "nvfp4_grouped_gemm_sf launch");
}

size_t nvfp4_grouped_packed_size(int64_t N, int64_t K, int32_t E, size_t* sf_bytes) {
  if (N <= 0 || K <= 0 || E <= 0 || K % 512 || K > (int64_t(1) << 22) || N > (1ll << 30) || E > 65535) {
    if (sf_bytes) *sf_bytes = 0;
    return 0;
  }
  return nvfp4::packed_b_bytes(N, K, E, sf_bytes);
}

namespace {
static nvfp4_status check_packed_shape(int64_t N, int64_t K, int32_t E) {
  if (N < 0 || E < 0) return fail(NVFP4_ERR_SHAPE, "N = %lld, E = %d must be >= 0", (long long)N, E);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (K % 512) return fail(NVFP4_ERR_UNSUPPORTED, "K = %lld: packed weights need K %% 512 == 0", (long long)K);
  if (N > (1ll << 30) || E > 65535) return fail(NVFP4_ERR_UNSUPPORTED, "N above 2^30 or E > 65535 not supported");
  return NVFP4_OK;
}
}  // namespace

nvfp4_status nvfp4_grouped_pack_b(const uint8_t* b, const uint8_t* b_sf, int64_t N, int64_t K, int32_t E,
                                  uint8_t* packed, uint8_t* packed_sf, void* stream) {
  nvfp4_status s = check_packed_shape(N, K, E);
  if (s != NVFP4_OK) return s;
  if (N == 0 || E == 0) return ok();
  if (!b || !b_sf || !packed || !packed_sf) return fail(NVFP4_ERR_NULL, "b, b_sf, packed and packed_sf must be non-NULL");
  if (!aligned(b, 16) || !aligned(b_sf, 16) || !aligned(packed, 16) || !aligned(packed_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "b, b_sf, packed and packed_sf must be 16-byte aligned");
  return hip_status(nvfp4::launch_pack_b(b, b_sf, N, K, E, packed, packed_sf, (hipStream_t)stream),
                    "nvfp4_grouped_pack_b launch");
}

nvfp4_status nvfp4_grouped_gemm_packed(const uint8_t* a, const uint8_t* a_sf, const uint8_t* packed,
                                       const uint8_t* packed_sf, const int32_t* offsets, const float* alpha,
                                       uint16_t* d, int64_t rows, int64_t N, int64_t K, int32_t E, int32_t* status,
                                       void* stream) {
  if (rows < 0) return fail(NVFP4_ERR_SHAPE, "rows = %lld must be >= 0", (long long)rows);
  nvfp4_status s = check_packed_shape(N, K, E);
  if (s != NVFP4_OK) return s;
  if (!offsets && E > 0) return fail(NVFP4_ERR_NULL, "offsets must be non-NULL");
  if (!aligned(offsets, 4) || !aligned(status, 4))
    return fail(NVFP4_ERR_ALIGN, "offsets and status must be 4-byte aligned");
  if (E == 0 || N == 0 || rows == 0) {
    nvfp4::GroupedLaunch p{a, a_sf, packed, packed_sf, offsets, alpha, d, rows, N, K, E};
    return hip_status(nvfp4::launch_grouped_packed(p, status, (hipStream_t)stream, false),
                      "nvfp4_grouped_gemm_packed status");
  }
  if (!a || !a_sf || !packed || !packed_sf || !d)
    return fail(NVFP4_ERR_NULL, "a, a_sf, packed, packed_sf and d must be non-NULL (alpha and status may be NULL)");
  if (!aligned(a, 16) || !aligned(packed, 16) || !aligned(a_sf, 16) || !aligned(packed_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "a, packed, a_sf and packed_sf must be 16-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4)) return fail(NVFP4_ERR_ALIGN, "d and alpha must be 4-byte aligned");
  if (rows > (1ll << 30)) return fail(NVFP4_ERR_UNSUPPORTED, "rows above 2^30 are not supported");
  nvfp4::GroupedLaunch p{a, a_sf, packed, packed_sf, offsets, alpha, d, rows, N, K, E};
  return hip_status(nvfp4::launch_grouped_packed(p, status, (hipStream_t)stream, true),
                    "nvfp4_grouped_gemm_packed launch");
}

namespace {
static nvfp4_status grouped_fused(const uint16_t* x, const int32_t* row_token, const float* a_gs, const uint8_t* b,
                                  const uint8_t* b_sf, const int32_t* offsets, const float* alpha, uint16_t* d,
                                  int64_t rows, int64_t T, int64_t N, int64_t K, int32_t E, int32_t* status,
                                  void* stream, bool packed, const char* fn) {
  if (rows < 0 || T < 0 || N < 0 || E < 0)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld, T = %lld, N = %lld, E = %d must be >= 0", (long long)rows,
                (long long)T, (long long)N, E);
  nvfp4_status s = check_k(K);
  if (s != NVFP4_OK) return s;
  if (K % 512) return fail(NVFP4_ERR_UNSUPPORTED, "K = %lld: the fused grouped GEMM needs K %% 512 == 0", (long long)K);
  if (T > 0 && T * K * 2 >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_UNSUPPORTED, "T * K * 2 = %lld bytes of activations: at most 2^31 - 1 supported",
                (long long)(T * K * 2));
  if (!row_token && rows > T)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld > T = %lld with row_token NULL (row i reads token i)", (long long)rows,
                (long long)T);
  if (N > (1ll << 30) || rows > (1ll << 30) || E > 65535)
    return fail(NVFP4_ERR_UNSUPPORTED, "rows or N above 2^30 (or E > 65535) are not supported");
  if (!offsets && E > 0) return fail(NVFP4_ERR_NULL, "offsets must be non-NULL");
  if (!aligned(offsets, 4) || !aligned(status, 4) || !aligned(row_token, 4))
    return fail(NVFP4_ERR_ALIGN, "offsets, row_token and status must be 4-byte aligned");
  nvfp4::GroupedLaunch p{nullptr, nullptr, b, b_sf, offsets, alpha, d, rows, N, K, E, x, row_token, a_gs, T};
  if (E == 0 || N == 0 || rows == 0)
    return hip_status(nvfp4::launch_grouped_fused(p, packed, status, (hipStream_t)stream, false), fn);
  if (!x || !b || !b_sf || !d)
    return fail(NVFP4_ERR_NULL, "x, b, b_sf and d must be non-NULL (row_token, a_global_scale, alpha and status "
                                "may be NULL)");
  if (!aligned(x, 16) || !aligned(b, 16) || !aligned(b_sf, 16))
    return fail(NVFP4_ERR_ALIGN, "x, b and b_sf must be 16-byte aligned");
  if (!aligned(d, 4) || !aligned(alpha, 4) || !aligned(a_gs, 4))
    return fail(NVFP4_ERR_ALIGN, "d, alpha and a_global_scale must be 4-byte aligned");
  return hip_status(nvfp4::launch_grouped_fused(p, packed, status, (hipStream_t)stream, true), fn);
}
}  // namespace

nvfp4_status nvfp4_grouped_gemm_fused(const uint16_t* x, const int32_t* row_token, const float* a_global_scale,
                                      const uint8_t* b, const uint8_t* b_sf, const int32_t* offsets,
                                      const float* alpha, uint16_t* d, int64_t rows, int64_t T, int64_t N,
                                      int64_t K, int32_t E, int32_t* status, void* stream) {
  return grouped_fused(x, row_token, a_global_scale, b, b_sf, offsets, alpha, d, rows, T, N, K, E, status, stream,
                       false, "nvfp4_grouped_gemm_fused launch");
}

nvfp4_status nvfp4_grouped_gemm_packed_fused(const uint16_t* x, const int32_t* row_token,
                                             const float* a_global_scale, const uint8_t* packed,
                                             const uint8_t* packed_sf, const int32_t* offsets, const float* alpha,
                                             uint16_t* d, int64_t rows, int64_t T, int64_t N, int64_t K, int32_t E,
                                             int32_t* status, void* stream) {
  return grouped_fused(x, row_token, a_global_scale, packed, packed_sf, offsets, alpha, d, rows, T, N, K, E, status,
                       stream, true, "nvfp4_grouped_gemm_packed_fused launch");
}

nvfp4_status nvfp4_quantize_rows_bf16(const uint16_t* x, const int32_t* row_token, const float* gs, uint8_t* q,
                                      uint8_t* sf, int64_t rows, int64_t T, int64_t K, void* stream) {
  if (rows < 0 || T < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "rows, T and K must be >= 0");
  if (K % 16) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of the block size 16", (long long)K);
  if (!row_token && rows > T)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld > T = %lld with row_token NULL", (long long)rows, (long long)T);
  if (rows == 0 || K == 0) return ok();
  if ((!x && T > 0) || !q || !sf) return fail(NVFP4_ERR_NULL, "x, q and sf must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(row_token, 4) || !aligned(gs, 4))
    return fail(NVFP4_ERR_ALIGN, "x and q must be 16-byte aligned, row_token and gs 4-byte aligned");
  return hip_status(nvfp4::launch_quantize_rows_bf16(x, row_token, rows, T, K, gs, q, sf, (hipStream_t)stream),
                    "nvfp4_quantize_rows_bf16 launch");
}

nvfp4_status nvfp4_swiglu_quantize(const uint16_t* gu, int64_t rows, int64_t I, const float* gs, uint8_t* q,
                                   uint8_t* sf, void* stream) {
  if (rows < 0 || I < 0) return fail(NVFP4_ERR_SHAPE, "rows = %lld, I = %lld must be >= 0", (long long)rows, (long long)I);
  if (I % 16) return fail(NVFP4_ERR_SHAPE, "I = %lld is not a multiple of the block size 16", (long long)I);
  if (rows == 0 || I == 0) return ok();
  if (!gu || !q || !sf) return fail(NVFP4_ERR_NULL, "gu, q and sf must be non-NULL (gs may be NULL)");
  if (!aligned(gu, 16) || !aligned(q, 16) || !aligned(gs, 4))
    return fail(NVFP4_ERR_ALIGN, "gu and q must be 16-byte aligned, gs 4-byte aligned");
  return hip_status(nvfp4::launch_swiglu_quantize(gu, rows, I, gs, q, sf, (hipStream_t)stream),
                    "nvfp4_swiglu_quantize launch");
}

nvfp4_status nvfp4_moe_combine(const uint16_t* down, const int32_t* rows_of, const float* weight, uint16_t* out,
                               int64_t T, int64_t H, int32_t top_k, int64_t rows, void* stream) {
  if (T < 0 || H < 0 || top_k < 0 || rows < 0)
    return fail(NVFP4_ERR_SHAPE, "T, H, top_k and rows must be >= 0");
  if (H % 8) return fail(NVFP4_ERR_SHAPE, "H = %lld must be a multiple of 8", (long long)H);
  if (T == 0 || H == 0) return ok();
  if (!out || (top_k > 0 && (!down || !rows_of || !weight)))
    return fail(NVFP4_ERR_NULL, "down, rows_of, weight and out must be non-NULL");
  if (!aligned(down, 16) || !aligned(out, 16) || !aligned(rows_of, 4) || !aligned(weight, 4))
    return fail(NVFP4_ERR_ALIGN, "down and out must be 16-byte aligned, rows_of and weight 4-byte aligned");
  return hip_status(nvfp4::launch_moe_combine(down, rows_of, weight, out, T, H, top_k, rows, (hipStream_t)stream),
                    "nvfp4_moe_combine launch");
}

}  // extern "C"

namespace {
// nvfp4_moe_ffn workspace: gate/up output bf16 [rows][2I], h codes
// [rows][I/2], h scales [rows][I/16], down output bf16 [rows][H], each
// segment starting on a 256-byte boundary.
struct FfnWs {
  size_t gu, hq, hsf, down, aq, asf, total;
};
size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }
FfnWs ffn_ws(int64_t T, int64_t H, int64_t I, int32_t top_k) {
  const size_t rows = (size_t)T * (size_t)top_k;
  FfnWs w;
  w.gu = 0;
  w.hq = w.gu + up256(rows * (size_t)I * 4);
  w.hsf = w.hq + up256(rows * (size_t)I / 2);
  w.down = w.hsf + up256(rows * (size_t)I / 16);
  w.aq = w.down + up256(rows * (size_t)H * 2);
  w.asf = w.aq + up256(rows * (size_t)H / 2);
  w.total = w.asf + up256(rows * (size_t)H / 16);
  return w;
}
}  // namespace

extern "C" {

size_t nvfp4_moe_ffn_workspace_size(int64_t T, int64_t H, int64_t I, int32_t top_k) {
  if (T < 0 || H < 0 || I < 0 || top_k < 0) return 0;
  return ffn_ws(T, H, I, top_k).total;
}

nvfp4_status nvfp4_moe_ffn(const uint16_t* x, const float* gs_x, const int32_t* row_token, const int32_t* offsets,
                           const uint8_t* w_gu, const uint8_t* w_gu_sf, const float* alpha_gu, const float* gs_h,
                           const uint8_t* w_d, const uint8_t* w_d_sf, const float* alpha_d,
                           const int32_t* token_rows, const float* token_weight, uint16_t* out, int64_t T,
                           int64_t H, int64_t I, int32_t E, int32_t top_k, void* workspace,
                           size_t workspace_bytes, int32_t* status, void* stream) {
  if (T < 0 || H < 0 || I < 0 || E < 0 || top_k < 0)
    return fail(NVFP4_ERR_SHAPE, "T, H, I, E and top_k must be >= 0");
  if (H % 512 || I % 512 || H == 0 || I == 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "H = %lld, I = %lld: the MoE FFN needs both positive multiples of 512",
                (long long)H, (long long)I);
  if (H > (int64_t(1) << 22) || I > (int64_t(1) << 22))
    return fail(NVFP4_ERR_UNSUPPORTED, "H and I must be <= 4194304");
  if (T * H * 2 >= (int64_t(1) << 31))
    return fail(NVFP4_ERR_UNSUPPORTED, "T * H * 2 = %lld bytes of activations: at most 2^31 - 1 supported",
                (long long)(T * H * 2));
  if (E > 65535 || (int64_t)T * top_k > (1ll << 30)) return fail(NVFP4_ERR_UNSUPPORTED, "E or T * top_k too large");
  const int64_t rows = T * (int64_t)top_k;
  if (T == 0) return ok();
  if (top_k > 0 && E == 0) return fail(NVFP4_ERR_SHAPE, "top_k = %d routed rows need E >= 1 experts", top_k);
  if (!x || !row_token || !offsets || !w_gu || !w_gu_sf || !w_d || !w_d_sf || !token_rows || !token_weight || !out)
    return fail(NVFP4_ERR_NULL, "x, row_token, offsets, weights, token_rows, token_weight and out must be non-NULL "
                                "(gs_x, gs_h, alphas and status may be NULL)");
  if (!aligned(x, 16) || !aligned(w_gu, 16) || !aligned(w_gu_sf, 16) || !aligned(w_d, 16) || !aligned(w_d_sf, 16) ||
      !aligned(out, 16) || !aligned(workspace, 256))
    return fail(NVFP4_ERR_ALIGN, "x, weights and out must be 16-byte aligned, the workspace 256-byte aligned");
  if (!aligned(row_token, 4) || !aligned(offsets, 4) || !aligned(token_rows, 4) || !aligned(token_weight, 4) ||
      !aligned(alpha_gu, 4) || !aligned(alpha_d, 4) || !aligned(gs_x, 4) || !aligned(gs_h, 4) || !aligned(status, 4))
    return fail(NVFP4_ERR_ALIGN, "index, weight, scale and status arrays must be 4-byte aligned");
  const FfnWs w = ffn_ws(T, H, I, top_k);
  if (!workspace || workspace_bytes < w.total)
    return fail(NVFP4_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, w.total);
  uint8_t* ws = (uint8_t*)workspace;
  uint16_t* gu = (uint16_t*)(ws + w.gu);
  uint8_t* hq = ws + w.hq;
  uint8_t* hsf = ws + w.hsf;
  uint16_t* down = (uint16_t*)(ws + w.down);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (rows > 0 && E > 0) {
    // gate/up: the tokens gathered and quantised once into the workspace,
    // then the packed grouped GEMM (measured faster here than quantising on
    // load, which every one of an expert's 2I / 256 column tiles repeats)
    uint8_t* aq = ws + w.aq;
    uint8_t* asf = ws + w.asf;
    nvfp4::GroupedLaunch pc{nullptr, nullptr, nullptr, nullptr, offsets, nullptr, nullptr, rows, 2 * I, H, E,
                            x, row_token, gs_x, T};
    e = nvfp4::launch_grouped_fused(pc, true, status, st, false);  // offsets and tokens into status
    if (e == hipSuccess) e = nvfp4::launch_quantize_rows_bf16(x, row_token, rows, T, H, gs_x, aq, asf, st);
    if (e == hipSuccess) {
      nvfp4::GroupedLaunch p1{aq, asf, w_gu, w_gu_sf, offsets, alpha_gu, gu, rows, 2 * I, H, E};
      e = nvfp4::launch_grouped_packed(p1, nullptr, st, true);
    }
    if (e == hipSuccess) e = nvfp4::launch_swiglu_quantize(gu, rows, I, gs_h, hq, hsf, st);
    if (e == hipSuccess) {
      nvfp4::GroupedLaunch p2{hq, hsf, w_d, w_d_sf, offsets, alpha_d, down, rows, H, I, E};
      e = nvfp4::launch_grouped_packed(p2, nullptr, st, true);
    }
  }
  if (e == hipSuccess) e = nvfp4::launch_moe_combine(down, token_rows, token_weight, out, T, H, top_k, rows, st);
  return hip_status(e, "nvfp4_moe_ffn launch");
}

size_t nvfp4_scales_128x4_size(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || K % 16) return 0;
  return nvfp4::tiled128x4_bytes(rows, K);
}

nvfp4_status nvfp4_scales_to_128x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, void* stream) {
  if (rows < 0 || K < 0 || K % 16) return fail(NVFP4_ERR_SHAPE, "rows >= 0 and K >= 0 with K %% 16 == 0 required");
  if (rows == 0 || K == 0) return ok();
  if (!sf || !tiled) return fail(NVFP4_ERR_NULL, "sf and tiled must be non-NULL");
  return hip_status(nvfp4::launch_scales_to_128x4(sf, tiled, rows, K, (hipStream_t)stream),
                    "nvfp4_scales_to_128x4 launch");
}

nvfp4_status nvfp4_scales_from_128x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, void* stream) {
  if (rows < 0 || K < 0 || K % 16) return fail(NVFP4_ERR_SHAPE, "rows >= 0 and K >= 0 with K %% 16 == 0 required");
  if (rows == 0 || K == 0) return ok();
  if (!sf || !tiled) return fail(NVFP4_ERR_NULL, "sf and tiled must be non-NULL");
  return hip_status(nvfp4::launch_scales_from_128x4(tiled, sf, rows, K, (hipStream_t)stream),
                    "nvfp4_scales_from_128x4 launch");
}

size_t nvfp4_scales_8x4_size(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || K % 16) return 0;
  return nvfp4::tiled8x4_bytes(rows, K);
}

nvfp4_status nvfp4_scales_to_8x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, void* stream) {
  if (rows < 0 || K < 0 || K % 16) return fail(NVFP4_ERR_SHAPE, "rows >= 0 and K >= 0 with K %% 16 == 0 required");
  if (rows == 0 || K == 0) return ok();
  if (!sf || !tiled) return fail(NVFP4_ERR_NULL, "sf and tiled must be non-NULL");
  return hip_status(nvfp4::launch_scales_to_8x4(sf, tiled, rows, K, (hipStream_t)stream), "nvfp4_scales_to_8x4 launch");
}

nvfp4_status nvfp4_scales_from_8x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, void* stream) {
  if (rows < 0 || K < 0 || K % 16) return fail(NVFP4_ERR_SHAPE, "rows >= 0 and K >= 0 with K %% 16 == 0 required");
  if (rows == 0 || K == 0) return ok();
  if (!sf || !tiled) return fail(NVFP4_ERR_NULL, "sf and tiled must be non-NULL");
  return hip_status(nvfp4::launch_scales_from_8x4(tiled, sf, rows, K, (hipStream_t)stream),
                    "nvfp4_scales_from_8x4 launch");
}

nvfp4_status nvfp4_quantize(const float* x, int64_t R, int64_t K, const float* global_scale, uint8_t* q,
                            uint8_t* sf, void* stream) {
  if (R < 0 || K < 0) return fail(NVFP4_ERR_SHAPE, "R = %lld, K = %lld must be >= 0", (long long)R, (long long)K);
  if (K % 16 != 0) return fail(NVFP4_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
  if (R == 0 || K == 0) return ok();
  if (!x || !q || !sf) return fail(NVFP4_ERR_NULL, "x, q and sf must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(global_scale, 4))
    return fail(NVFP4_ERR_ALIGN, "x must be 16-byte aligned, q 8-byte aligned, global_scale 4-byte aligned");
  return hip_status(nvfp4::launch_quantize(x, R, K, global_scale, q, sf, (hipStream_t)stream),
                    "nvfp4_quantize launch");
}

nvfp4_status nvfp4_global_scale(const float* x, int64_t n, float* gs, void* stream) {
  if (n < 0) return fail(NVFP4_ERR_SHAPE, "n = %lld must be >= 0", (long long)n);
  if (!gs || (!x && n > 0)) return fail(NVFP4_ERR_NULL, "x and gs must be non-NULL");
  if (!aligned(x, 16) || !aligned(gs, 4)) return fail(NVFP4_ERR_ALIGN, "x must be 16-byte aligned, gs 4-byte");
  return hip_status(nvfp4::launch_global_scale(x, n, gs, (hipStream_t)stream), "nvfp4_global_scale launch");
}

nvfp4_status nvfp4_alpha_from_scales(const float* gs_a, const float* gs_b, float* alpha, int32_t count,
                                     void* stream) {
  if (count < 0) return fail(NVFP4_ERR_SHAPE, "count = %d must be >= 0", count);
  if (count == 0) return ok();
  if (!gs_a || !gs_b || !alpha) return fail(NVFP4_ERR_NULL, "gs_a, gs_b and alpha must be non-NULL");
  if (!aligned(gs_a, 4) || !aligned(gs_b, 4) || !aligned(alpha, 4))
    return fail(NVFP4_ERR_ALIGN, "gs_a, gs_b and alpha must be 4-byte aligned");
  return hip_status(nvfp4::launch_alpha(gs_a, gs_b, alpha, count, (hipStream_t)stream), "nvfp4_alpha launch");
}

}  // extern "C"
