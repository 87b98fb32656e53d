// Host-layer driver for the AddressSanitizer / UndefinedBehaviorSanitizer build
// of the C ABI (tests/test_abi_sanitized.py compiles api.hip, gemm.hip,
// layout.hip, moe.hip and quantize.hip host-only with the sanitizers and links
// this file).  No GPU is touched: every call below is either a query or a call
// the host-side validation rejects before anything is enqueued.  It walks the
// plan choice over a grid of shapes (every plan kind forced in turn, every
// split count) and every entry point's error paths, checking the documented
// status codes; a sanitizer report aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nvfp4.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, nvfp4_last_error());
    g_fail = 1;
  }
}

int main() {
  // an aligned non-NULL address that is never dereferenced (every call using it is rejected on the host)
  uint8_t* F = (uint8_t*)(uintptr_t)0x10000;
  uint16_t* D = (uint16_t*)F;
  const int64_t Ms[] = {1, 15, 16, 17, 31, 64, 100, 128, 300, 512, 1000, 1024, 4096, 8192, 16384, 1 << 20};
  const int64_t Ns[] = {1, 16, 17, 256, 330, 768, 2048, 6144, 1 << 20};
  const int64_t Ks[] = {256, 512, 768, 1536, 6144, 1 << 16, 1 << 22};
  // plan queries over the grid, the library's own choice and every forced kind and split count
  for (int fam = 0; fam < 2; ++fam) {
    for (int kind = -1; kind < 24; ++kind) {
      for (int splits = 0; splits <= 16; splits += 3) {
        expect(nvfp4_force_plan(fam, kind, splits), NVFP4_OK, "force_plan");
        for (int64_t M : Ms)
          for (int64_t N : Ns)
            for (int64_t K : Ks) {
              size_t ws = fam ? nvfp4_mx_gemm_workspace_size(M, N, K) : nvfp4_gemm_workspace_size(M, N, K);
              const char* name = fam ? nvfp4_mx_gemm_plan(M, N, K) : nvfp4_gemm_plan(M, N, K);
              if (!name || !name[0]) {
                fprintf(stderr, "FAIL empty plan name\n");
                g_fail = 1;
              }
              // a plan that needs a workspace rejects a call without one, before any launch
              if (ws > 0) {
                int st = fam ? nvfp4_mx_gemm(F, F, F, F, NULL, D, M, N, K, NULL, 0, NULL)
                             : nvfp4_gemm(F, F, F, F, NULL, D, M, N, K, NULL, 0, NULL);
                expect(st, NVFP4_ERR_WORKSPACE, "gemm without workspace");
                if (!fam && ws > (size_t(16) << 20))
                  expect(nvfp4_gemm_noalloc(F, F, F, F, NULL, D, M, N, K, NULL), NVFP4_ERR_WORKSPACE,
                         "noalloc beyond its scratch");
              }
            }
      }
    }
    expect(nvfp4_force_plan(fam, -1, 0), NVFP4_OK, "force_plan reset");
  }
  expect(nvfp4_force_plan(2, 3, 0), NVFP4_OK, "force grouped");
  expect(nvfp4_force_plan(2, -1, 0), NVFP4_OK, "reset grouped");
  expect(nvfp4_force_plan(3, 0, 0), NVFP4_ERR_SHAPE, "force_plan family");
  expect(nvfp4_force_plan(0, 0, 17), NVFP4_ERR_SHAPE, "force_plan splits");
  // degenerate and sizes beyond the supported range
  expect(nvfp4_gemm_workspace_size(0, 16, 256) == 0 && nvfp4_gemm_workspace_size(16, 16, 40) == 0, 1, "sizes");
  expect(strcmp(nvfp4_gemm_plan(16, 16, 100), "none") == 0, 1, "plan none");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, INT64_MAX, 16, 256, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED, "huge M");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, 16, INT64_MAX, 256, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED, "huge N");
  // single GEMM error paths (nvfp4_gemm, nvfp4_gemm_noalloc, nvfp4_mx_gemm)
  expect(nvfp4_gemm(F, F, F, F, NULL, D, 16, 16, 40, NULL, 0, NULL), NVFP4_ERR_SHAPE, "K % 16");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, 16, 16, 128, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED, "K % 256");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, 16, 16, 0, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED, "K = 0");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, 16, 16, INT64_MAX & ~int64_t(255), NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED,
         "K huge");
  expect(nvfp4_gemm(F, F, F, F, NULL, D, -1, 16, 256, NULL, 0, NULL), NVFP4_ERR_SHAPE, "M < 0");
  expect(nvfp4_gemm(NULL, F, F, F, NULL, D, 16, 16, 256, NULL, 0, NULL), NVFP4_ERR_NULL, "a NULL");
  expect(nvfp4_gemm(F + 8, F, F, F, NULL, D, 16, 16, 256, NULL, 0, NULL), NVFP4_ERR_ALIGN, "a align");
  expect(nvfp4_gemm(F, F, F, F, NULL, D + 1, 16, 16, 256, NULL, 0, NULL), NVFP4_ERR_ALIGN, "d align");
  expect(nvfp4_gemm(NULL, NULL, NULL, NULL, NULL, NULL, 0, 16, 256, NULL, 0, NULL), NVFP4_OK, "M = 0");
  expect(nvfp4_gemm_noalloc(NULL, F, F, F, NULL, D, 16, 16, 256, NULL), NVFP4_ERR_NULL, "noalloc a NULL");
  expect(nvfp4_gemm_noalloc(F, F, F, F, NULL, D, 16, 16, 40, NULL), NVFP4_ERR_SHAPE, "noalloc K");
  expect(nvfp4_mx_gemm(F, F, F, F, NULL, D, 16, 16, 48, NULL, 0, NULL), NVFP4_ERR_SHAPE, "mx K % 32");
  expect(nvfp4_mx_gemm(F, F + 2, F, F, NULL, D, 16, 16, 256, NULL, 0, NULL), NVFP4_ERR_ALIGN, "mx a_sf align");
  expect(nvfp4_workspace_init(NULL, 64, NULL), NVFP4_ERR_NULL, "workspace_init NULL");
  // grouped GEMMs
  int32_t* O = (int32_t*)F;
  expect(nvfp4_grouped_gemm(F, F, F, F, O, NULL, D, 64, 64, 24, 4, NULL, 0, NULL, NULL), NVFP4_ERR_SHAPE,
         "grouped K");
  expect(nvfp4_grouped_gemm(F, F, F, F, NULL, NULL, D, 64, 64, 256, 4, NULL, 0, NULL, NULL), NVFP4_ERR_NULL,
         "grouped offsets");
  expect(nvfp4_grouped_gemm(F, F, F, F, O, NULL, D, 64, 64, 256, 70000, NULL, 0, NULL, NULL), NVFP4_ERR_UNSUPPORTED,
         "grouped E");
  expect(nvfp4_grouped_gemm(F, F, F, F, O, NULL, D, -5, 64, 256, 4, NULL, 0, NULL, NULL), NVFP4_ERR_SHAPE,
         "grouped rows");
  size_t sfb = 7;
  expect(nvfp4_grouped_packed_size(2048, 6144, 256, &sfb) > 0 && sfb > 0, 1, "packed size");
  expect(nvfp4_grouped_packed_size(2048, 768, 256, &sfb) == 0 && sfb == 0, 1, "packed size K % 512");
  expect(nvfp4_grouped_packed_size(int64_t(1) << 40, 6144, 256, &sfb) == 0, 1, "packed size huge");
  expect(nvfp4_grouped_pack_b(NULL, F, 256, 512, 2, F, F, NULL), NVFP4_ERR_NULL, "pack NULL");
  expect(nvfp4_grouped_pack_b(F, F, 256, 768, 2, F, F, NULL), NVFP4_ERR_UNSUPPORTED, "pack K");
  expect(nvfp4_grouped_gemm_packed(F, F, F, F, O, NULL, D, 64, 256, 768, 2, NULL, NULL), NVFP4_ERR_UNSUPPORTED,
         "packed K");
  uint16_t* X = (uint16_t*)F;
  expect(nvfp4_grouped_gemm_fused(X, O, NULL, F, F, O, NULL, D, 64, 8, 256, 768, 2, NULL, NULL),
         NVFP4_ERR_UNSUPPORTED, "fused K % 512");
  expect(nvfp4_grouped_gemm_fused(X, NULL, NULL, F, F, O, NULL, D, 64, 8, 256, 512, 2, NULL, NULL), NVFP4_ERR_SHAPE,
         "fused rows > T");
  expect(nvfp4_grouped_gemm_packed_fused(X, O, NULL, F, F, O, NULL, D, 64, int64_t(1) << 30, 256, 512, 2, NULL,
                                         NULL),
         NVFP4_ERR_UNSUPPORTED, "fused T * K");
  // MoE FFN and its pieces
  expect(nvfp4_moe_ffn(X, NULL, O, O, F, F, NULL, NULL, F, F, NULL, O, (float*)F, X, 4, 500, 512, 2, 2, F, 0, NULL,
                       NULL),
         NVFP4_ERR_UNSUPPORTED, "ffn H");
  expect(nvfp4_moe_ffn(X, NULL, O, O, F, F, NULL, NULL, F, F, NULL, O, (float*)F, X, 4, 512, 512, 2, 2, F, 16, NULL,
                       NULL),
         NVFP4_ERR_WORKSPACE, "ffn workspace");
  expect(nvfp4_moe_ffn_workspace_size(512, 6144, 2048, 8) > 0 && nvfp4_moe_ffn_workspace_size(-1, 1, 1, 1) == 0, 1,
         "ffn ws size");
  expect(nvfp4_swiglu_quantize(X, 4, 40, NULL, F, F, NULL), NVFP4_ERR_SHAPE, "swiglu I");
  expect(nvfp4_moe_combine(X, O, (float*)F, X, 4, 12, 2, 8, NULL), NVFP4_ERR_SHAPE, "combine H");
  expect(nvfp4_quantize_rows_bf16(X, NULL, NULL, F, F, 9, 8, 64, NULL), NVFP4_ERR_SHAPE, "rows bf16");
  // quantiser, scales, layouts
  expect(nvfp4_quantize((float*)F, 4, 40, NULL, F, F, NULL), NVFP4_ERR_SHAPE, "quantize K");
  expect(nvfp4_quantize((float*)(F + 4), 4, 64, NULL, F, F, NULL), NVFP4_ERR_ALIGN, "quantize align");
  expect(nvfp4_global_scale(NULL, 10, (float*)F, NULL), NVFP4_ERR_NULL, "global scale NULL");
  expect(nvfp4_alpha_from_scales((float*)F, (float*)F, NULL, 4, NULL), NVFP4_ERR_NULL, "alpha NULL");
  const int64_t Rs[] = {0, 1, 9, 130, int64_t(1) << 20}, Ts[] = {16, 80, 6144};
  for (int64_t rows : Rs)
    for (int64_t K : Ts) {
      if (nvfp4_scales_128x4_size(rows, K) < (size_t)(rows * (K / 16)) ||
          nvfp4_scales_8x4_size(rows, K) < (size_t)(rows * (K / 16))) {
        fprintf(stderr, "FAIL tiled size %lld %lld\n", (long long)rows, (long long)K);
        g_fail = 1;
      }
    }
  expect(nvfp4_scales_to_128x4(F, F, 4, 40, NULL), NVFP4_ERR_SHAPE, "128x4 K");
  expect(nvfp4_scales_from_8x4(NULL, F, 4, 64, NULL), NVFP4_ERR_NULL, "8x4 NULL");
  if (!g_fail) printf("abi sanitize: all host checks passed\n");
  return g_fail;
}
