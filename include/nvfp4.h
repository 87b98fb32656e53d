/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled GEMM library.
 *
 * The operation is the FP4 GEMM debugged and benchmarked on the pages
 * "The Art of Reading the Manual: Debugging FP4 GEMM Kernels on Blackwell
 * SM120" (section "The Message": mm_fp4(a, b, a_descale, b_descale, alpha,
 * out_dtype=bfloat16, out, block_size=16, ...)), "The Moment the Zeros
 * Disappeared: A Pivotal FP4 Kernel Test on Blackwell SM120" (section "The
 * Subject Message: A Corrected Test": scalar alpha, caller-allocated out, b as
 * the column-major K x N operand, scales as uint8 bytes viewed as
 * float8_e4m3fn) and "When a Benchmark Crashes: The Elusive FP4 GEMM
 * Comparison on Blackwell SM120" (section "Input Knowledge Required", items 3
 * and 4: two 4-bit floats per uint8, float8_e4m3fn block scales, dequantise on
 * the fly and accumulate in higher precision):
 *
 *   D[m][n] = bf16_rne( alpha * sum_k xA[m][k] * xB[n][k] )
 *   xA[m][k] = E2M1(code of element k of row m of A) * E4M3(a_sf[m][k/16])
 *   xB[n][k] = E2M1(code of element k of row n of B) * E4M3(b_sf[n][k/16])
 *
 * Layouts (all row-major, no padding between rows):
 *   A     uint8 [M][K/2]   two e2m1 codes per byte, element 2j in bits 0-3
 *                          and element 2j+1 in bits 4-7 of byte j
 *   a_sf  uint8 [M][K/16]  raw e4m3fn bytes, one per 16-element K block
 *   B     uint8 [N][K/2]   the K x N operand stored column-major, i.e. each
 *                          of the N columns is K-contiguous
 *   b_sf  uint8 [N][K/16]
 *   D     uint16 [M][N]    bf16 bit patterns
 *
 * Ownership and execution: every pointer argument except `workspace`-free
 * host scalars is device memory owned by the caller.  The library never
 * allocates device memory and keeps no device state between calls.  All work
 * is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 * stream) with no internal synchronisation, so calls can be captured in a HIP
 * graph.  Argument errors are detected on the host before anything is
 * enqueued; faults inside kernels surface at the caller's next
 * synchronisation, as with any HIP launch.
 *
 * Errors: every entry point returns an nvfp4_status; a non-zero status leaves
 * all outputs untouched and nvfp4_last_error() returns a message for the
 * calling thread (compare the K-mismatch error of the pages, "The Art of
 * Reading the Manual", section "Why This Message Was Written").  There is no
 * backend choice and no fallback chain: one code path for gfx950.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* negative size, K % 16 != 0, offsets/E invalid */
  NVFP4_ERR_ALIGN = 3,       /* a base pointer is not aligned as documented */
  NVFP4_ERR_UNSUPPORTED = 4, /* valid NVFP4 call outside the library's supported shapes (K % 256 != 0, K > 2^22) */
  NVFP4_ERR_WORKSPACE = 5,   /* workspace missing or smaller than *_workspace_size() */
  NVFP4_ERR_HIP = 6          /* a HIP runtime call or launch failed */
} nvfp4_status;

/*
 * Single GEMM (mm_fp4).  a, b, a_sf, b_sf: 16-byte aligned;
 * d: 4-byte aligned.  K must be a multiple of 256 and at most 2^22
 * (ERR_UNSUPPORTED otherwise; ERR_SHAPE if not a multiple of 16).  alpha: device fp32 scalar, NULL means
 * 1.0f.  M == 0 or N == 0 is a successful no-op.  workspace: device memory of
 * at least nvfp4_gemm_workspace_size(M, N, K) bytes (may be NULL when that
 * size is 0), 256-byte aligned.  Split-K plans keep per-tile arrival
 * counters (first 4096 bytes) and fp32 partial tiles (after them) in it: the
 * buffer must be zero-filled once before its first use (nvfp4_workspace_init,
 * or any zero fill), and every completed call leaves the counters at zero
 * again, so one workspace serves any number of calls and shapes.  Calls that
 * share a workspace must be ordered on one stream (concurrent calls on one
 * workspace race).
 */
nvfp4_status nvfp4_gemm(const uint8_t* a, const uint8_t* a_sf,
                        const uint8_t* b, const uint8_t* b_sf,
                        const float* alpha, uint16_t* d,
                        int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same checks, plans, kernels and results as nvfp4_gemm, with the split-K
 * counters and partial tiles in a fixed 16 MiB array that the library holds on
 * each GPU it runs on, until the process ends.  No allocation and no workspace
 * argument.  The first call on a device looks the array up
 * (hipGetSymbolAddress) and clears its counters with a kernel on `stream`;
 * every completed call leaves them at zero again.  Every call on one GPU
 * shares the array: calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  A shape whose plan needs
 * more scratch than the array holds (none of the library's own plans does:
 * at most 12 MiB) returns NVFP4_ERR_WORKSPACE.
 */
nvfp4_status nvfp4_gemm_noalloc(const uint8_t* a, const uint8_t* a_sf,
                                const uint8_t* b, const uint8_t* b_sf,
                                const float* alpha, uint16_t* d,
                                int64_t M, int64_t N, int64_t K, void* stream);

/* Workspace bytes nvfp4_gemm needs for this shape: 0 unless the plan splits K
 * across work-groups (mid M with few output tiles, e.g. 512 x 768 x 6144). */
size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/* Zero-fill a workspace on `stream` with a kernel (safe inside graph capture). */
nvfp4_status nvfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-by-expert GEMM (the per-expert FP4 GEMMs of an MoE layer: pages
 * "When a Benchmark Crashes", section "Why This Message Was Written": 256
 * experts, 8 active per token, tokens scattered thinly over experts).
 * Rows offsets[e] .. offsets[e+1]-1 of A are multiplied by expert e's weights:
 *   D[r][n] = bf16_rne( alpha[e] * sum_k xA[r][k] * xB_e[n][k] ).
 *   a      uint8 [rows][K/2],  a_sf uint8 [rows][K/16]
 *   b      uint8 [E][N][K/2],  b_sf uint8 [E][N][K/16]
 *   offsets int32 [E+1], device memory, offsets[0] = 0, non-decreasing,
 *          offsets[E] <= rows.  Rows at or beyond offsets[E] are not written.
 *   alpha  fp32 [E], device memory; NULL means all 1.0f.
 *   d      uint16 [rows][N] bf16.
 *   status optional device int32: if non-NULL it is set to 0 when offsets are
 *          valid, or to 1 + (first bad expert) when offsets decrease or exceed
 *          rows; bad experts are skipped (their rows are not written).
 * Empty experts cost no weight traffic.  workspace, workspace_bytes:
 * reserved.  No grouped kernel keeps scratch memory, so
 * nvfp4_grouped_workspace_size() returns 0 and the arguments are ignored
 * (NULL and 0 are valid).
 */
nvfp4_status nvfp4_grouped_gemm(const uint8_t* a, const uint8_t* a_sf,
                                const uint8_t* b, const uint8_t* b_sf,
                                const int32_t* offsets, const float* alpha,
                                uint16_t* d, int64_t rows, int64_t N, int64_t K,
                                int32_t E, void* workspace, size_t workspace_bytes,
                                int32_t* status, void* stream);

size_t nvfp4_grouped_workspace_size(int64_t rows, int64_t N, int64_t K, int32_t E);

/*
 * Grouped GEMM on pre-packed weights.  The pages run the MoE expert GEMM
 * over static expert weights ("When a Benchmark Crashes: The Elusive FP4 GEMM
 * Comparison on Blackwell SM120", section "Why This Message Was Written": 256
 * experts, per-expert batches of 16-64 tokens), which makes it bound by the
 * weight stream from HBM.  Rearranging those weights once, so that each
 * 256-element K stage of each 256-row slab of an expert is one contiguous
 * block, lets the kernel stream them in long runs.  The arithmetic is that of
 * nvfp4_grouped_gemm; only the weight layout differs.
 *
 * nvfp4_grouped_packed_size: bytes of the packed codes (return value) and of
 * the packed scales (*sf_bytes, if non-NULL) for E experts of N x K weights;
 * 0 when the shape is not supported (K % 512 != 0, K > 2^22, N, E <= 0).
 *
 * nvfp4_grouped_pack_b: b uint8 [E][N][K/2] and b_sf uint8 [E][N][K/16]
 * (the nvfp4_grouped_gemm layout) -> packed, packed_sf (caller-allocated,
 * sizes from nvfp4_grouped_packed_size).  Layout, per expert e, slab
 * t = 0 .. ceil(N/256)-1 and stage k = 0 .. K/256-1: block
 * k * (E * ceil(N/256)) + e * ceil(N/256) + t (stage-major, so the work-groups
 * running at one time read neighbouring blocks) holds rows t*256 .. t*256+255
 * of expert e and K elements 256k .. 256k+255 (rows past N are zero).  A code block is
 * 2048 chunks of 16 bytes: chunk c (0..7, K elements 256k + 32c ..) of row r
 * (0..255) is stored at chunk position
 * (((r / 32) * 2 + (r % 32) / 16) * 2 + c / 4) * 64 + (c % 4) * 16 + r % 16,
 * the order in which the kernel's lanes load them.  A scale block is 1024
 * words of 4 bytes: word w (0..3, scale bytes 4w .. 4w+3 of the stage) of row
 * r is stored at word position
 * ((((r / 32) * 16 + r % 16) * 2 + w % 2) * 4 + ((r % 32) / 16) * 2 + w / 2,
 * so that each lane's four words are one 16-byte chunk.  All pointers
 * 16-byte aligned.
 * K % 512 == 0 (ERR_UNSUPPORTED otherwise).  Asynchronous on stream.
 *
 * nvfp4_grouped_gemm_packed: as nvfp4_grouped_gemm with b, b_sf replaced by
 * the packed buffers; no workspace.  K % 512 == 0.
 */
size_t nvfp4_grouped_packed_size(int64_t N, int64_t K, int32_t E, size_t* sf_bytes);
nvfp4_status nvfp4_grouped_pack_b(const uint8_t* b, const uint8_t* b_sf, int64_t N, int64_t K, int32_t E,
                                  uint8_t* packed, uint8_t* packed_sf, void* stream);
nvfp4_status nvfp4_grouped_gemm_packed(const uint8_t* a, const uint8_t* a_sf, const uint8_t* packed,
                                       const uint8_t* packed_sf, const int32_t* offsets, const float* alpha,
                                       uint16_t* d, int64_t rows, int64_t N, int64_t K, int32_t E,
                                       int32_t* status, void* stream);

/*
 * Grouped GEMM with the activation quantisation fused into the A load: the
 * step before the GEMM in an MoE layer (token gather and NVFP4 quantisation
 * of the activations), done by the GEMM kernel itself instead of a quantise
 * kernel and a gather.  The pages benchmark the expert GEMM on already
 * quantised operands ("When a Benchmark Crashes: The Elusive FP4 GEMM
 * Comparison on Blackwell SM120", section "Why This Message Was Written");
 * the quantisation rules are those of nvfp4_quantize below.
 *
 *   A[i][:] = NVFP4(x[row_token[i]][:], *a_global_scale)   (x[i] if row_token is NULL)
 *   D = nvfp4_grouped_gemm(A, B, offsets, alpha)
 *
 * x: bf16 [T][K] activations (device, 16-byte aligned); bf16 values are
 * exact fp32 values, so the result equals nvfp4_quantize on their fp32
 * copy, a row gather and nvfp4_grouped_gemm, bit for bit.  row_token: int32
 * [rows] device, token of each expert-sorted row, or NULL (then rows <= T).
 * Tokens outside [0, T) read as zero rows.  a_global_scale: device fp32
 * encode scale shared by all rows (a static activation scale; NULL = 1.0).
 * b, b_sf: [E][N][K/2] and [E][N][K/16] (nvfp4_grouped_gemm_fused) or the
 * buffers of nvfp4_grouped_pack_b (nvfp4_grouped_gemm_packed_fused).
 * offsets, alpha, d, status: as nvfp4_grouped_gemm; in addition, when the
 * offsets are valid, *status = -(1 + i) for the first row i whose token lies
 * outside [0, T).  K % 512 == 0 and T * K * 2 < 2^31 (ERR_UNSUPPORTED
 * otherwise); no workspace.  Asynchronous on stream.
 */
nvfp4_status nvfp4_grouped_gemm_fused(const uint16_t* x, const int32_t* row_token, const float* a_global_scale,
                                      const uint8_t* b, const uint8_t* b_sf, const int32_t* offsets,
                                      const float* alpha, uint16_t* d, int64_t rows, int64_t T, int64_t N,
                                      int64_t K, int32_t E, int32_t* status, void* stream);
nvfp4_status nvfp4_grouped_gemm_packed_fused(const uint16_t* x, const int32_t* row_token,
                                             const float* a_global_scale, const uint8_t* packed,
                                             const uint8_t* packed_sf, const int32_t* offsets, const float* alpha,
                                             uint16_t* d, int64_t rows, int64_t T, int64_t N, int64_t K, int32_t E,
                                             int32_t* status, void* stream);

/*
 * The MoE expert FFN over the grouped GEMM.  The pages run each MoE layer's
 * experts through a fused MoE kernel (cutlass_moe) with 256 experts, 8 active
 * per token, hidden size H = 6144 and expert intermediate size I = 2048
 * ("When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on Blackwell
 * SM120", sections "Why This Message Was Written" and "The Thinking Process
 * Visible in Reasoning Parts").  The activation is not named on the pages;
 * it is read as SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + exp(-g)),
 * with gate and up the first and second I columns of the gate/up output.
 *
 * nvfp4_swiglu_quantize: gu bf16 [rows][2I] -> h in fp32 -> NVFP4 with the
 * quantiser of nvfp4_quantize and the device encode scale gs (NULL = 1.0):
 * q uint8 [rows][I/2], sf uint8 [rows][I/16].  I % 16 == 0; gu, q 16-byte
 * aligned.
 *
 * nvfp4_moe_combine: out bf16 [T][H] row t = sum over j < top_k, in j
 * order, of weight[t][j] * down[rows_of[t][j]] (bf16 [rows][H]), in fp32,
 * rounded once to bf16; an index outside [0, rows) adds nothing.  H % 8 == 0;
 * down, out 16-byte aligned.
 *
 * nvfp4_moe_ffn: one MoE layer's experts for T tokens routed top_k of E:
 *   gu   = nvfp4_grouped_gemm_packed_fused(x, row_token, gs_x, w_gu)  [rows][2I]
 *   h    = nvfp4_swiglu_quantize(gu, gs_h)                            [rows][I] NVFP4
 *   down = nvfp4_grouped_gemm_packed(h, w_d)                          [rows][H]
 *   out  = nvfp4_moe_combine(down, token_rows, token_weight)          [T][H]
 * with rows = T * top_k sorted by expert (offsets [E+1], row_token [rows]:
 * the token of each row) and token_rows [T][top_k] the inverse map (the row
 * of each of a token's experts); token_weight [T][top_k] fp32 routing
 * weights; token_rows must name rows that the offsets cover (rows outside
 * every expert range hold unspecified values).  x bf16 [T][H]; w_gu, w_gu_sf:
 * expert weights [E][2I][H/2] packed
 * by nvfp4_grouped_pack_b (N = 2I, K = H); w_d, w_d_sf: [E][H][I/2] packed
 * (N = H, K = I); alpha_gu, alpha_d: device fp32 [E] (NULL = 1.0); gs_x, gs_h:
 * device encode scales (NULL = 1.0).  The intermediates live in the
 * caller's workspace (nvfp4_moe_ffn_workspace_size bytes, 256-byte
 * aligned).  H % 512 == 0 and I % 512 == 0 (ERR_UNSUPPORTED otherwise),
 * T * H * 2 < 2^31.  status: as nvfp4_grouped_gemm_fused (offsets, then
 * tokens).  Asynchronous on stream.
 */
/*
 * nvfp4_quantize_rows_bf16: the gather and quantisation of the fused grouped
 * GEMM as a separate step: row i of q uint8 [rows][K/2], sf uint8
 * [rows][K/16] is the NVFP4 quantisation (the rules of nvfp4_quantize, encode
 * scale *gs, NULL = 1.0) of bf16 row row_token[i] of x [T][K] (row i when
 * row_token is NULL, then rows <= T); tokens outside [0, T) give zero rows.
 * K % 16 == 0; x, q 16-byte aligned.  Asynchronous on stream.
 */
nvfp4_status nvfp4_quantize_rows_bf16(const uint16_t* x, const int32_t* row_token, const float* gs, uint8_t* q,
                                      uint8_t* sf, int64_t rows, int64_t T, int64_t K, void* stream);
nvfp4_status nvfp4_swiglu_quantize(const uint16_t* gu, int64_t rows, int64_t I, const float* gs, uint8_t* q,
                                   uint8_t* sf, void* stream);
nvfp4_status nvfp4_moe_combine(const uint16_t* down, const int32_t* rows_of, const float* weight, uint16_t* out,
                               int64_t T, int64_t H, int32_t top_k, int64_t rows, void* stream);
size_t nvfp4_moe_ffn_workspace_size(int64_t T, int64_t H, int64_t I, int32_t top_k);
nvfp4_status nvfp4_moe_ffn(const uint16_t* x, const float* gs_x, const int32_t* row_token, const int32_t* offsets,
                           const uint8_t* w_gu, const uint8_t* w_gu_sf, const float* alpha_gu, const float* gs_h,
                           const uint8_t* w_d, const uint8_t* w_d_sf, const float* alpha_d,
                           const int32_t* token_rows, const float* token_weight, uint16_t* out, int64_t T,
                           int64_t H, int64_t I, int32_t E, int32_t top_k, void* workspace,
                           size_t workspace_bytes, int32_t* status, void* stream);

/*
 * Scale-layout interop.  The pages only name the switch between scale
 * layouts ("The Art of Reading the Manual: Debugging FP4 GEMM Kernels on
 * Blackwell SM120", section "The Message": use_8x4_sf_layout=False); this
 * library takes linear [rows][K/16] scales.  These calls convert to and from
 * the 128 x 4 tiled layout of the CUTLASS NVFP4 path (read as: the scale
 * matrix, zero-padded to a multiple of 128 rows and 4 columns, stored as
 * 512-byte tiles of 128 rows x 4 columns in row-major tile order, the scale
 * of row r and column c of a tile at byte (r % 32) * 16 + ((r % 128) / 32) * 4
 * + c % 4), for example once at weight-load time.
 *
 * nvfp4_scales_128x4_size: bytes of the tiled layout for rows x K (K % 16 ==
 * 0; 0 for invalid sizes).  nvfp4_scales_to_128x4: sf uint8 [rows][K/16] ->
 * tiled (padding written as zero).  nvfp4_scales_from_128x4: tiled -> sf.
 * Device pointers, no alignment requirement; asynchronous on stream.
 */
size_t nvfp4_scales_128x4_size(int64_t rows, int64_t K);
nvfp4_status nvfp4_scales_to_128x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, void* stream);
nvfp4_status nvfp4_scales_from_128x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, void* stream);

/*
 * The same conversions for the 8 x 4 layout, the one use_8x4_sf_layout=True
 * selects in the mm_fp4 signature ("The Art of Reading the Manual", section
 * "The Message"; not described there either), read as: the scale matrix,
 * zero-padded to a multiple of 8 rows and 4 columns, stored as 32-byte tiles
 * of 8 rows x 4 columns in row-major tile order, the scale of row r and column
 * c of a tile at byte (r % 8) * 4 + c % 4.  Sizes, padding, pointers and
 * errors as for the 128 x 4 calls.
 */
size_t nvfp4_scales_8x4_size(int64_t rows, int64_t K);
nvfp4_status nvfp4_scales_to_8x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, void* stream);
nvfp4_status nvfp4_scales_from_8x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, void* stream);

/*
 * nvfp4_gemm with both scale tensors in one of the tiled layouts above (the
 * counterpart of the use_8x4_sf_layout switch of the mm_fp4 signature, "The
 * Art of Reading the Manual", section "The Message"): sf_layout 1 = the 128 x 4
 * layout of nvfp4_scales_to_128x4, 2 = the 8 x 4 layout of
 * nvfp4_scales_to_8x4, 0 = linear (then the call is nvfp4_gemm).  a_sf holds
 * the tiled bytes of the M x K operand (nvfp4_scales_128x4_size(M, K) or
 * nvfp4_scales_8x4_size(M, K)), b_sf those of the N x K operand; padding
 * bytes are not read.  Every automatic plan reads 8 x 4 scales in place, and
 * the plans of small M (the register tiles, M <= 128 at most widths) read
 * 128 x 4 scales in place too; the other plans first write linear copies of
 * 128 x 4 scales into the workspace (two conversion launches on stream, then
 * the GEMM).  The workspace must hold
 * nvfp4_gemm_sf_workspace_size(M, N, K, sf_layout) bytes, 256-byte aligned,
 * zero-filled once before first use as for nvfp4_gemm.  Everything else
 * (arguments, alignment, results bit for bit, errors) is as for nvfp4_gemm;
 * an sf_layout outside 0..2 is NVFP4_ERR_SHAPE.  The layouts are readings:
 * the pages name the switch and describe no layout.
 */
nvfp4_status nvfp4_gemm_sf(const uint8_t* a, const uint8_t* a_sf,
                           const uint8_t* b, const uint8_t* b_sf,
                           const float* alpha, uint16_t* d,
                           int64_t M, int64_t N, int64_t K, int32_t sf_layout,
                           void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes of nvfp4_gemm_sf (0 for invalid sizes or layouts). */
size_t nvfp4_gemm_sf_workspace_size(int64_t M, int64_t N, int64_t K, int32_t sf_layout);

/*
 * nvfp4_grouped_gemm with its scales in one of the tiled layouts (sf_layout 1
 * = 128 x 4, 2 = 8 x 4, 0 = linear, then the call is nvfp4_grouped_gemm
 * without a workspace): a_sf is the tiled form of the [rows][K/16] activation
 * scales (nvfp4_scales_<layout>_size(rows, K) bytes), b_sf that of the
 * experts' scales taken as one [E * N][K/16] matrix (row e * N + n;
 * nvfp4_scales_<layout>_size(E * N, K) bytes).  The register-streamed kernels
 * read both in place; K must be a multiple of 512 (NVFP4_ERR_UNSUPPORTED
 * otherwise).  Everything else (offsets, alpha, status, results bit for bit)
 * is as for nvfp4_grouped_gemm.  For the weights' scales the 8 x 4 layout
 * also loads fewer cache lines per instruction than the linear one.
 */
nvfp4_status nvfp4_grouped_gemm_sf(const uint8_t* a, const uint8_t* a_sf,
                                   const uint8_t* b, const uint8_t* b_sf,
                                   const int32_t* offsets, const float* alpha, uint16_t* d,
                                   int64_t rows, int64_t N, int64_t K, int32_t E, int32_t sf_layout,
                                   int32_t* status, void* stream);

/*
 * Quantise fp32 x [R][K] to NVFP4 (q uint8 [R][K/2], sf uint8 [R][K/16]).
 * The pages never quantise (their test used random bytes); this follows the
 * block_size 16 and e4m3fn scale format of the pages above with these steps,
 * all fp32 round-to-nearest-even, per 16-element block of one row:
 *   t  = (amax_block / 6) * gs;         sf = e4m3fn_rne_saturating(t)
 *   r  = gs / E4M3(sf)  (0 if E4M3(sf) == 0, correctly rounded division)
 *   code = e2m1_rne_saturating(x * r)   (sign bit kept, so -0 -> 0x8)
 * global_scale: device fp32 encode scale gs; NULL means 1.0f.  K % 16 == 0;
 * x 16-byte aligned, q 8-byte aligned (ERR_ALIGN otherwise); non-finite
 * inputs are outside the contract.
 */
nvfp4_status nvfp4_quantize(const float* x, int64_t R, int64_t K,
                            const float* global_scale, uint8_t* q, uint8_t* sf,
                            void* stream);

/*
 * Per-tensor encode scale: gs = (6 * 448) / max|x| in fp32 (1.0f if all x
 * are zero), written to the device fp32 *gs.  n >= 0.  The caller's *gs is
 * also used as the reduction cell, so it must not alias x.
 */
nvfp4_status nvfp4_global_scale(const float* x, int64_t n, float* gs, void* stream);

/*
 * alpha[i] = 1.0f / (gs_a[0] * gs_b[i]) in fp32 for i < count: the product of
 * the two decode factors, for one activation tensor and `count` weight
 * tensors (count = E for the grouped GEMM, 1 for a single GEMM).
 */
nvfp4_status nvfp4_alpha_from_scales(const float* gs_a, const float* gs_b,
                                     float* alpha, int32_t count, void* stream);

/* Name of the kernel plan nvfp4_gemm picks for a shape (static string). */
const char* nvfp4_gemm_plan(int64_t M, int64_t N, int64_t K);

/*
 * MXFP4 GEMM: the format the signature of mm_fp4 switches to with
 * use_nvfp4 = False ("The Art of Reading the Manual: Debugging FP4 GEMM
 * Kernels on Blackwell SM120", section "The Message").  The pages do not
 * describe it; this follows the OCP Microscaling Formats (MX) v1.0 MXFP4
 * element and scale types:
 *   D[m][n] = bf16_rne(alpha * sum_k E2M1(a[m][k]) * 2^(a_sf[m][k/32] - 127)
 *                                    * E2M1(b[n][k]) * 2^(b_sf[n][k/32] - 127))
 * a uint8 [M][K/2], b uint8 [N][K/2] (two codes per byte, element 2j in the
 * low nibble of byte j; b is the column-major K x N operand, as in
 * nvfp4_gemm), a_sf uint8 [M][K/32], b_sf uint8 [N][K/32] (E8M0 exponents).
 * The hardware scaled FP4 MFMA applies the scales and accumulates in fp32.
 * Scale byte 0xFF (NaN) and products outside the fp32 range are outside
 * the contract.  K % 256 == 0 and K <= 2^22 (ERR_UNSUPPORTED; ERR_SHAPE if
 * not a multiple of 32); a, b 16-byte aligned; a_sf, b_sf 4-byte aligned;
 * d, alpha 4-byte aligned.  alpha, workspace, ownership and stream as for
 * nvfp4_gemm (the workspace query below; split-K plans keep their counters
 * in the first 4096 bytes, which every completed call leaves at zero).
 */
nvfp4_status nvfp4_mx_gemm(const uint8_t* a, const uint8_t* a_sf,
                           const uint8_t* b, const uint8_t* b_sf,
                           const float* alpha, uint16_t* d,
                           int64_t M, int64_t N, int64_t K,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes nvfp4_mx_gemm needs for this shape (0 unless it splits K). */
size_t nvfp4_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/* Name of the kernel plan nvfp4_mx_gemm picks for a shape (static string). */
const char* nvfp4_mx_gemm_plan(int64_t M, int64_t N, int64_t K);

/*
 * Plan override, for tuning sweeps and tests only: every later call of the
 * family in this process runs plan `kind` (the kinds are the library's
 * kernel instantiations; a kind the family does not have leaves its own
 * choice in place) with `splits` K splits where the plan can split K
 * (splits <= 0: the plan's own count).  family: 0 = nvfp4_gemm, 1 =
 * nvfp4_mx_gemm, 2 = the grouped GEMMs (kinds 0..3: per-wave dequantisation,
 * shared f16 A tile, 32-row and 64-row register kernels; the packed and fused
 * calls take kind 3 as 64-row passes and anything else as 32-row passes).
 * kind < 0 restores the library's choice.  The plan and workspace queries
 * follow the override.  Not synchronised with calls in flight on other
 * threads: set it while no call of the family is being made.  ERR_SHAPE for
 * an unknown family or out-of-range kind or splits (> 16).
 */
nvfp4_status nvfp4_force_plan(int32_t family, int32_t kind, int32_t splits);

/* Message describing the calling thread's last error ("" if none). */
const char* nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
