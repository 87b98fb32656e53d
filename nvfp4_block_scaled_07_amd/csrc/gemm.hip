// NVFP4 block-scaled GEMM kernels for gfx950.
//
// D[m][n] = bf16(alpha * sum_k xA[m][k] * xB[n][k]), x = E2M1(code) * E4M3(scale)
// (pages "The Art of Reading the Manual: Debugging FP4 GEMM Kernels on
// Blackwell SM120", section "The Message", and "When a Benchmark Crashes: The
// Elusive FP4 GEMM Comparison on Blackwell SM120", section "Input Knowledge
// Required", item 4: dequantise on the fly, multiply-accumulate in higher
// precision).
//
// Design (gfx950):
//  * HBM -> LDS: packed codes and scale bytes go straight into LDS with
//    buffer_load ... lds (16 or 4 bytes per lane, no VGPR staging; rows past
//    the operand read as zero), STAGES-deep ring of buffers, one barrier per
//    stage.  Code rows are stored row-major
//    with the 16-byte chunks XOR-swizzled per row, which keeps both the
//    coalesced global loads and the MFMA-side ds_read_b128 free of bank
//    conflicts.
//  * LDS -> VGPR -> MFMA: each lane reads one 16-byte chunk (32 consecutive K
//    elements of one row) and turns it into the f16 operands of 4 MFMA
//    K-steps: hardware e2m1->f16 conversion plus one packed f16 multiply by
//    the e4m3 block scale (exact in f16).  A and B use the same lane->K map,
//    so the order of K inside a chunk does not change the sum's terms.
//  * The contraction is v_mfma_f32_32x32x16_f16 (large tiles) or
//    v_mfma_f32_16x16x32_f16 (skinny and grouped tiles) with fp32
//    accumulators.  The e4m3 scales are not powers of two and come per 16
//    elements, so they cannot ride the E8M0-per-32 scaled FP4 MFMA exactly.
//  * K-groups: KS groups of waves share each LDS stage and take different
//    MFMA sub-steps of it; their accumulators are summed through LDS.  This
//    gives small problems several waves per SIMD (VALU issue from a single
//    wave is slow) without shrinking the wave tile.
//  * Split-K: each split writes its fp32 partial tile to the workspace in the
//    accumulators' register order; the last split of a tile to arrive
//    (device-scope counter) sums the partials in split order, applies alpha
//    and stores bf16, then resets the counter.  Partials and counters are
//    accessed only with agent-coherent operations, so no cache-wide fence
//    is needed.  One launch, bitwise deterministic.
//  * Register streaming: small-M tiles (k_gemm_kreg) and the grouped MoE
//    kernels (k_grouped_reg) load operands straight into VGPRs in whole
//    128-byte lines per row, two or three 256-element K units ahead, and put
//    them into MFMA layout with one DPP exchange; there the number of reads
//    a CU keeps in flight, not LDS, bounds the rate.  Expert weights can be
//    packed once (k_pack_b) into the grouped kernel's lane order.
//  * Work-group order is remapped so that work-groups sharing operand rows
//    run on the same XCD (its own 4 MB L2).
//  * The LDS read addresses of a lane are computed once per tile; stage
//    buffers, row blocks and later sub-steps are compile-time offsets in the
//    instructions' offset fields (the stage loop is unrolled by the number of
//    stages), so the stage loop issues no address arithmetic.
//
// Files: the LDS-staged tile kernel k_gemm and its helpers are in
// gemm_tile.h; the two large-M 8-wave NVFP4 tiles are instantiated in
// gemm_large.hip (built with another instruction schedule); this file holds
// the other tiles, the register-streamed and grouped kernels, the plans and
// the launchers.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "device.h"
#include "internal.h"

#include "gemm_tile.h"

namespace nvfp4 {

// Offsets check for the grouped GEMM: status = 0, or 1 + first bad expert.
__global__ void k_check_offsets(const int32_t* __restrict__ offsets, int E, int64_t rows, int32_t* status) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t bad = 0;
  for (int e = 0; e < E; ++e) {
    const int64_t lo = offsets[e], hi = offsets[e + 1];
    if (lo < 0 || hi < lo || hi > rows) {
      bad = e + 1;
      break;
    }
  }
  *status = bad;
}

// Grouped GEMM: one work-group per (expert, N tile); consecutive logical ids
// (one XCD) walk the N tiles of one expert, so its A rows stay in that L2.
template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void k_grouped(GroupedLaunch p) {
  __shared__ __attribute__((aligned(16))) Smem<C> sm;
  const int tiles_n = (int)((p.N + C::BN - 1) / C::BN);
  const int L = xcd_remap(blockIdx.x, tiles_n * p.E);
  const int e = L / tiles_n;
  const int64_t n0 = (int64_t)(L % tiles_n) * C::BN;
  const int64_t lo = p.offsets[e], hi = p.offsets[e + 1];
  if (lo < 0 || hi <= lo || hi > p.rows) return;  // empty or invalid expert
  const int64_t ld = p.K / 2, lds = p.K / 16;
  const float alpha = p.alpha ? p.alpha[e] : 1.0f;
  Operand B{p.b + ((int64_t)e * p.N + n0) * ld, p.b_sf + ((int64_t)e * p.N + n0) * lds, ld, lds,
            (int)min<int64_t>(C::BN, p.N - n0)};
  const int nk = (int)(p.K / C::BK);
  for (int64_t mc = lo; mc < hi; mc += C::BM) {
    const int rows_c = (int)min<int64_t>(C::BM, hi - mc);
    const int tm_active = (rows_c + C::MF - 1) / C::MF;  // row blocks (one wave row: WM == 1)
    Operand A{p.a + mc * ld, p.a_sf + mc * lds, ld, lds, rows_c};
    typename C::Acc acc[C::TM][C::TN];
    mainloop<C>(sm, A, B, 0, nk, tm_active, acc);
    store_bf16<C>(acc, tm_active, alpha, p.d + mc * p.N + n0, p.N, rows_c, B.rows);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with a shared f16 A tile.  Per expert only a few rows of A
// meet a wide slab of B, so the waves split N and every wave needs all A
// rows: dequantising A once per stage per work-group into LDS (instead of
// once per wave) leaves each wave only its own B columns to dequantise, and
// the kernel stays ahead of the B stream from HBM.
// ---------------------------------------------------------------------------
template <class C>
struct SmemGA {
  Smem<C> ring;
  // f16 bits of the stage's A rows, [BM][BK]; 16-byte chunk j of row r is
  // stored at slot j ^ (r & 15) (16-row MFMA reads hit 16 distinct slots)
  uint16_t af[C::BM * C::BK];
};

__device__ __forceinline__ void ds_write128(uint32_t a, const u4_t& v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// Dequantise rows [0, rows16) of ring stage `buf` into af.  One 16-byte code
// chunk (32 values) per thread and step.
template <class C>
__device__ __forceinline__ void dequant_a_stage(const SmemGA<C>& sm, int buf, int rows16) {
  const uint32_t a_base = lds_addr(sm.ring.a[buf]), as_base = lds_addr(sm.ring.asf[buf]);
  const uint32_t f_base = lds_addr(sm.af);
  const int n = rows16 * C::CH;
  for (int q = threadIdx.x; q < n; q += C::kThreads) {
    const int r = q / C::CH, c = q % C::CH;
    u4_t v;
    uint32_t sw;
    ds_read128(v, a_base + r * C::RB + ((c ^ swz<C::CH, C::MF>(r)) << 4));
    ds_read32(sw, as_base + r * C::SB + 4 * (c >> 1));
    lgkm_wait();
    pin(v);
    pin(sw);
    const h2_t sp = e4m3x2_to_h2(sw >> (16 * (c & 1)));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const h8_t o = dequant8(v[t], scale_pair(sp, t >> 1));
      u4_t w;
      __builtin_memcpy(&w, &o, 16);
      ds_write128(f_base + (r * C::BK + (((4 * c + t) ^ (r & 15)) << 3)) * 2, w);
    }
  }
}

// One stage: A operands straight from af (f16), B dequantised per wave.
template <class C>
__device__ __forceinline__ void compute_stage_ga(const SmemGA<C>& sm, int buf, int tm_active,
                                                 typename C::Acc (&acc)[C::TM][C::TN]) {
  static_assert(C::MF == 16 && C::WM == 1 && C::KS == 1, "grouped layout");
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wn = wave % C::WN;
  const int r_in = lane % C::MF, g = lane / C::MF;
  const uint32_t b_base = lds_addr(sm.ring.b[buf]), bs_base = lds_addr(sm.ring.bsf[buf]);
  const uint32_t f_base = lds_addr(sm.af);
#pragma unroll
  for (int s = 0; s < C::kSub; ++s) {
    const int c = C::KG * s + g;
    u4_t bc[C::TN];
    uint32_t bsw[C::TN];
    u4_t af[C::TM][4];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int row = wn * C::kWN + tn * C::MF + r_in;
      ds_read128(bc[tn], b_base + row * C::RB + ((c ^ swz<C::CH, C::MF>(row)) << 4));
      ds_read32(bsw[tn], bs_base + row * C::SB + 4 * (c >> 1));
    }
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      if (tm < tm_active) {
        const int row = tm * C::MF + r_in;
#pragma unroll
        for (int t = 0; t < 4; ++t) ds_read128(af[tm][t], f_base + (row * C::BK + (((4 * c + t) ^ (row & 15)) << 3)) * 2);
      }
    }
    lgkm_wait();
    h2_t bsp[C::TN];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      pin(bc[tn]);
      pin(bsw[tn]);
      bsp[tn] = e4m3x2_to_h2(bsw[tn] >> (16 * (c & 1)));
    }
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
      if (tm < tm_active)
#pragma unroll
        for (int t = 0; t < 4; ++t) pin(af[tm][t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const h8_t bf = dequant8(bc[tn][t], scale_pair(bsp[tn], t >> 1));
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) {
          if (tm < tm_active) {
            h8_t a;
            __builtin_memcpy(&a, &af[tm][t], 16);
            acc[tm][tn] = Mfma<C::MF>::run(a, bf, acc[tm][tn]);
          }
        }
      }
    }
  }
}

// LDS writes of this wave done, then a work-group barrier; loads in flight
// (vmcnt) are left alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void k_grouped_a16(GroupedLaunch p) {
  __shared__ __attribute__((aligned(16))) SmemGA<C> sm;
  const int tiles_n = (int)((p.N + C::BN - 1) / C::BN);
  const int L = xcd_remap(blockIdx.x, tiles_n * p.E);
  const int e = L / tiles_n;
  const int64_t n0 = (int64_t)(L % tiles_n) * C::BN;
  const int64_t lo = p.offsets[e], hi = p.offsets[e + 1];
  if (lo < 0 || hi <= lo || hi > p.rows) return;  // empty or invalid expert
  const int64_t ld = p.K / 2, lds = p.K / 16;
  const float alpha = p.alpha ? p.alpha[e] : 1.0f;
  Operand B{p.b + ((int64_t)e * p.N + n0) * ld, p.b_sf + ((int64_t)e * p.N + n0) * lds, ld, lds,
            (int)min<int64_t>(C::BN, p.N - n0)};
  const int n = (int)(p.K / C::BK);
  const int lane = threadIdx.x & 63, wave = wave_id();
  for (int64_t mc = lo; mc < hi; mc += C::BM) {
    const int rows_c = (int)min<int64_t>(C::BM, hi - mc);
    const int tm_active = (rows_c + C::MF - 1) / C::MF;
    Operand A{p.a + mc * ld, p.a_sf + mc * lds, ld, lds, rows_c};
    typename C::Acc acc[C::TM][C::TN];
    zero_acc<C>(acc);
    wait_vm_barrier<0>();  // the previous row chunk is done with every buffer
#pragma unroll
    for (int i = 0; i < C::STAGES - 1; ++i)
      if (i < n) issue_stage<C>(sm.ring, i, A, B, i, wave, lane, tm_active * C::MF);
    stage_ready<C>(min(C::STAGES - 2, n - 1));
    for (int i = 0; i < n; ++i) {
      const int pre = i + C::STAGES - 1;
      if (pre < n) issue_stage<C>(sm.ring, pre % C::STAGES, A, B, pre, wave, lane, tm_active * C::MF);
      dequant_a_stage<C>(sm, i % C::STAGES, tm_active * C::MF);
      lds_barrier();
      compute_stage_ga<C>(sm, i % C::STAGES, tm_active, acc);
      if (i + 1 < n) stage_ready<C>(min(C::STAGES - 2, n - 2 - i));
    }
    store_bf16<C>(acc, tm_active, alpha, p.d + mc * p.N + n0, p.N, rows_c, B.rows);
  }
}

// Whole-line operand loads: two 16-byte loads per lane cover a 16-row block of
// one 256-K unit (128 bytes per row) as 8 whole lines each, lane l reading row
// l % 8 (words 0..3) and row 8 + l % 8 (words 4..7), chunk l / 8 of each.
// Exchange with the lane 8 away in the same row of 16 so that lane 16 g + r
// holds row r, chunk 2 g in words 0..3 and chunk 2 g + 1 in words 4..7: the
// 16x16x32 MFMA operand layout, with K permuted the same way for A and B.
__device__ __forceinline__ void kreg_exchange(uint32_t (&w)[8], bool lo8) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t p = w[j], q = w[4 + j];
    const uint32_t give = lo8 ? q : p;
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, 0x128, 0xF, 0xF, false);  // row_ror:8
    w[j] = lo8 ? p : recv;
    w[4 + j] = lo8 ? recv : q;
  }
}

// Scale layouts the register-streamed kernels can read in place
// (nvfp4_gemm_sf, nvfp4_grouped_gemm_sf): 0 linear [rows][K/16]; 1 the 128 x
// 4 tiled layout (512-byte tiles of 128 rows x 4 scale columns, row-major
// tile order; row r, column c at byte (r % 32) 16 + ((r % 128) / 32) 4 + c %
// 4); 2 the 8 x 4 one (32-byte tiles of 8 rows x 4 columns; row r, column c
// at byte (r % 8) 4 + c % 4).  In both tiled layouts the 4 scales of columns
// 4 j .. 4 j + 3 of a row are one aligned word, the word a lane loads, so
// only its address changes.
template <int SFL>
struct SfLayout {
  static_assert(SFL >= 0 && SFL <= 2, "scale layout");
  // bytes between consecutive 256-element units of one row (4 words)
  static constexpr uint32_t kUnitStep = SFL == 0 ? 16 : (SFL == 1 ? 4 * 512 : 4 * 32);
  // Rows [r0, r0 + rows_valid) of a scale matrix with lds = K/16 bytes per
  // row (r0 counts rows from the matrix start, any alignment): a descriptor
  // bounded by the bytes of the row groups those rows occupy, and the offset
  // of word j of local row r in unit 0.
  static __device__ __forceinline__ rsrc_t rsrc(const uint8_t* sf, int64_t r0, int rows_valid, int64_t lds) {
    if constexpr (SFL == 0) return make_rsrc(sf + r0 * lds, (uint32_t)(rows_valid * lds));
    else if constexpr (SFL == 1)
      return make_rsrc(sf + (r0 >> 7) * 128 * lds, (uint32_t)(((r0 & 127) + rows_valid + 127) / 128 * 128 * lds));
    else return make_rsrc(sf + (r0 >> 3) * 8 * lds, (uint32_t)(((r0 & 7) + rows_valid + 7) / 8 * 8 * lds));
  }
  static __device__ __forceinline__ uint32_t offset(int64_t r0, int r, int j, int64_t lds) {
    if constexpr (SFL == 0) return (uint32_t)(r * lds + 4 * j);
    else if constexpr (SFL == 1) {
      const int q = (int)(r0 & 127) + r;
      return (uint32_t)((q >> 7) * 128 * lds + 512 * j + (q & 31) * 16 + ((q >> 5) & 3) * 4);
    } else {
      const int q = (int)(r0 & 7) + r;
      return (uint32_t)((q >> 3) * 8 * lds + 32 * j + (q & 7) * 4);
    }
  }
};

// ---------------------------------------------------------------------------
// Grouped GEMM streaming B through registers.  Every B element is used by
// exactly one wave, so B skips LDS: each lane loads its own 16-byte code
// chunks and scale words D stages ahead (buffer loads, rows past the expert's
// N read as zero), which keeps D stages of the weight stream in flight per
// wave.  A (a few rows per expert) is loaded the same way by one thread per
// 16-byte chunk, dequantised once per stage into a double-buffered f16 LDS
// tile and read by every wave.  No DMA and no manual wait counts: the
// compiler orders every load.
// ---------------------------------------------------------------------------
template <class C>
struct SmemGR {
  // f16 bits of one stage's A rows, [BM][BK]; 16-byte chunk j of row r sits at
  // slot j ^ (r & 15)
  uint16_t af[2][C::BM * C::BK];
};

template <class C, int D>
struct GRegs {
  // A: each 16-byte code chunk of the stage's A tile is split over kAP threads
  static constexpr int kAP = C::kThreads / (C::BM * C::CH);
  static_assert(kAP * C::BM * C::CH == C::kThreads && (kAP == 1 || kAP == 2 || kAP == 4), "A chunk split");
  typedef uint32_t u1_t __attribute__((ext_vector_type(1)));
  typedef typename std::conditional<kAP == 1, u4_t, typename std::conditional<kAP == 2, u2_t, u1_t>::type>::type AQ;
  u4_t bq[D][C::TN][C::kSub];
  uint32_t bs[D][C::TN][C::kSub];
  // linear scales four stages at a time: the words of stages 4 k .. 4 k + 3
  uint32_t bsq[C::TN][4];
  AQ aq[D];
  uint32_t as[D];
  // A scales four stages at a time: lane l of each DPP quad holds its word of
  // stage 4 k + l % 4 (the quad's four lanes share one word of every stage)
  uint32_t asq;
  // fused quantisation: kAX 16-byte chunks of bf16 activations per lane and
  // stage, one per 8-element half block (whole-line loads: 32 lanes per row)
  static constexpr int kAX = C::BM * C::BK * 2 / 16 / C::kThreads;
  u4_t ax[D][kAX];
};

// Loads of stage kt into register slot u.  Always the same instructions (so
// the compiler can count outstanding loads exactly); a dead stage (live ==
// false, past the end of K) uses out-of-range offsets, which return zero
// without a memory access.  Unpacked weights (whole-line loads) need one
// scale word per 16-row block and stage: with linear scales the kernel loads
// the words of four stages at once (gr_load_sq, when 4 divides the stage
// count) or the even slots those of two (8 bytes per lane, 32 of each row),
// so a 16-row block's scale load touches its 16 rows' lines once per four or
// two stages instead of once per stage; tiled scales take one word per stage
// (two lines per block in the 8 x 4 layout).  With four-stage B loads the
// A scale words come four stages at a time too where each DPP quad shares
// one word (GrQuad::kA): lane l % 4 of the quad loads stage 4 k + l % 4 and
// each stage broadcasts its lane to the quad.  With four-stage scale loads
// the weight codes are loaded non-temporal (read once), which keeps the
// scale lines, each loaded in two halves four stages apart, and the A rows
// in L2.  Packed weights hold a lane's four scale
// words (both row blocks, both sub-steps) in one 16-byte chunk.
// Packed weights: stage kt of a slab is the block at base + kt * stride
// (codes) and sbase + kt * sstride (scales); the buffer resource of each
// stage is formed from the 64-bit address, so no 32-bit offset limits the
// size of the packed tensor.
struct PackedStream {
  const uint8_t* base;
  const uint8_t* sbase;
  int64_t stride, sstride;
};

// Lane v (0..3, a constant after unrolling) of each DPP quad, broadcast to
// the quad (quad_perm v, v, v, v).
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x, int v) {
  switch (v) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xFF, 0xF, 0xF, false);
  }
}

// Which scale loads take four stages at a time: B's on plain weights with
// linear scales, and A's where each DPP quad of lanes shares one A scale word
// (two threads per A code chunk).
template <class C, int D, bool PACKED, bool FUSED, int SFL, int SG>
struct GrQuad {
  static constexpr bool kB = SG == 4 && SFL == 0 && !PACKED;
  static constexpr bool kA = kB && !FUSED && GRegs<C, D>::kAP == 2;
};

template <class C, int D, bool PACKED, bool FUSED, int SFL, int SG>
__device__ __forceinline__ void gr_load(GRegs<C, D>& R, int u, int kt, bool live, const PackedStream& ps,
                                        const rsrc_t& rb, const rsrc_t& rbs,
                                        const uint32_t (&vb)[C::TN][C::kSub], const uint32_t (&vbs)[C::TN][C::kSub],
                                        uint32_t b_step, uint32_t bs_step, const rsrc_t& ra, const rsrc_t& ras,
                                        uint32_t va, uint32_t vas, const uint32_t (&vax)[GRegs<C, D>::kAX]) {
  constexpr uint32_t kOut = 0x80000000u;
  rsrc_t rbk = rb, rbsk = rbs;
  uint32_t bo = kt * b_step, bso = kt * bs_step;
  if constexpr (PACKED) {
    rbk = make_rsrc(ps.base + (int64_t)kt * ps.stride, C::BN * C::RB);
    rbsk = make_rsrc(ps.sbase + (int64_t)kt * ps.sstride, C::BN * C::SB);
    bo = bso = 0;
  }
  if constexpr (FUSED) {
    // bf16 activations (512 bytes per row and stage), issued before the
    // slot's weights so that waiting for them leaves the weights in flight
#pragma unroll
    for (int i = 0; i < GRegs<C, D>::kAX; ++i)
      R.ax[u][i] = __builtin_bit_cast(
          u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? vax[i] : kOut, kt * C::BK * 2, 0));
  }
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
    for (int s = 0; s < C::kSub; ++s) {
      R.bq[u][tn][s] = __builtin_bit_cast(
          u4_t, __builtin_amdgcn_raw_buffer_load_b128(rbk, live ? vb[tn][s] : kOut, bo,
                                                      GrQuad<C, D, PACKED, FUSED, SFL, SG>::kB ? 2 : 0));
      if (!PACKED && s == 0) {
        if constexpr (SFL == 0) {
          // linear scales: an even slot loads the words of two stages (u odd
          // loads none), spread over the lane rows as gr_compute expects
          if (SG == 2 && u % 2 == 0) {
            const u2_t w = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(rbsk, live ? vbs[tn][0] : kOut,
                                                                                         bso, 0));
            R.bs[u][tn][0] = w[0];
            R.bs[u][tn][1] = w[1];
          }
        } else {
          R.bs[u][tn][0] = __builtin_amdgcn_raw_buffer_load_b32(rbsk, live ? vbs[tn][0] : kOut, bso, 0);
        }
      }
    }
  if constexpr (PACKED) {
    const u4_t w = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rbsk, live ? vbs[0][0] : kOut,
                                                                                  bso, 0));
    R.bs[u][0][0] = w[0]; R.bs[u][0][1] = w[1]; R.bs[u][1][0] = w[2]; R.bs[u][1][1] = w[3];
  }
  typedef typename GRegs<C, D>::AQ AQ;
  if constexpr (!FUSED) {
    if constexpr (GRegs<C, D>::kAP == 1)
      R.aq[u] = __builtin_bit_cast(AQ, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? va : kOut, kt * C::RB, 0));
    else if constexpr (GRegs<C, D>::kAP == 2)
      R.aq[u] = __builtin_bit_cast(AQ, __builtin_amdgcn_raw_buffer_load_b64(ra, live ? va : kOut, kt * C::RB, 0));
    else
      R.aq[u] = __builtin_bit_cast(AQ, __builtin_amdgcn_raw_buffer_load_b32(ra, live ? va : kOut, kt * C::RB, 0));
    if constexpr (!GrQuad<C, D, PACKED, FUSED, SFL, SG>::kA)
      R.as[u] = __builtin_amdgcn_raw_buffer_load_b32(ras, live ? vas : kOut,
                                                     kt * (SFL == 0 ? C::SB : (int)SfLayout<SFL>::kUnitStep), 0);
  }
}

// Linear B scales four stages at a time (stages kt .. kt + 3, kt % 4 == 0):
// lane row g (lanes 16 g .. 16 g + 15) loads the 16 bytes of stage kt + g of
// its row, so the instruction touches each of a 16-row block's lines once per
// four stages.  gr_split_sq then leaves word g of stage kt + s in bsq[tn][s]
// (a 4 x 4 transpose over lane rows and registers: lane-row halves swapped
// with permlane32, then single lane rows with permlane16).
template <class C, int D, bool AQ>
__device__ __forceinline__ void gr_load_sq(GRegs<C, D>& R, int kt, bool live, const rsrc_t& rbs,
                                           const uint32_t (&vbs)[C::TN][C::kSub], uint32_t bs_step, const rsrc_t& ras,
                                           uint32_t vas) {
  if constexpr (AQ) R.asq = __builtin_amdgcn_raw_buffer_load_b32(ras, live ? vas : 0x80000000u, kt * C::SB, 0);
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
    const u4_t w = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rbs, live ? vbs[tn][0] : 0x80000000u,
                                                                                  kt * bs_step, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) R.bsq[tn][j] = w[j];
  }
}

template <class C, int D>
__device__ __forceinline__ void gr_split_sq(GRegs<C, D>& R) {
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
    uint32_t* q = R.bsq[tn];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto w = __builtin_amdgcn_permlane32_swap(q[j], q[j + 2], false, false);
      q[j] = w[0];
      q[j + 2] = w[1];
    }
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const auto w = __builtin_amdgcn_permlane16_swap(q[j], q[j + 1], false, false);
      q[j] = w[0];
      q[j + 1] = w[1];
    }
  }
}

// PACKED: B (codes and scales) in the layout written by k_pack_b (each
// stage of a 256-row slab is one block, blocks in stage-major order; rows
// past N are zero);
// every code load instruction reads 1 KB in lane order, lane 16 g + r holds
// chunks g and 4 + g of row r, and a wave's scale words for the stage are one
// 512-byte run.  Unpacked `[E][N][K/2]` weights are read in
// whole 128-byte lines as in the register K-group tile: sub-step s loads rows
// 8 s + lane % 8 of each 16-row block, chunk lane / 8, and one DPP rotation
// gives lane 16 g + r chunks 2 g and 2 g + 1 of row r, whose four scales are
// one word.
//
// FUSED: A is not stored quantised.  Wave w loads rows w * BM/8 .. of the
// stage from the bf16 activations (row row_token[i] of x for the expert's row
// i) in whole lines, two rows per instruction: lane l reads 16 bytes
// (elements 8 (l % 32) .. + 7) of row 2 j + l / 32 of its rows, so the lane
// pairs (l, l ^ 1) hold the two halves of one 16-element block.  Each lane
// takes the block's amax over its pair (one DPP swap), quantises its half
// with the rules of the quantise kernel (quantize_half_block16) and writes
// the dequantised f16 values to the A tile, so the tile, and therefore D, is
// bit for bit what the quantise kernel, a row gather and the unfused kernel
// produce.  Tokens outside [0, T) read as zero rows.
// The stage's A codes of register slot u (this thread's part ah of chunk ac
// of row ar) dequantised into the f16 A tile af.
template <class C, int D>
__device__ __forceinline__ void gr_dequant_a(const GRegs<C, D>& R, int u, uint16_t* af, int ar, int ac, int ah) {
  typedef GRegs<C, D> RT;
  const h2_t sp = e4m3x2_to_h2(R.as[u] >> (16 * (ac & 1)));
#pragma unroll
  for (int tt = 0; tt < 4 / RT::kAP; ++tt) {
    const int t = ah * (4 / RT::kAP) + tt;  // 8-value group of the chunk
    const h8_t o = dequant8(R.aq[u][tt], scale_pair(sp, t >> 1));
    *(h8_t*)(af + ar * C::BK + (((4 * ac + t) ^ (ar & 15)) << 3)) = o;
  }
}

// One stage of the grouped register kernels after the A tile is in LDS:
// the B fragments of register slot u (whole-line loads are first put into
// MFMA layout by the DPP exchange) dequantised and multiplied with the f16 A
// tile af.
template <class C, int D, bool PACKED, int SFL, int SG>
__device__ __forceinline__ void gr_compute(GRegs<C, D>& R, int u, const uint16_t* af,
                                           typename C::Acc (&acc)[C::TM][C::TN], int r_in, int g, bool lo8) {
  if constexpr (!PACKED && SFL == 0) {
    // linear scales of stages kt (this slot) and kt + 1 (the next): lane row
    // g (lanes 16 g .. 16 g + 15) loaded the 8 bytes at 8 ((g & 1) 2 + g / 2)
    // of the two stages' 32, so rows 0 and 2 hold words 0, 1 and 2, 3 of
    // stage kt and rows 1 and 3 those of stage kt + 1.  Swapping the odd rows
    // of the first word with the even rows of the second leaves word g of
    // stage kt in the first and word g of stage kt + 1 in the second.
    if (SG == 2 && u % 2 == 0) {
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const auto w = __builtin_amdgcn_permlane16_swap(R.bs[u][tn][0], R.bs[u][tn][1], false, false);
        R.bs[u][tn][0] = w[0];
        R.bs[u + 1][tn][0] = w[1];
      }
    }
  }
  if constexpr (!PACKED) {
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) { w[j] = R.bq[u][tn][0][j]; w[4 + j] = R.bq[u][tn][1][j]; }
      kreg_exchange(w, lo8);
#pragma unroll
      for (int j = 0; j < 4; ++j) { R.bq[u][tn][0][j] = w[j]; R.bq[u][tn][1][j] = w[4 + j]; }
    }
  }
#pragma unroll
  for (int s = 0; s < C::kSub; ++s) {
    const int c = PACKED ? C::KG * s + g : 2 * g + s;
    h2_t bsp[C::TN];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
      bsp[tn] = PACKED ? e4m3x2_to_h2(R.bs[u][tn][s] >> (16 * (c & 1))) : e4m3x2_to_h2(R.bs[u][tn][0] >> (16 * s));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (C::TM <= 2) {
        h8_t a[C::TM];
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) {
          const int row = tm * C::MF + r_in;
          a[tm] = *(const h8_t*)(af + row * C::BK + (((4 * c + t) ^ (row & 15)) << 3));
        }
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
          const h8_t bf = dequant8(R.bq[u][tn][s][t], scale_pair(bsp[tn], t >> 1));
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm) acc[tm][tn] = Mfma<C::MF>::run(a[tm], bf, acc[tm][tn]);
        }
      } else {
        // taller tiles: dequantise the B fragments first, then stream
        // one A fragment at a time (fewer live registers)
        h8_t bf[C::TN];
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bf[tn] = dequant8(R.bq[u][tn][s][t], scale_pair(bsp[tn], t >> 1));
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) {
          const int row = tm * C::MF + r_in;
          const h8_t a = *(const h8_t*)(af + row * C::BK + (((4 * c + t) ^ (row & 15)) << 3));
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = Mfma<C::MF>::run(a, bf[tn], acc[tm][tn]);
        }
      }
    }
  }
}

// Fused quantisation of one stage's activations (register slot ax) into the
// f16 A tile af: each lane quantises its half blocks and writes their
// dequantised values as 8-value group lane % 32 of its rows.
template <class C, int D>
__device__ __forceinline__ void gr_fused_a(const u4_t (&ax)[GRegs<C, D>::kAX], uint16_t* af, float gs, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < GRegs<C, D>::kAX; ++i) {
    const int r = wave * 2 * GRegs<C, D>::kAX + 2 * i + (lane >> 5);
    f4_t lo, hi;
    bf16x8_to_f32(ax[i], lo, hi);
    uint32_t w;
    const uint32_t code = quantize_half_block16(lo, hi, gs, w);
    const _Float16 sh = (_Float16)e4m3_value_pos(code);  // exact
    *(h8_t*)(af + r * C::BK + (((lane & 31) ^ (r & 15)) << 3)) = dequant8(w, h2_t{sh, sh});
  }
}

template <class C, int D, bool PACKED, bool FUSED = false, int SFL = 0, int SG = 2>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_grouped_reg(
    GroupedLaunch p) {
  static_assert(C::MF == 16 && C::WM == 1 && C::KS == 1, "grouped layout");
  static_assert(SFL == 0 || (!PACKED && C::BK == 256), "tiled scales: plain weights, one unit per stage");
  // SG: stages per linear B scale load (plain weights): 2, or 4 when 4
  // divides the stage count (the launcher's choice)
  constexpr bool kQuad = GrQuad<C, D, PACKED, FUSED, SFL, SG>::kB;
  constexpr bool kAQ = GrQuad<C, D, PACKED, FUSED, SFL, SG>::kA;
  static_assert(SG == 2 || (kQuad && D == 2), "scale groups of four: plain weights, linear scales, two slots");
  constexpr int G = kQuad ? 4 : D;  // stages per loop iteration
  static_assert(D % 2 == 0, "A tile double buffer alternates with the stage");
  static_assert(C::BM * C::CH <= C::kThreads, "one A chunk per thread");
  static_assert(PACKED || (C::kSub == 2 && C::KG == 4), "whole-line loads pair the two sub-steps of a 256-K stage");
  static_assert(!PACKED || (C::TN == 2 && C::kSub == 2 && C::MF == 16 && C::kWN == 32), "packed scale chunk layout");
  static_assert(!FUSED || (C::kWaves * 2 * GRegs<C, D>::kAX == C::BM && C::BK == 256),
                "fused quantisation: each wave loads whole rows, two per instruction");
  __shared__ __attribute__((aligned(16))) SmemGR<C> sm;
  const int tiles_n = (int)((p.N + C::BN - 1) / C::BN);
  const int L = xcd_remap(blockIdx.x, tiles_n * p.E);
  const int e = L / tiles_n;
  const int64_t n0 = (int64_t)(L % tiles_n) * C::BN;
  const int64_t lo = p.offsets[e], hi = p.offsets[e + 1];
  if (lo < 0 || hi <= lo || hi > p.rows) return;  // empty or invalid expert
  const int64_t ld = p.K / 2, lds = p.K / 16;
  const float alpha = p.alpha ? p.alpha[e] : 1.0f;
  const float gs_a = FUSED && p.a_gs ? *p.a_gs : 1.0f;
  const int b_rows = (int)min<int64_t>(C::BN, p.N - n0);
  const int n = (int)(p.K / C::BK);
  const uint8_t *bt, *bst;
  uint32_t b_bytes, bs_bytes, b_step, bs_step, b_ld, bs_ld;
  PackedStream ps{nullptr, nullptr, 0, 0};
  if constexpr (PACKED) {
    // stage-major blocks: stage kt of slab s at (kt * slabs + s) * block
    const int64_t slab = (int64_t)e * tiles_n + L % tiles_n, slabs = (int64_t)p.E * tiles_n;
    ps.base = p.b + slab * (C::BN * C::RB);
    ps.sbase = p.b_sf + slab * (C::BN * C::SB);
    ps.stride = slabs * (C::BN * C::RB);
    ps.sstride = slabs * (C::BN * C::SB);
    b_step = bs_step = 0;
    bt = ps.base;
    bst = ps.sbase;
    b_bytes = C::BN * C::RB;
    bs_bytes = C::BN * C::SB;
    b_ld = C::RB;
    bs_ld = C::SB;
  } else {
    b_step = C::RB;
    bs_step = SFL == 0 ? C::SB : SfLayout<SFL>::kUnitStep;
    bt = p.b + ((int64_t)e * p.N + n0) * ld;
    bst = p.b_sf + ((int64_t)e * p.N + n0) * lds;
    b_bytes = (uint32_t)(b_rows * ld);
    bs_bytes = (uint32_t)(b_rows * lds);
    b_ld = (uint32_t)ld;
    bs_ld = (uint32_t)lds;
  }
  const rsrc_t rb = make_rsrc(bt, b_bytes);
  // SFL > 0: the weights' scales are one tiled matrix of E * N rows
  const rsrc_t rbs = SFL == 0 ? make_rsrc(bst, bs_bytes) : SfLayout<SFL>::rsrc(p.b_sf, (int64_t)e * p.N + n0, b_rows, lds);
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wn = wave % C::WN, r_in = lane % C::MF, g = lane / C::MF;
  // per-lane B offsets (row part included; rows >= b_rows masked out of range)
  uint32_t vb[C::TN][C::kSub], vbs[C::TN][C::kSub];
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
    const int row = wn * C::kWN + tn * C::MF + r_in;
#pragma unroll
    for (int s = 0; s < C::kSub; ++s) {
      if constexpr (PACKED) {
        // rows past N are zero in the packed block; the scale chunk of lane
        // 16 g + r_in is (wn * 16 + r_in) * 2 + g / 2
        vb[tn][s] = row < b_rows ? (uint32_t)(((wn * C::TN + tn) * C::kSub + s) * 64 + lane) * 16 : 0x80000000u;
        vbs[tn][s] = (uint32_t)(((wn * 16 + r_in) * 2 + (g >> 1)) * 16);
      } else {
        const int lrow = wn * C::kWN + tn * C::MF + 8 * s + (lane & 7);
        vb[tn][s] = lrow < b_rows ? (uint32_t)(lrow * b_ld + 16 * (lane >> 3)) : 0x80000000u;
        // linear: the bytes this lane row loads of each pair (quad) of stages
        if constexpr (SFL == 0 && kQuad) vbs[tn][s] = row < b_rows ? (uint32_t)(row * bs_ld + 16 * g) : 0x80000000u;
        else if constexpr (SFL == 0) vbs[tn][s] = row < b_rows ? (uint32_t)(row * bs_ld + 8 * (((g & 1) << 1) | (g >> 1))) : 0x80000000u;
        else vbs[tn][s] = row < b_rows ? SfLayout<SFL>::offset((int64_t)e * p.N + n0, row, g, lds) : 0x80000000u;
      }
    }
  }
  const bool lo8 = (lane & 8) == 0;
  typedef GRegs<C, D> RT;
  // this thread's part (ah of kAP) of A code chunk ac of row ar
  const int q = threadIdx.x / RT::kAP, ah = threadIdx.x % RT::kAP, ar = q / C::CH, ac = q % C::CH;
  for (int64_t mc = lo; mc < hi; mc += C::BM) {
    const int rows_c = (int)min<int64_t>(C::BM, hi - mc);
    const int tm_active = (rows_c + C::MF - 1) / C::MF;
    // every row block is computed (the kernel waits on HBM, not on MFMA), so
    // the loop has no per-block branches; rows past the expert load as zero
    // and their outputs are never stored
    rsrc_t ra, ras;
    uint32_t va, vas, vax[RT::kAX];
    if constexpr (FUSED) {
      // the whole activation tensor (T * K * 2 < 2^31 bytes, checked by the
      // host), addressed through each row's token
      ra = make_rsrc(p.x, (uint32_t)(p.T * p.K * 2));
      ras = ra;
#pragma unroll
      for (int i = 0; i < RT::kAX; ++i) {
        const int r = wave * 2 * RT::kAX + 2 * i + (lane >> 5);
        int64_t tok = -1;
        if (r < rows_c) tok = p.row_token ? (int64_t)p.row_token[mc + r] : mc + r;
        vax[i] = tok >= 0 && tok < p.T ? (uint32_t)(tok * p.K * 2 + (lane & 31) * 16) : 0x80000000u;
      }
      va = vas = 0x80000000u;
    } else {
      ra = make_rsrc(p.a + mc * ld, (uint32_t)(rows_c * ld));
      ras = SfLayout<SFL>::rsrc(p.a_sf, mc, rows_c, lds);
      va = ar < rows_c ? (uint32_t)(ar * ld + ac * 16 + ah * (16 / RT::kAP)) : 0x80000000u;
      vas = ar < rows_c ? SfLayout<SFL>::offset(mc, ar, ac >> 1, lds) : 0x80000000u;
      // four stages per load: lane l % 4 of the quad takes stage 4 k + l % 4
      if (kAQ && ar < rows_c) vas += 16 * (threadIdx.x & 3);
#pragma unroll
      for (int i = 0; i < RT::kAX; ++i) vax[i] = 0x80000000u;
    }
    typename C::Acc acc[C::TM][C::TN];
    zero_acc<C>(acc);
    GRegs<C, D> R;
    __syncthreads();  // the previous row chunk is done with both A tiles
    if constexpr (kQuad) gr_load_sq<C, D, kAQ>(R, 0, true, rbs, vbs, bs_step, ras, vas);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      gr_load<C, D, PACKED, FUSED, SFL, SG>(R, u, u, true, ps, rb, rbs, vb, vbs, b_step, bs_step, ra, ras, va, vas, vax);
      __builtin_amdgcn_sched_barrier(0);  // slots are issued in order 0, 1, ...
    }
    // fused: the A tile of stage s + 1 is written during stage s, after the
    // barrier that ends every read of that buffer (stage s - 1), so the
    // quantisation overlaps the other waves' MFMAs instead of holding every
    // wave at the barrier; stage 0's is written here
    if constexpr (FUSED) gr_fused_a<C, D>(R.ax[0], sm.af[0], gs_a, wave, lane);
    for (int i0 = 0; i0 < n; i0 += G) {
#pragma unroll
      for (int v = 0; v < G; ++v) {
        const int u = v % D;
        const int st = i0 + v;  // < n: the launcher picks this kernel only when G divides n
        {
          if constexpr (kQuad) {
            if (v == 0) gr_split_sq<C, D>(R);
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) R.bs[u][tn][0] = R.bsq[tn][v];
          }
          // this stage's A scale word from lane v of the quad
          if constexpr (kAQ) R.as[u] = quad_bcast(R.asq, v);
          uint16_t* af = sm.af[u & 1];
          if constexpr (!FUSED) gr_dequant_a<C, D>(R, u, af, ar, ac, ah);
          // LDS-only barrier: a __syncthreads() fence would also wait for the
          // prefetched loads (loads and stores share one counter)
          lds_barrier();
          gr_compute<C, D, PACKED, SFL, SG>(R, u, af, acc, r_in, g, lo8);
          if constexpr (FUSED) {
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < n) gr_fused_a<C, D>(R.ax[(u + 1) % D], sm.af[(u + 1) & 1], gs_a, wave, lane);
          }
          // keep the reload of slot u after its last reads, so old and new
          // contents share registers (no copies that would wait on the load)
          __builtin_amdgcn_sched_barrier(0);
          // the next four stages' scales, issued before the codes of stage
          // st + D so that waiting for them leaves those codes in flight
          if constexpr (kQuad)
            if (v == G - 1) gr_load_sq<C, D, kAQ>(R, i0 + G, i0 + G < n, rbs, vbs, bs_step, ras, vas);
          gr_load<C, D, PACKED, FUSED, SFL, SG>(R, u, st + D, st + D < n, ps, rb, rbs, vb, vbs, b_step, bs_step, ra, ras,
                                       va, vas, vax);
        }
      }
    }
    store_bf16<C>(acc, tm_active, alpha, p.d + mc * p.N + n0, p.N, rows_c, b_rows);
  }
}

// ---------------------------------------------------------------------------
// Register-streamed K-group GEMM for small and mid M (no LDS staging).  A
// work-group owns one BM x BN output tile and a K range (all of K, or split z
// of S); its KS waves are K-groups: wave w takes the 256-element K units w,
// w + KS, w + 2 KS, ... of the range.  Every lane loads its 16-byte code
// chunks and scale words straight into registers, D units ahead, dequantises
// them and issues 16x16x32 f16 MFMAs on its wave's full tile.  The KS partial
// tiles are summed through LDS in wave order (deterministic); with S > 1 the
// last split to finish sums the S partials in split order.
//
// A unit is 128 bytes of codes per row, one cache line.  Each 16-row block is
// loaded with two instructions that each cover 8 whole lines: lane l reads
// row l % 8 (then row 8 + l % 8), bytes 16 (l / 8) .. 16 (l / 8) + 15.  On a
// cold call the number of outstanding requests per CU is what limits the
// rate, and whole-line requests carry twice the bytes of the half lines a
// 16-row instruction would fetch.  One DPP rotation by 8 lanes within each
// row of 16 then gives lane l = 16 g + r row r with chunks 2 g (words 0..3)
// and 2 g + 1 (words 4..7), K elements 64 g .. 64 g + 63 of the unit; its
// scale word is bytes 4 g .. 4 g + 3 of the row's 16 unit scales.  MFMA t of
// chunk c multiplies elements 8 t .. 8 t + 7 of that chunk, the same K set
// for A and B.
//
// MX tiles (MXFP4: one E8M0 scale per 32 elements) use the same loads and
// exchange and no dequantisation: chunk c of every lane (32 codes, one MX
// block) is the lane's operand of one v_mfma_scale_f32_16x16x128_f8f6f4
// (lane 16 g + r: row r, K block g of the MFMA; its scale operand's low byte
// applies to that row and block; the output layout is that of the 16x16 f16
// MFMA).  Lane 16 g + r loads scale word g / 2 of the row's 8 unit scales;
// bytes 2 g and 2 g + 1 of the unit are those of its chunks.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int KS_, int D_, int OCC_, int MX_ = 0>
struct KCfg {
  static constexpr int BM = BM_, BN = BN_, KS = KS_, D = D_, OCC = OCC_;
  static constexpr bool kMx = MX_ != 0;
  static constexpr int SBLK = kMx ? 32 : 16;        // elements per scale
  static constexpr int TM = BM / 16, TN = BN / 16;
  static constexpr int kThreads = KS * 64;
  static constexpr int kTileFloats = BM * BN;        // one wave's partial tile
  static constexpr int kUnit = 256;                  // K elements per unit
  static_assert(BM % 16 == 0 && BN % 16 == 0, "16-row MFMA blocks");
  static_assert(KS >= 1 && KS <= 16, "waves per work-group");
  static_assert(KS * kTileFloats * 4 <= 65536, "partial tiles fit in 64 KB of LDS");
};

template <class C>
struct KRegs {
  uint32_t aq[C::D][C::TM][8], bq[C::D][C::TN][8];  // two 16-byte code chunks as words
  uint32_t as[C::D][C::TM], bs[C::D][C::TN];        // scale words (4 e4m3)
};

// Loads of unit `unit` into slot u; dead units (past the end of the range)
// read out of range, which returns zero without a memory access, so every
// iteration issues the same loads.
template <class C, int SFL>
__device__ __forceinline__ void kreg_load(KRegs<C>& R, int u, int unit, bool live, const rsrc_t& ra,
                                          const rsrc_t& ras, const rsrc_t& rb, const rsrc_t& rbs,
                                          const uint32_t (&va)[C::TM][2], const uint32_t (&vas)[C::TM],
                                          const uint32_t (&vb)[C::TN][2], const uint32_t (&vbs)[C::TN]) {
  constexpr uint32_t kOut = 0x80000000u;
  const int so = unit * (C::kUnit / 2);
  const int sso = unit * (SFL == 0 ? C::kUnit / C::SBLK : (int)SfLayout<SFL>::kUnitStep);
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u4_t v = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, live ? va[tm][h] : kOut, so, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) R.aq[u][tm][4 * h + j] = v[j];
    }
    R.as[u][tm] = __builtin_amdgcn_raw_buffer_load_b32(ras, live ? vas[tm] : kOut, sso, 0);
  }
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u4_t v = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, live ? vb[tn][h] : kOut, so, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) R.bq[u][tn][4 * h + j] = v[j];
    }
    R.bs[u][tn] = __builtin_amdgcn_raw_buffer_load_b32(rbs, live ? vbs[tn] : kOut, sso, 0);
  }
}

template <class C, int SFL = 0>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gemm_kreg(
    GemmLaunch p) {
  static_assert(SFL == 0 || !C::kMx, "the tiled scale layouts are NVFP4 layouts");
  __shared__ __attribute__((aligned(16))) float red[C::KS * C::kTileFloats];
  __shared__ int last_flag;
  const int tiles_n = (int)p.tiles_n, S = p.splits;
  const int L = xcd_remap(blockIdx.x, (int)(p.tiles_m * p.tiles_n) * S);
  const int tile = L / S, z = L % S;
  const int64_t m0 = (int64_t)(tile / tiles_n) * C::BM, n0 = (int64_t)(tile % tiles_n) * C::BN;
  const int64_t ld = p.K / 2, lds = p.K / C::SBLK;
  const int rows_a = (int)min<int64_t>(C::BM, p.M - m0), rows_b = (int)min<int64_t>(C::BN, p.N - n0);
  const rsrc_t ra = make_rsrc(p.a + m0 * ld, (uint32_t)(rows_a * ld));
  const rsrc_t ras = SfLayout<SFL>::rsrc(p.a_sf, m0, rows_a, lds);
  const rsrc_t rb = make_rsrc(p.b + n0 * ld, (uint32_t)(rows_b * ld));
  const rsrc_t rbs = SfLayout<SFL>::rsrc(p.b_sf, n0, rows_b, lds);
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int r_in = lane & 15, g = lane >> 4;
  // code offsets: rows lane % 8 and 8 + lane % 8 of each 16-row block, bytes
  // 16 (lane / 8) of the unit; scale word g (MX: g / 2) of row r_in
  const int sw = C::kMx ? 4 * (g >> 1) : 4 * g;
  uint32_t va[C::TM][2], vas[C::TM], vb[C::TN][2], vbs[C::TN];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = tm * 16 + 8 * h + (lane & 7);
      va[tm][h] = r < rows_a ? (uint32_t)(r * ld + 16 * (lane >> 3)) : 0x80000000u;
    }
    const int r = tm * 16 + r_in;
    if constexpr (SFL == 0) vas[tm] = r < rows_a ? (uint32_t)(r * lds + sw) : 0x80000000u;
    else vas[tm] = r < rows_a ? SfLayout<SFL>::offset(m0, r, g, lds) : 0x80000000u;
  }
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = tn * 16 + 8 * h + (lane & 7);
      vb[tn][h] = r < rows_b ? (uint32_t)(r * ld + 16 * (lane >> 3)) : 0x80000000u;
    }
    const int r = tn * 16 + r_in;
    if constexpr (SFL == 0) vbs[tn] = r < rows_b ? (uint32_t)(r * lds + sw) : 0x80000000u;
    else vbs[tn] = r < rows_b ? SfLayout<SFL>::offset(n0, r, g, lds) : 0x80000000u;
  }
  // this work-group's K units [u_lo, u_hi): all of K, or split z of S
  const int nu_all = (int)(p.K / C::kUnit);
  const int u_lo = (int)((int64_t)z * nu_all / S), u_hi = (int)((int64_t)(z + 1) * nu_all / S);
  const int nu = u_hi - u_lo;
  // every wave runs the same number of iterations (a multiple of D); units
  // past the end are dead
  const int per_wave = (nu + C::KS - 1) / C::KS;
  const int iters = (per_wave + C::D - 1) / C::D * C::D;
  Mfma<16>::Acc acc[C::TM][C::TN];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = Mfma<16>::Acc{0.f, 0.f, 0.f, 0.f};
  KRegs<C> R;
#pragma unroll
  for (int u = 0; u < C::D; ++u) {
    const int unit = wave + u * C::KS;
    kreg_load<C, SFL>(R, u, u_lo + unit, unit < nu, ra, ras, rb, rbs, va, vas, vb, vbs);
    __builtin_amdgcn_sched_barrier(0);
  }
  const bool lo8 = (lane & 8) == 0;
  for (int i0 = 0; i0 < iters; i0 += C::D) {
#pragma unroll
    for (int u = 0; u < C::D; ++u) {
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) kreg_exchange(R.aq[u][tm], lo8);
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) kreg_exchange(R.bq[u][tn], lo8);
      if constexpr (C::kMx) {
        typedef int v8i_t __attribute__((ext_vector_type(8)));
        const int ssh = 16 * (g & 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          v8i_t bv[C::TN];
          int sb[C::TN];
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            const uint32_t* w = R.bq[u][tn] + 4 * c;
            bv[tn] = v8i_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
            sb[tn] = (int)(R.bs[u][tn] >> (ssh + 8 * c));
          }
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm) {
            const uint32_t* w = R.aq[u][tm] + 4 * c;
            const v8i_t av = v8i_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
            const int sa = (int)(R.as[u][tm] >> (ssh + 8 * c));
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn)
              acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[tn], acc[tm][tn], 4, 4, 0, sa, 0,
                                                                             sb[tn]);
          }
        }
      } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        h2_t asp[C::TM], bsp[C::TN];
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) asp[tm] = e4m3x2_to_h2(R.as[u][tm] >> (16 * c));
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bsp[tn] = e4m3x2_to_h2(R.bs[u][tn] >> (16 * c));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          h8_t bf[C::TN];
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) bf[tn] = dequant8(R.bq[u][tn][4 * c + t], scale_pair(bsp[tn], t >> 1));
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm) {
            const h8_t af = dequant8(R.aq[u][tm][4 * c + t], scale_pair(asp[tm], t >> 1));
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = Mfma<16>::run(af, bf[tn], acc[tm][tn]);
          }
        }
      }
      }
      // the slot's reload stays after its last reads (old and new contents
      // share registers; no copies that would wait on the load)
      __builtin_amdgcn_sched_barrier(0);
      const int unit = wave + (i0 + u + C::D) * C::KS;
      kreg_load<C, SFL>(R, u, u_lo + unit, unit < nu, ra, ras, rb, rbs, va, vas, vb, vbs);
    }
  }
  // K-group sum: wave w's partial tile at red[w][.], element (tm, tn, lane, j)
  // at ((tm * TN + tn) * 64 + lane) * 4 + j
  float* mine = red + wave * C::kTileFloats;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) *(f4_t*)(mine + ((tm * C::TN + tn) * 64 + lane) * 4) = acc[tm][tn];
  __syncthreads();
  const float alpha = p.alpha ? *p.alpha : 1.0f;
  // the work-group's tile, row-major, columns fastest (contiguous stores)
  const rsrc_t part = partial_rsrc(p.ws + kCounterBytes / 4 + (int64_t)tile * S * C::kTileFloats, S, C::kTileFloats);
  for (int x = threadIdx.x; x < C::kTileFloats; x += C::kThreads) {
    const int row = x / C::BN, col = x % C::BN;
    const int rr = row & 15, cc = col & 15;
    const int idx = (((row >> 4) * C::TN + (col >> 4)) * 64 + (rr >> 2) * 16 + cc) * 4 + (rr & 3);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < C::KS; ++w) sum += red[w * C::kTileFloats + idx];
    if (S > 1) store_coherent(part, (uint32_t)(z * C::kTileFloats + x) * 4, sum);
    else if (row < rows_a && col < rows_b) p.d[(m0 + row) * p.N + n0 + col] = f32_to_bf16_bits(alpha * sum);
  }
  if (S == 1) return;
  // split K: publish the partial, count arrivals, the last split sums all S
  // partials in split order and stores bf16 (then resets the counter)
  int* counter = (int*)p.ws + tile;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) last_flag = count_arrival(counter, S);
  __syncthreads();
  if (!last_flag) return;
  for (int x = threadIdx.x; x < C::kTileFloats; x += C::kThreads) {
    const int row = x / C::BN, col = x % C::BN;
    float sum = 0.f;
    for (int zz = 0; zz < S; ++zz) sum += load_coherent(part, (uint32_t)(zz * C::kTileFloats + x) * 4);
    if (row < rows_a && col < rows_b) p.d[(m0 + row) * p.N + n0 + col] = f32_to_bf16_bits(alpha * sum);
  }
  if (threadIdx.x == 0) reset_counter(counter);
}

// ---------------------------------------------------------------------------
// Plans and launchers.
// ---------------------------------------------------------------------------
typedef Cfg<256, 256, 2, 2, 32, 128, 4> CfgTile256;     // large M and N: 128x128 wave tiles
typedef Cfg<128, 128, 2, 2, 32, 128, 4, 0, 1, 2> CfgTile128;  // mid-large shapes (split-K)
typedef Cfg<64, 64, 2, 2, 32, 128, 6, 0, 1, 2> CfgTile64;      // mid shapes (split-K)
typedef Cfg<16, 64, 1, 4, 16, 128, 8, 0, 1, 3> CfgSkinny16;    // decode (split-K)
typedef Cfg<32, 64, 1, 4, 16, 128, 6, 0, 1, 3> CfgSkinny32;    // decode (split-K)
typedef Cfg<64, 64, 1, 4, 16, 128, 6, 0, 1, 2> CfgSkinny64;    // decode (split-K)
typedef Cfg<256, 256, 2, 4, 32, 128, 4> CfgTile256w8;   // large: 8 waves of 128x64 (2 per SIMD)
typedef Cfg<256, 256, 2, 2, 32, 128, 4, 4> CfgTile256il; // large, MFMA/VALU interleave hint
typedef Cfg<128, 128, 2, 2, 32, 128, 4, 4, 1, 2> CfgTile128il;  // mid-large, interleave hint
typedef Cfg<64, 64, 1, 1, 32, 256, 2, 0, 4, 4> CfgTile64k4;  // mid: 4 K-groups of one 64x64 wave
// register-streamed K-group tiles: 4 waves, 2 or 3 units in flight per wave
typedef KCfg<16, 16, 4, 3, 4> KReg16x16;
typedef KCfg<32, 16, 4, 3, 4> KReg32x16;
typedef KCfg<32, 32, 4, 3, 2> KReg32x32;
typedef KCfg<64, 32, 4, 2, 2> KReg64x32;
// MXFP4 register-streamed tiles (scaled FP4 MFMA, no dequantisation)
typedef KCfg<16, 16, 4, 3, 4, 1> MxReg16x16;
typedef KCfg<32, 16, 4, 3, 4, 1> MxReg32x16;
typedef KCfg<32, 32, 4, 3, 2, 1> MxReg32x32;
typedef KCfg<64, 32, 4, 2, 2, 1> MxReg64x32;
// 256 K per stage (each row's codes one 128-byte line), 2 stages; the
// 256x256 and 256x192 tiles of this kind are in gemm_large.hip
typedef Cfg<128, 128, 2, 2, 32, 256, 2, 0, 1, 2> CfgTile128k256;    // 4 waves of 64x64
// the same tiles on scales in the 8 x 4 tiled layout (nvfp4_gemm_sf)
typedef Cfg<64, 64, 1, 1, 32, 256, 2, 0, 4, 4, 16, 0, 2> CfgTile64k4Sf8;
typedef Cfg<128, 128, 2, 2, 32, 256, 2, 0, 1, 2, 16, 0, 2> CfgTile128k256Sf8;
// MXFP4 tiles (E8M0 scale per 32 elements, scaled FP4 MFMA)
typedef Cfg<256, 256, 2, 2, 32, 256, 2, 0, 1, 1, 32> CfgMx256;      // 4 waves x 128x128, 136 KB LDS
typedef Cfg<128, 128, 2, 2, 32, 256, 2, 0, 1, 2, 32, 2> CfgMx128;   // 4 waves x 64x64, 68 KB (split-K), waves 0-1 load
                                                                     // (1024 x 6144 x 6144: 45.1 -> 42.0 us)
typedef Cfg<64, 64, 2, 2, 32, 256, 3, 0, 1, 2, 32> CfgMx64;         // 4 waves x 32x32 (split-K)
// The 8-wave MX tiles issue each stage's loads from waves 0-3 only (one wave
// per SIMD): the other four start their LDS reads and MFMAs at once instead
// of waiting on the memory pipeline too (8192 x 6144 x 6144: 179.6 -> 172.0
// us, 4096 x 6144 x 6144 on 256x192 tiles: 105.8 -> 98.9 us; bitwise the
// same).  The NVFP4 256-row tiles do the same (gemm_large.hip); on the
// NVFP4 K-group tile it made no difference.
typedef Cfg<256, 256, 2, 4, 32, 256, 2, 0, 1, 2, 32, 4> CfgMx256w8;    // 8 waves x 128x64
typedef Cfg<256, 256, 2, 4, 32, 128, 4, 0, 1, 2, 32> CfgMx256w8s4;     // all waves load, 4 stages of 128
typedef Cfg<256, 192, 4, 2, 32, 256, 2, 0, 1, 2, 32, 4> CfgMx256x192;  // 8 waves x 64x96, 119 KB
typedef Cfg<64, 256, 1, 8, 16, 256, 3> CfgGrouped;      // MoE experts: <= 64 rows per pass
static_assert(CfgGrouped::WM == 1, "grouped row-block count assumes one wave row");
typedef Cfg<32, 256, 1, 8, 16, 256, 3> CfgGroupedA16;   // MoE experts, shared f16 A: <= 32 rows per pass
typedef Cfg<32, 256, 1, 8, 16, 256, 2, 0, 1, 4> CfgGroupedReg;  // MoE experts, B streamed through registers: 2 WGs per CU
typedef Cfg<64, 256, 1, 8, 16, 256, 2, 0, 1, 2> CfgGroupedReg64;  // the same with 64-row passes over each expert
typedef Cfg<32, 256, 1, 8, 16, 256, 2, 0, 1, 4> CfgGroupedRegF;  // 32-row passes quantising A on load: 2 WGs per CU

struct PlanKind {
  const char* name;
  int bm, bn, bk;
  bool splitk;
  bool kreg;  // register-streamed K-group kernel
  bool mx;    // MXFP4 tile
  int ks;     // K-groups (waves) of a register-streamed or K-group LDS tile
  int d;      // register-streamed tiles: K units in flight per wave
};
static const PlanKind kKinds[] = {
    {"tile256x256_mfma32", 256, 256, 128, false},
    {"tile128x128_mfma32", 128, 128, 128, true},
    {"tile64x64_mfma32", 64, 64, 128, true},
    {"skinny16x64_mfma16", 16, 64, 128, true},
    {"skinny32x64_mfma16", 32, 64, 128, true},
    {"skinny64x64_mfma16", 64, 64, 128, true},
    {"tile256x256w8_mfma32", 256, 256, 128, false},
    {"tile256x256il_mfma32", 256, 256, 128, false},
    {"tile128x128il_mfma32", 128, 128, 128, true},
    {"tile64x64k4_mfma32", 64, 64, 256, true, false, false, 4},
    {"kreg16x16_mfma16", 16, 16, 256, true, true, false, KReg16x16::KS, KReg16x16::D},
    {"kreg32x16_mfma16", 32, 16, 256, true, true, false, KReg32x16::KS, KReg32x16::D},
    {"kreg32x32_mfma16", 32, 32, 256, true, true, false, KReg32x32::KS, KReg32x32::D},
    {"kreg64x32_mfma16", 64, 32, 256, true, true, false, KReg64x32::KS, KReg64x32::D},
    {"tile256x256w8k256_mfma32", 256, 256, 256, false},
    {"tile128x128k256_mfma32", 128, 128, 256, true},
    {"tile256x192w8k256_mfma32", 256, 192, 256, false},
};
static const PlanKind kMxKinds[] = {
    {"mx256x256_fp4mfma", 256, 256, 256, false, false, true},
    {"mx128x128_fp4mfma", 128, 128, 256, true, false, true},
    {"mx64x64_fp4mfma", 64, 64, 256, true, false, true},
    {"mx256x256w8_fp4mfma", 256, 256, 256, false, false, true},
    {"mx256x256w8s4_fp4mfma", 256, 256, 128, false, false, true},
    {"mxreg16x16_fp4mfma", 16, 16, 256, true, true, true, MxReg16x16::KS, MxReg16x16::D},
    {"mxreg32x16_fp4mfma", 32, 16, 256, true, true, true, MxReg32x16::KS, MxReg32x16::D},
    {"mxreg32x32_fp4mfma", 32, 32, 256, true, true, true, MxReg32x32::KS, MxReg32x32::D},
    {"mxreg64x32_fp4mfma", 64, 32, 256, true, true, true, MxReg64x32::KS, MxReg64x32::D},
    {"mx256x192w8_fp4mfma", 256, 192, 256, false, false, true},
};
static constexpr int kNumMxKinds = (int)(sizeof(kMxKinds) / sizeof(kMxKinds[0]));
static constexpr int kNumKinds = (int)(sizeof(kKinds) / sizeof(kKinds[0]));

static const int kCUs = 256;
static_assert(kCounterBytes / 4 >= kCUs, "split-K runs only below kCUs tiles");
static const int64_t kMaxPartialBytesPerTile = 256 * 1024;  // one CU reduces a tile

static const int64_t kTargetBlocks = 384;   // 1.5 work-groups per CU
static const int64_t kK4Blocks = 768;  // K-group LDS tiles: target work-groups
static const int64_t kMinStagesPerSplit = 6;
static const int64_t kMxTargetBlocks = 576;  // MX LDS tiles: target work-groups

// Forced plans (nvfp4_force_plan; tuning sweeps and tests): per operation
// family, 0 = none, else (kind + 1) | splits << 16, one word so that kind and
// splits are always read together.
static std::atomic<int> g_forced[kForceFamilies];

void set_forced_plan(int family, int kind, int splits) {
  g_forced[family].store(kind < 0 ? 0 : (kind + 1) | ((splits < 0 ? 0 : splits) << 16));
}

static bool forced_plan(int family, int* kind, int* splits) {
  const int v = g_forced[family].load();
  if (v == 0) return false;
  *kind = (v & 0xFFFF) - 1;
  *splits = v >> 16;
  return true;
}

static void plan_splits(GemmPlan& pl, const PlanKind& k, int64_t K, int forced) {
  const int64_t tiles = pl.tiles_m * pl.tiles_n;
  const int64_t nk = K / k.bk;
  int64_t s = 1;
  const bool kgroup_lds = k.ks > 1 && !k.kreg;
  const bool can_split = k.splitk && (tiles < kCUs || (kgroup_lds && tiles < 2 * kCUs) ||
                                      (forced > 1 && tiles <= kCounterBytes / 4));
  if (can_split) {
    if (forced > 0) {
      s = forced;
    } else if (k.kreg) {
      // register K-group tiles: the fewest splits that let every wave hold
      // all its K units in flight at once (one memory round trip, ks * d
      // units per work-group), at most one work-group per CU.  Each further
      // round trip costs about 2 us on cold operands and a split exchange
      // about 1.4 (cold sweeps, 16 x 768: K = 2048 4.7 us unsplit against 6.2
      // split in two; K = 6144 7.0 split in two against 7.4 unsplit and 7.3
      // in three; K = 12288 8.1 in four against 9.1 in two and 11.5 unsplit;
      // 16 x 2048 x 12288, 128 tiles: 9.3 in two against 10.3 in four)
      const int64_t per_wg = (int64_t)k.ks * k.d;
      s = (nk + per_wg - 1) / per_wg;
      while (s > 1 && tiles * s > kCUs) --s;
    } else if (kgroup_lds) {
      // K-group LDS tiles: about three work-groups per CU, at most 5 splits
      // (cold sweeps at K = 6144: 1024 x 768, 192 tiles, 19.7 us at 4 splits
      // against 23.3 unsplit and 20.7 / 22.4 at 3 / 6; 512 x 768, 96 tiles,
      // 14.2 us at 5 against 15.4 / 15.6 at 6 / 8; 256 x 768, 48 tiles, 12.4
      // us at 5 against 13.1 at 8; 2048 x 768, 384 tiles, 28.5 against 29.3)
      s = kK4Blocks / tiles;
      if (s > 5) s = 5;
    } else if (k.mx) {
      // MX LDS tiles: about two work-groups per CU, at least 6 stages per
      // split (cold sweeps at K = 6144: 1024 x 768, 192 tiles of 64x64, 16.6
      // us at 3 splits against 20.7 unsplit; 512 x 768, 96 tiles, 12.6 at 4
      // against 15.3 at 2; 256 x 2048, 128 tiles, 14.8 at 4)
      s = kMxTargetBlocks / tiles;
      if (s > nk / kMinStagesPerSplit) s = nk / kMinStagesPerSplit;
    } else {
      s = (kTargetBlocks + tiles - 1) / tiles;
      int64_t cap = kMaxPartialBytesPerTile / ((int64_t)k.bm * k.bn * 4);
      if (cap > nk / kMinStagesPerSplit) cap = nk / kMinStagesPerSplit;
      if (s > cap) s = cap;
    }
    if (s > kMaxSplits) s = kMaxSplits;
    if (s > nk) s = nk;
    if (s < 1) s = 1;
  }
  pl.splits = (int)s;
  pl.workspace = 0;
  if (s > 1) {
    // fixed counter block first (same offsets for every shape, so counters a
    // completed call leaves at zero stay valid for any later shape), partials after
    const size_t part = (size_t)tiles * (size_t)s * (size_t)k.bm * (size_t)k.bn * sizeof(float);
    pl.workspace = kCounterBytes + part;
  }
}

// Plan choice, from sweeps on MI355X of the pages' shapes (K = 6144,
// N = 768 / 2048 / 6144; cold below M = 4096, warm above): up to M = 128,
// the register-streamed K-group tile (4 waves per work-group), the smallest
// of 16x16, 32x16, 32x32, 64x32 that needs at most one work-group per CU;
// above that, 64x64 K-group tiles split K about three work-groups per CU
// (256 x 768: 12.4 us against 13.2 for the 32x32 register tile; 512 x 768:
// 14.2 against 19.7 for the 64x32 one) until 128x128 tiles fill the CUs
// three times, then 128x128 tiles,
// and tiles of 8 waves, 256x256 or 256x192, once either fills the CUs twice
// (all staging 256 K per stage: whole 128-byte lines per row).
GemmPlan choose_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan pl;
  int kind = -1;
  int forced_splits = 0;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t t192 = ((M + 255) / 256) * ((N + 191) / 192);
  if (M <= 128) {
    // 16x16, 32x16, 32x32; the 64x32 register tile (13) lost to the split
    // 64x64 K-group tile wherever it was the first fit (64 x 6144 x 6144:
    // 20.0 us against 16.6; 64 x 8192: 20.2 against 19.6)
    static const int kreg_kinds[] = {10, 11, 12};
    for (int kk : kreg_kinds) {
      const PlanKind& k = kKinds[kk];
      if (((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) <= kCUs) {
        kind = kk;
        break;
      }
    }
    // wide weights at M <= 32: 32x32 register tiles, up to four work-groups
    // per CU, unsplit (16 x 16384 x 6144: 21.1 us against 28.2 for the
    // skinny LDS tile; 32 x 16384: 23.8 against 35.4)
    if (kind < 0 && M <= 32 && ((N + 31) / 32) <= 4 * kCUs) kind = 12;
  }
  if (kind < 0 && M > 64 && (t256 >= 2 * kCUs || t192 >= 2 * kCUs)) {
    // 256x256 or 256x192 tiles, one work-group per CU: the 192-column tile
    // when its rounds of 256 work-groups cover less tile area (its 64x96
    // wave tiles cost about 5% more dequantisation per MFMA)
    const int64_t r256 = (t256 + kCUs - 1) / kCUs, r192 = (t192 + kCUs - 1) / kCUs;
    if (r192 * 192 * 105 < r256 * 256 * 100) kind = 16;
    else if (t256 >= 2 * kCUs) kind = 14;
  } else if (kind < 0 && M > 64 && t192 % kCUs == 0 && t192 > 0) {
    // exactly one round of 256x192 tiles (2048 x 6144 x 6144: 142 us against
    // 155 for 128x128 tiles; at 1.5 rounds, 3072 x 6144, the 128x128 tiles
    // win: 237 us against 257)
    kind = 16;
  }
  if (kind < 0) {
    // (the skinny split-K LDS tiles, kinds 3 and 4, lost to these at every
    // M <= 64 measured: 64 x 16384 x 6144 on the split 64x64 K-group tile
    // 26.8 us against 44.2)
    if (t128 >= 3 * kCUs && M > 64) kind = 15;
    else kind = 9;
  }
  // a plan forced by nvfp4_force_plan (tuning sweeps and tests only)
  int fk = -1, fs = 0;
  if (forced_plan(kForceGemm, &fk, &fs) && fk < kNumKinds) {
    kind = fk;
    forced_splits = fs;
  }
  const PlanKind& k = kKinds[kind];
  pl.kind = kind;
  pl.name = k.name;
  pl.tiles_m = (M + k.bm - 1) / k.bm;
  pl.tiles_n = (N + k.bn - 1) / k.bn;
  pl.group_m = 8;
  if (!k.splitk || pl.tiles_m * pl.tiles_n > kCounterBytes / 4) forced_splits = 1;
  plan_splits(pl, k, K, forced_splits);
  return pl;
}

bool plan_reads_tiled_scales(const GemmPlan& plan, int sf_layout) {
  if (plan.kind >= 10 && plan.kind <= 13) return true;  // register tiles: both layouts
  return sf_layout == 2 && (plan.kind == 9 || plan.kind == 14 || plan.kind == 15 || plan.kind == 16);
}

template <class C>
static void launch_kreg(const GemmPlan& pl, const GemmLaunch& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(pl.tiles_m * pl.tiles_n * pl.splits);
  if constexpr (!C::kMx) {
    if (p.sf_layout == 1) {
      hipLaunchKernelGGL((k_gemm_kreg<C, 1>), dim3(grid), dim3(C::kThreads), 0, stream, p);
      return;
    }
    if (p.sf_layout == 2) {
      hipLaunchKernelGGL((k_gemm_kreg<C, 2>), dim3(grid), dim3(C::kThreads), 0, stream, p);
      return;
    }
  }
  hipLaunchKernelGGL((k_gemm_kreg<C, 0>), dim3(grid), dim3(C::kThreads), 0, stream, p);
}

template <class C, bool SPLITK>
static void launch_one(const GemmPlan& pl, const GemmLaunch& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(pl.tiles_m * pl.tiles_n * pl.splits);
  hipLaunchKernelGGL((k_gemm<C, SPLITK>), dim3(grid), dim3(C::kThreads), 0, stream, p);
}

hipError_t launch_gemm(const GemmPlan& pl, GemmLaunch p, hipStream_t stream) {
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.splits = pl.splits;
  p.group_m = pl.group_m;
  if (p.sf_layout == 2 && pl.kind != 10 && pl.kind != 11 && pl.kind != 12 && pl.kind != 13) {
    // 8 x 4 scales read by the LDS tiles (plan_reads_tiled_scales)
    if (pl.kind == 9) launch_one<CfgTile64k4Sf8, true>(pl, p, stream);
    else if (pl.kind == 15) launch_one<CfgTile128k256Sf8, true>(pl, p, stream);
    else launch_large_tile(pl.kind, p, (unsigned)(pl.tiles_m * pl.tiles_n), stream);
    return hipGetLastError();
  }
  switch (pl.kind) {
    case 0: launch_one<CfgTile256, false>(pl, p, stream); break;  // plan keeps splits == 1
    case 1: launch_one<CfgTile128, true>(pl, p, stream); break;
    case 2: launch_one<CfgTile64, true>(pl, p, stream); break;
    case 3: launch_one<CfgSkinny16, true>(pl, p, stream); break;
    case 4: launch_one<CfgSkinny32, true>(pl, p, stream); break;
    case 5: launch_one<CfgSkinny64, true>(pl, p, stream); break;
    case 6: launch_one<CfgTile256w8, false>(pl, p, stream); break;
    case 7: launch_one<CfgTile256il, false>(pl, p, stream); break;
    case 8: launch_one<CfgTile128il, true>(pl, p, stream); break;
    case 10: launch_kreg<KReg16x16>(pl, p, stream); break;
    case 11: launch_kreg<KReg32x16>(pl, p, stream); break;
    case 12: launch_kreg<KReg32x32>(pl, p, stream); break;
    case 13: launch_kreg<KReg64x32>(pl, p, stream); break;
    case 14: launch_large_tile(14, p, (unsigned)(pl.tiles_m * pl.tiles_n), stream); break;  // splits == 1
    case 15: launch_one<CfgTile128k256, true>(pl, p, stream); break;
    case 16: launch_large_tile(16, p, (unsigned)(pl.tiles_m * pl.tiles_n), stream); break;  // splits == 1
    default: launch_one<CfgTile64k4, true>(pl, p, stream); break;
  }
  return hipGetLastError();
}

// MXFP4 plan, from cold sweeps at K = 6144: up to M = 512 the register tile
// (the same rule as for NVFP4: the smallest of 16x16, 32x16, 32x32, 64x32
// with at most one work-group per CU); else 256x256 tiles of 8 waves while
// they fill the CUs, then 128x128 (two work-groups per CU) while those fill
// them, else 64x64 with split-K up to about 1.5 work-groups per CU.
// nvfp4_force_plan can force one (tuning sweeps and tests only).
GemmPlan choose_mx_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan pl;
  int kind = -1, forced_splits = 0;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256), t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (M <= 128) {
    // register tiles 16x16, 32x16, 32x32, 64x32; above M = 128 the split
    // 64x64 LDS tile is faster (512 x 768 x 6144: 12.6 us against 17.1 for
    // the 64x32 register tile; 256 x 768: 11.3 against 12.0 for 32x32)
    for (int kk = 5; kk <= 8; ++kk) {
      const PlanKind& k = kMxKinds[kk];
      if (((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) <= kCUs) {
        kind = kk;
        break;
      }
    }
  }
  if (kind < 0) {
    // 256x192 tiles when they fill the CUs twice and their rounds of 256
    // work-groups cover less tile area than 256x256 tiles (its 64x96 wave
    // tiles read about 11% more LDS bytes per MFMA)
    const int64_t t192 = ((M + 255) / 256) * ((N + 191) / 192);
    const int64_t r256 = (t256 + kCUs - 1) / kCUs, r192 = (t192 + kCUs - 1) / kCUs;
    if (t192 >= 2 * kCUs && r192 * 192 * 112 < r256 * 256 * 100) kind = 9;
    // 256x256 tiles from three quarters of a round (2048 x 6144 x 6144, 192
    // tiles: 63.0 us against 76.2 for 128x128 tiles)
    else kind = 4 * t256 >= 3 * kCUs ? 3 : (t128 >= kCUs ? 1 : 2);
  }
  int fk = -1, fs = 0;
  if (forced_plan(kForceMx, &fk, &fs) && fk < kNumMxKinds) {
    kind = fk;
    forced_splits = fs;
  }
  const PlanKind& k = kMxKinds[kind];
  pl.kind = kind;
  pl.name = k.name;
  pl.tiles_m = (M + k.bm - 1) / k.bm;
  pl.tiles_n = (N + k.bn - 1) / k.bn;
  pl.group_m = 8;
  if (!k.splitk || pl.tiles_m * pl.tiles_n >= kCUs) forced_splits = 1;
  plan_splits(pl, k, K, forced_splits);
  return pl;
}

hipError_t launch_mx_gemm(const GemmPlan& pl, GemmLaunch p, hipStream_t stream) {
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.splits = pl.splits;
  p.group_m = pl.group_m;
  switch (pl.kind) {
    case 0: launch_one<CfgMx256, false>(pl, p, stream); break;
    case 1: launch_one<CfgMx128, true>(pl, p, stream); break;
    case 3: launch_one<CfgMx256w8, false>(pl, p, stream); break;
    case 4: launch_one<CfgMx256w8s4, false>(pl, p, stream); break;
    case 9: launch_one<CfgMx256x192, false>(pl, p, stream); break;
    case 5: launch_kreg<MxReg16x16>(pl, p, stream); break;
    case 6: launch_kreg<MxReg32x16>(pl, p, stream); break;
    case 7: launch_kreg<MxReg32x32>(pl, p, stream); break;
    case 8: launch_kreg<MxReg64x32>(pl, p, stream); break;
    default: launch_one<CfgMx64, true>(pl, p, stream); break;
  }
  return hipGetLastError();
}

// The host sees only the total row count: experts averaging more than 40
// rows get 64-row passes.
static void grouped_forced(int* gk) {
  int fk = -1, fs = 0;
  if (forced_plan(kForceGrouped, &fk, &fs) && fk <= 3) *gk = fk;
}

static bool tall_experts(const GroupedLaunch& p) { return p.rows > 40 * (int64_t)p.E; }

hipError_t launch_grouped(GroupedLaunch p, int32_t* status, hipStream_t stream, bool compute) {
  if (status) {
    hipLaunchKernelGGL(k_check_offsets, dim3(1), dim3(64), 0, stream, p.offsets, p.E, p.rows, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!compute) return hipSuccess;
  // Kernel choice, measured on the 256-expert top-8 workload and on uniform
  // 16/32/64-row experts (K = 6144): B streamed through registers (2 stages
  // ahead) when 2 divides K / 256, else the shared-f16-A kernel.  The
  // register kernel takes 32-row passes over each expert (4 waves per SIMD);
  // when the experts average more than 40 rows, 64-row passes (2 waves per
  // SIMD, but every weight byte read once for up to 64 rows) are faster.
  // nvfp4_force_plan can force the per-wave-dequant, shared-f16-A, 32-row
  // or 64-row register kernel (kinds 0..3; tuning and tests only).
  int gk = (p.K / 256) % 2 == 0 ? (tall_experts(p) ? 3 : 2) : 1;
  grouped_forced(&gk);
  if (gk >= 2 && (p.K / 256) % 2) gk = 1;
  if (p.sf_layout != 0) {
    // tiled scales (K % 512 == 0, checked by the API): the register kernels
    if (gk < 2) gk = 2;
    const bool tall = gk == 3;
    const unsigned bn = tall ? CfgGroupedReg64::BN : CfgGroupedReg::BN;
    const dim3 grid((unsigned)((p.N + bn - 1) / bn) * (unsigned)p.E);
    if (tall && p.sf_layout == 1)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false, false, 1>), grid, dim3(CfgGroupedReg64::kThreads), 0, stream, p);
    else if (tall)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false, false, 2>), grid, dim3(CfgGroupedReg64::kThreads), 0, stream, p);
    else if (p.sf_layout == 1)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg, 2, false, false, 1>), grid, dim3(CfgGroupedReg::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg, 2, false, false, 2>), grid, dim3(CfgGroupedReg::kThreads), 0, stream, p);
    return hipGetLastError();
  }
  if (gk == 0) {
    const unsigned tiles_n = (unsigned)((p.N + CfgGrouped::BN - 1) / CfgGrouped::BN);
    hipLaunchKernelGGL(k_grouped<CfgGrouped>, dim3(tiles_n * (unsigned)p.E), dim3(CfgGrouped::kThreads), 0, stream,
                       p);
  } else if (gk == 2) {
    // linear scales four stages per load when 4 divides K / 256, else two
    const unsigned tiles_n = (unsigned)((p.N + CfgGroupedReg::BN - 1) / CfgGroupedReg::BN);
    if ((p.K / CfgGroupedReg::BK) % 4 == 0)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg, 2, false, false, 0, 4>), dim3(tiles_n * (unsigned)p.E),
                         dim3(CfgGroupedReg::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg, 2, false>), dim3(tiles_n * (unsigned)p.E),
                         dim3(CfgGroupedReg::kThreads), 0, stream, p);
  } else if (gk == 3) {
    const unsigned tiles_n = (unsigned)((p.N + CfgGroupedReg64::BN - 1) / CfgGroupedReg64::BN);
    if ((p.K / CfgGroupedReg64::BK) % 4 == 0)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false, false, 0, 4>), dim3(tiles_n * (unsigned)p.E),
                         dim3(CfgGroupedReg64::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false>), dim3(tiles_n * (unsigned)p.E),
                         dim3(CfgGroupedReg64::kThreads), 0, stream, p);
  } else {
    const unsigned tiles_n = (unsigned)((p.N + CfgGroupedA16::BN - 1) / CfgGroupedA16::BN);
    hipLaunchKernelGGL(k_grouped_a16<CfgGroupedA16>, dim3(tiles_n * (unsigned)p.E), dim3(CfgGroupedA16::kThreads),
                       0, stream, p);
  }
  return hipGetLastError();
}

// Weight pre-pack for the grouped GEMM: [E][N][K/2] codes and [E][N][K/16]
// scales -> per (expert, 256-row slab, 256-element K stage) one contiguous
// block of 256 rows x 128 code bytes (and 256 x 16 scale bytes), rows past N
// zero, blocks ordered by stage, then expert, then slab: the work-groups on
// the chip at one time walk neighbouring blocks, which streams faster from
// HBM than each reading its own slab's run.  Inside a code block the 16-byte chunks are in the order the grouped
// kernel's lanes load them (wave, column block, sub-step, lane), so each load
// instruction reads 1 KB in one run; a scale block holds each lane's four
// scale words in one 16-byte chunk (packed_sf_word).  One 16-byte source chunk
// per thread and step.
constexpr int kPackRows = CfgGroupedReg::BN, kPackK = CfgGroupedReg::BK;
static_assert(CfgGroupedReg64::BN == kPackRows && CfgGroupedReg64::kWN == CfgGroupedReg::kWN &&
                  CfgGroupedReg64::TN == CfgGroupedReg::TN && CfgGroupedReg64::BK == kPackK,
              "both packed kernels share one layout");

// position of chunk c (0..7) of row r (0..255) inside a packed code block
__host__ __device__ constexpr int packed_chunk(int r, int c) {
  typedef CfgGroupedReg G;
  return (((r / G::kWN) * G::TN + (r % G::kWN) / G::MF) * G::kSub + c / G::KG) * 64 + (c % G::KG) * G::MF + r % G::MF;
}

// word position of scale word w (0..3: bytes 4 w .. 4 w + 3) of row r (0..255)
// inside a packed scale block: the lane 16 g + r % 16 of wave r / 32 that
// needs it reads words [row r0, s = 0], [r0, s = 1], [r0 + 16, s = 0],
// [r0 + 16, s = 1] (r0 = 32 (r / 32) + r % 16, word 2 s + g / 2) as one chunk
__host__ __device__ constexpr int packed_sf_word(int r, int w) {
  typedef CfgGroupedReg G;
  return (((r / G::kWN) * G::MF + r % G::MF) * 2 + w % 2) * 4 + ((r % G::kWN) / G::MF) * 2 + w / 2;
}

__global__ __launch_bounds__(256) void k_pack_b(const u4_t* __restrict__ b, const u4_t* __restrict__ b_sf, int64_t N,
                                                int64_t K, int32_t E, u4_t* __restrict__ pb,
                                                u4_t* __restrict__ psf) {
  const int64_t tiles = (N + kPackRows - 1) / kPackRows, nst = K / kPackK;
  const int64_t code_chunks = (int64_t)E * tiles * nst * kPackRows * 8;  // 8 x 16 B per row and stage
  const int64_t sf_chunks = (int64_t)E * tiles * nst * kPackRows;       // 16 B per row and stage
  const int64_t ld16 = K / 32, lds16 = K / 256;                          // 16-byte chunks per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // q enumerates source chunks: code chunk c of row r of (slab, stage), then
  // the scale chunks
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < code_chunks + sf_chunks; q += stride) {
    const bool code = q < code_chunks;
    const int64_t qq = code ? q : q - code_chunks;
    const int c = code ? (int)(qq % 8) : 0;
    const int64_t blk = code ? qq / 8 : qq;          // (slab, stage, row)
    const int r = (int)(blk % kPackRows);
    const int64_t block = blk / kPackRows;           // source order: slab * nst + stage
    const int64_t kst = block % nst, slab = block / nst;
    const int64_t e = slab / tiles, row = (slab % tiles) * kPackRows + r;
    const int64_t dst = kst * ((int64_t)E * tiles) + slab;  // stage-major: stage, then (expert, slab)
    u4_t v = {0u, 0u, 0u, 0u};
    if (row < N) v = code ? b[(e * N + row) * ld16 + kst * 8 + c] : b_sf[(e * N + row) * lds16 + kst];
    if (code) {
      pb[dst * (kPackRows * 8) + packed_chunk(r, c)] = v;
    } else {
      uint32_t* sw = (uint32_t*)(psf + dst * kPackRows);
#pragma unroll
      for (int w = 0; w < 4; ++w) sw[packed_sf_word(r, w)] = v[w];
    }
  }
}

size_t packed_b_bytes(int64_t N, int64_t K, int32_t E, size_t* sf_bytes) {
  const int64_t tiles = (N + kPackRows - 1) / kPackRows;
  if (sf_bytes) *sf_bytes = (size_t)E * tiles * kPackRows * (K / 16);
  return (size_t)E * tiles * kPackRows * (K / 2);
}

hipError_t launch_pack_b(const uint8_t* b, const uint8_t* b_sf, int64_t N, int64_t K, int32_t E, uint8_t* pb,
                         uint8_t* psf, hipStream_t stream) {
  size_t sfb = 0;
  const size_t cb = packed_b_bytes(N, K, E, &sfb);
  const int64_t chunks = (int64_t)((cb + sfb) / 16);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(k_pack_b, dim3((unsigned)blocks), dim3(256), 0, stream, (const u4_t*)b, (const u4_t*)b_sf, N, K,
                     E, (u4_t*)pb, (u4_t*)psf);
  return hipGetLastError();
}

hipError_t launch_grouped_packed(GroupedLaunch p, int32_t* status, hipStream_t stream, bool compute) {
  if (status) {
    hipLaunchKernelGGL(k_check_offsets, dim3(1), dim3(64), 0, stream, p.offsets, p.E, p.rows, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!compute) return hipSuccess;
  static_assert(CfgGroupedReg64::BN == CfgGroupedReg::BN && CfgGroupedReg64::WN == CfgGroupedReg::WN &&
                    CfgGroupedReg64::BK == CfgGroupedReg::BK,
                "both row heights read the same packed layout");
  const unsigned tiles_n = (unsigned)((p.N + CfgGroupedReg::BN - 1) / CfgGroupedReg::BN);
  // row passes of 32 or 64 rows, chosen as for the unpacked weights
  int gk = tall_experts(p) ? 3 : 2;
  grouped_forced(&gk);
  if (gk == 3)
    hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, true>), dim3(tiles_n * (unsigned)p.E),
                       dim3(CfgGroupedReg64::kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg, 2, true>), dim3(tiles_n * (unsigned)p.E),
                       dim3(CfgGroupedReg::kThreads), 0, stream, p);
  return hipGetLastError();
}

// Token check of the fused grouped GEMM: when the offsets were valid
// (status 0), status = -(1 + i) for the first row i whose token lies outside
// [0, T).  Runs after k_check_offsets on the same stream.
__global__ __launch_bounds__(256) void k_check_tokens(const int32_t* __restrict__ tok, int64_t rows, int64_t T,
                                                      int32_t* status) {
  __shared__ int first;
  if (threadIdx.x == 0) first = INT_MAX;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < rows; i += blockDim.x) {
    const int32_t t = tok[i];
    if (t < 0 || t >= T) atomicMin(&first, (int)i);
  }
  __syncthreads();
  if (threadIdx.x == 0 && first != INT_MAX && *status == 0) *status = -(first + 1);
}

hipError_t launch_grouped_fused(GroupedLaunch p, bool packed, int32_t* status, hipStream_t stream, bool compute) {
  if (status) {
    hipLaunchKernelGGL(k_check_offsets, dim3(1), dim3(64), 0, stream, p.offsets, p.E, p.rows, status);
    if (p.row_token && p.rows > 0)
      hipLaunchKernelGGL(k_check_tokens, dim3(1), dim3(256), 0, stream, p.row_token, p.rows, p.T, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!compute) return hipSuccess;
  // the register kernels only (the host requires K % 512 == 0); row passes of
  // 32 or 64 rows chosen as for the unfused calls
  const unsigned tiles_n = (unsigned)((p.N + CfgGroupedReg::BN - 1) / CfgGroupedReg::BN);
  int gk = tall_experts(p) ? 3 : 2;
  grouped_forced(&gk);
  gk = gk == 3 ? 3 : 2;
  const dim3 grid(tiles_n * (unsigned)p.E);
  if (packed) {
    if (gk == 3)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, true, true>), grid, dim3(CfgGroupedReg64::kThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedRegF, 2, true, true>), grid, dim3(CfgGroupedRegF::kThreads), 0,
                         stream, p);
  } else if ((p.K / CfgGroupedRegF::BK) % 4 == 0) {
    // linear weight scales four stages per load
    if (gk == 3)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false, true, 0, 4>), grid, dim3(CfgGroupedReg64::kThreads),
                         0, stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedRegF, 2, false, true, 0, 4>), grid, dim3(CfgGroupedRegF::kThreads), 0,
                         stream, p);
  } else {
    if (gk == 3)
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedReg64, 2, false, true>), grid, dim3(CfgGroupedReg64::kThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((k_grouped_reg<CfgGroupedRegF, 2, false, true>), grid, dim3(CfgGroupedRegF::kThreads), 0,
                         stream, p);
  }
  return hipGetLastError();
}

size_t grouped_workspace(int64_t, int64_t, int64_t, int32_t) { return 0; }

// Scratch for nvfp4_gemm_noalloc, the entry point for callers that cannot
// allocate device memory: the split-K arrival counters (first kCounterBytes)
// and fp32 partial tiles that nvfp4_gemm keeps in its workspace.  Every GPU
// that runs the library holds its own copy until the process ends.  In host
// code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the counters must start at zero (every completed call leaves them so)
    e = launch_workspace_init(p, kCounterBytes, stream);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}



__global__ void k_fill_zero(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)ws, n);
  return hipGetLastError();
}

}  // namespace nvfp4
