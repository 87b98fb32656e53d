// LDS-staged tile GEMM kernel (k_gemm) and the device helpers it is built
// from: the HBM -> LDS stage ring, the dequantising and scaled-FP4 MFMA
// stage loops, the bf16 epilogue and the coherent split-K exchange.
//
// Included by gemm.hip and gemm_large.hip.  A kernel instantiation (one Cfg)
// must live in exactly one of them: each source becomes its own code object,
// and the host-side launch stub of an instantiation made in both would be
// registered twice.  gemm_large.hip holds the two large NVFP4 tiles and is
// compiled with a different instruction schedule.
#pragma once

#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace nvfp4 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// f(std::integral_constant<int, I>) for I = 0 .. N - 1
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Split-K workspace: int32 arrival counters for up to 1024 tiles, then the
// fp32 partial tiles.
constexpr int64_t kCounterBytes = 4096;

template <int MF>
struct Mfma;
template <>
struct Mfma<32> {
  typedef f16_t Acc;
  static constexpr int kAcc = 16;
  __device__ __forceinline__ static Acc run(h8_t a, h8_t b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // row of accumulator j for lane group g (lane / 32)
  __device__ __forceinline__ static int row(int j, int g) { return 8 * (j >> 2) + 4 * g + (j & 3); }
};
template <>
struct Mfma<16> {
  typedef f4_t Acc;
  static constexpr int kAcc = 4;
  __device__ __forceinline__ static Acc run(h8_t a, h8_t b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static int row(int j, int g) { return 4 * g + j; }
};

template <int BM_, int BN_, int WM_, int WN_, int MF_, int BK_, int STAGES_, int IL_ = 0, int KS_ = 1,
          int OCC_ = 1, int SBLK_ = 16, int DW_ = 0, int SFL_ = 0>
struct Cfg {
  // SFL 2: the scales are in the 8 x 4 tiled layout (32-byte tiles of 8 rows
  // x 4 scale columns, row r and column c at byte (r % 8) 4 + c % 4, tiles
  // row-major).  One stage of 8 rows is then one run of 8 SB bytes, word-major
  // ([column / 4][row % 8][4 bytes]), and the stage is staged in LDS as it is
  // stored; 0: linear [rows][K/16].
  static constexpr int SFL = SFL_;
  // SBLK: elements per scale: 16 (NVFP4, e4m3 scales, f16 MFMA after
  // dequantisation) or 32 (MXFP4, E8M0 scales, scaled FP4 MFMA)
  static constexpr int SBLK = SBLK_;
  static constexpr bool kMx = SBLK_ == 32;
  // OCC: waves per SIMD the register allocation must leave room for
  static constexpr int OCC = OCC_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_, BK = BK_, STAGES = STAGES_;
  // IL > 0: ask the scheduler to interleave IL VALU instructions after each
  // MFMA of a sub-step (dequantisation of the next K-step under the MFMAs)
  static constexpr int IL = IL_;
  // KS K-groups of WM x WN waves share every LDS stage: group k takes MFMA
  // sub-steps k, k + KS, ... of each stage, and the groups' accumulators are
  // summed through LDS at the end.  More waves per SIMD for the same wave tile.
  static constexpr int KS = KS_;
  static constexpr int kGroupWaves = WM * WN;
  static constexpr int kWaves = KS * WM * WN;
  static constexpr int kThreads = kWaves * 64;
  // DW > 0: only waves 0 .. DW - 1 issue the stage loads (the others go
  // straight to their LDS reads and MFMAs while those wait on the memory
  // pipeline); 0: every wave issues its share
  static constexpr int kDmaWaves = DW_ == 0 ? kWaves : DW_;
  static_assert(DW_ >= 0 && DW_ <= kWaves, "DMA waves");
  static constexpr int kWM = BM / WM;        // rows per wave
  static constexpr int kWN = BN / WN;        // cols per wave
  static constexpr int TM = kWM / MF;        // MFMA tiles per wave along M
  static constexpr int TN = kWN / MF;
  static constexpr int KG = 64 / MF;         // lane groups along K in one MFMA
  static constexpr int CH = BK / 32;         // 16-byte code chunks per row per stage
  static constexpr int RB = BK / 2;          // code bytes per row per stage
  static constexpr int SB = BK / SBLK;       // scale bytes per row per stage
  static constexpr int kSub = CH / KG;       // MFMA sub-steps per stage (4 K-steps each)
  static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile shape");
  static_assert(BK == 128 || BK == 256, "stage depth");
  static_assert(STAGES >= 2 && STAGES <= 8, "pipeline");
  static_assert(KS == 1 || KS == 2 || KS == 4, "K-groups");
  static_assert(kSub % KS == 0, "sub-steps per K-group");
  static_assert(SBLK == 16 || (SBLK == 32 && MF == 32 && IL == 0), "MX tiles use the 32x32x64 scaled MFMA");
  static_assert(SFL == 0 || (SFL == 2 && SBLK == 16 && BM % 8 == 0 && BN % 8 == 0 && MF % 8 == 0 && KG * KS % 2 == 0),
                "8 x 4 scales: NVFP4 tiles of whole 8-row groups");
  typedef typename Mfma<MF>::Acc Acc;
};

template <class C>
struct Smem {
  uint8_t a[C::STAGES][C::BM * C::RB];
  uint8_t b[C::STAGES][C::BN * C::RB];
  uint8_t asf[C::STAGES][C::BM * C::SB];
  uint8_t bsf[C::STAGES][C::BN * C::SB];
};

// XOR swizzle of the 16-byte chunk index of row r (CH chunks per row), chosen
// per MFMA shape by measuring ds_read_b128 throughput of the MFMA-side read
// pattern on gfx950 (rows r_in of one chunk per lane group): 32-row reads
// prefer pairs of rows sharing a slot, 16-row reads a plain rotation.
template <int CH, int MF>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 8) return MF == 32 ? ((r >> 1) & 7) : (r & 7);
  else return MF == 32 ? ((r >> 1) & 3) : (r & 3);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over `bytes` bytes at `base`: loads at or beyond `bytes` return
// zero, which is how rows past the end of an operand are filled.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copy the [ROWS][BYTES] slice at column offset col of a row-major operand
// (row r at base + r * ld, rows >= rows_valid read as zero) into contiguous
// LDS with buffer_load ... lds, VEC bytes per lane.  SWZ stores 16-byte chunk
// c of row r at slot c ^ swz(r).  Wave-instruction j of this tile is issued by
// wave (BASE + j) % NWAVES, so the instructions of all tiles of a stage spread
// evenly over the waves; instructions whose rows are all >= rows_dma are
// skipped (uniform).
template <int ROWS, int BYTES, int VEC>
struct DmaShape {
  static constexpr int kPerRow = BYTES / VEC;
  static constexpr int kRowsPerInst = 64 / kPerRow;
  static constexpr int kInst = (ROWS + kRowsPerInst - 1) / kRowsPerInst;
  static_assert(64 % kPerRow == 0, "row split");
  static_assert(VEC == 16 || VEC == 4, "dma width");
};

// Rows between repeats of swz(r): the swizzle of row j * RPI + lr equals that
// of row (j % 2) * RPI + lr whenever this divides 2 * RPI.
template <int CH, int MF>
constexpr int swz_period() {
  return CH == 8 ? (MF == 32 ? 16 : 8) : (CH == 4 ? (MF == 32 ? 8 : 4) : 8);
}

// wave < 0: this wave issues none of the tile's instructions.  UNIFORM: the
// descriptor and scalar offsets are passed through readfirstlane (they are
// uniform; with some waves skipping the loads the compiler no longer proves
// it and would otherwise loop over lanes for every instruction).
template <int ROWS, int BYTES, int VEC, int SWZ_MF, int NWAVES, int BASE, bool UNIFORM = false>
__device__ __forceinline__ void dma_tile(uint8_t* dst, const uint8_t* base, int64_t ld, int rows_valid, int col,
                                         int wave, int lane, int rows_dma = ROWS) {
  typedef DmaShape<ROWS, BYTES, VEC> D;
  static_assert(SWZ_MF == 0 || (2 * D::kRowsPerInst) % swz_period<D::kPerRow, SWZ_MF>() == 0, "swizzle period");
  rsrc_t rs;
  if constexpr (UNIFORM) {
    const uint64_t pb = (uint64_t)(uintptr_t)(base + col);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pb), hi = __builtin_amdgcn_readfirstlane((uint32_t)(pb >> 32));
    rs = make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)rows_valid * ld - col)));
  } else {
    rs = make_rsrc(base + col, (uint32_t)((int64_t)rows_valid * ld - col));
  }
  const int lr = lane / D::kPerRow, p = lane % D::kPerRow;
  const bool full = rows_valid >= ROWS;  // uniform
  // per-lane byte offset within a group of kRowsPerInst rows (two variants:
  // even and odd instructions); the row step goes in the scalar offset.
  // Lanes of rows >= rows_valid get a vector offset of 2^31, out of range
  // whether or not the hardware adds the scalar offset before its range
  // check, so they read zero and never touch memory past the operand.
  uint32_t voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int c = p;
    if constexpr (SWZ_MF != 0) c = p ^ swz<D::kPerRow, SWZ_MF>(h * D::kRowsPerInst + lr);
    voff[h] = (uint32_t)(lr * ld + c * VEC);
  }
  // only this wave's instructions: j = j0, j0 + NWAVES, ... (a loop over
  // every j with a per-j wave test costs a scalar branch per instruction of
  // the whole stage in every wave)
  int j0 = ((wave - BASE) % NWAVES + NWAVES) % NWAVES;
  if constexpr (UNIFORM) j0 = wave < 0 ? D::kInst : j0;
  constexpr int kPerWave = (D::kInst + NWAVES - 1) / NWAVES;
#pragma unroll
  for (int jj = 0; jj < kPerWave; ++jj) {
    const int j = j0 + jj * NWAVES;
    if (j < D::kInst && j * D::kRowsPerInst < rows_dma) {
      const int r = j * D::kRowsPerInst + lr;
      if (D::kInst * D::kRowsPerInst == ROWS || r < ROWS) {
        uint32_t soff = (uint32_t)(j * D::kRowsPerInst * ld);
        if constexpr (UNIFORM) soff = __builtin_amdgcn_readfirstlane(soff);
        const uint32_t vo = (full || r < rows_valid) ? voff[j & 1] : 0x80000000u;
        if constexpr (VEC == 16)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 64 * VEC), 16, vo, soff, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 64 * VEC), 4, vo, soff, 0, 0);
      }
    }
  }
}

// Wave index as a scalar: the compiler then emits uniform branches (not
// exec-masked ones) for per-wave work such as the DMA assignment.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// One operand tile: rows [0, rows) of `data` are valid (rows >= 1).
struct Operand {
  const uint8_t* data;
  const uint8_t* sf;
  int64_t ld;    // code bytes per row (K/2)
  int64_t lds;   // scale bytes per row (K/16)
  int rows;
};

template <class C>
struct StageDma {
  static constexpr int SV = C::SB == 16 ? 16 : 4;
  typedef DmaShape<C::BM, C::RB, 16> A;
  typedef DmaShape<C::BN, C::RB, 16> B;
  // 8 x 4 scales: each 8-row group's stage is one row of 8 SB bytes
  typedef typename std::conditional<C::SFL == 2, DmaShape<C::BM / 8, 8 * C::SB, 16>, DmaShape<C::BM, C::SB, SV>>::type AS;
  typedef typename std::conditional<C::SFL == 2, DmaShape<C::BN / 8, 8 * C::SB, 16>, DmaShape<C::BN, C::SB, SV>>::type BS;
  static constexpr int kTotal = A::kInst + B::kInst + AS::kInst + BS::kInst;
  // Every wave that issues loads issues at least this many per stage.  A's
  // code instructions come first and may be skipped (rows an expert does not
  // have), so only the instructions after them are counted.
  static constexpr int kMinPerWave = (kTotal - A::kInst) / C::kDmaWaves;
  static_assert(kMinPerWave * (C::STAGES - 2) <= 63, "vmcnt range");
};

template <class C>
__device__ __forceinline__ void issue_stage(Smem<C>& sm, int buf, const Operand& A, const Operand& B, int kt,
                                            int wave, int lane, int a_rows_dma) {
  typedef StageDma<C> D;
  constexpr int W = C::kDmaWaves;
  constexpr bool U = W < C::kWaves;
  if constexpr (U) wave = wave < W ? wave : -1;
  dma_tile<C::BM, C::RB, 16, C::MF, W, 0, U>(sm.a[buf], A.data, A.ld, A.rows, kt * C::RB, wave, lane, a_rows_dma);
  dma_tile<C::BN, C::RB, 16, C::MF, W, D::A::kInst, U>(sm.b[buf], B.data, B.ld, B.rows, kt * C::RB, wave, lane);
  if constexpr (C::SFL == 2) {
    // the operand's scale pointer is its first row's group (rows start on a
    // group); groups past the last row are padding of the tiled matrix
    dma_tile<C::BM / 8, 8 * C::SB, 16, 0, W, D::A::kInst + D::B::kInst, U>(sm.asf[buf], A.sf, 8 * A.lds,
                                                                            (A.rows + 7) / 8, kt * 8 * C::SB, wave, lane);
    dma_tile<C::BN / 8, 8 * C::SB, 16, 0, W, D::A::kInst + D::B::kInst + D::AS::kInst, U>(
        sm.bsf[buf], B.sf, 8 * B.lds, (B.rows + 7) / 8, kt * 8 * C::SB, wave, lane);
  } else {
    dma_tile<C::BM, C::SB, D::SV, 0, W, D::A::kInst + D::B::kInst, U>(sm.asf[buf], A.sf, A.lds, A.rows,
                                                                          kt * C::SB, wave, lane);
    dma_tile<C::BN, C::SB, D::SV, 0, W, D::A::kInst + D::B::kInst + D::AS::kInst, U>(sm.bsf[buf], B.sf, B.lds,
                                                                                         B.rows, kt * C::SB, wave, lane);
  }
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then a work-group barrier.  The empty asm
// keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until the stage whose loads were followed by `later` more issued
// stages has landed in LDS (loads of one wave return in order), then barrier.
template <class C, int L = C::STAGES - 2>
__device__ __forceinline__ void stage_ready(int later) {
  if constexpr (L <= 0) {
    wait_vm_barrier<0>();
  } else {
    if (later >= L) {
      wait_vm_barrier<L * StageDma<C>::kMinPerWave>();
      return;
    }
    stage_ready<C, L - 1>(later);
  }
}

__device__ __forceinline__ h2_t scale_pair(h2_t sp, int hi) {
  h2_t r;
  r[0] = sp[hi];
  r[1] = sp[hi];
  return r;
}

// LDS reads of the MFMA operands are issued as inline asm: the compiler then
// does not treat them as aliasing the in-flight global_load_lds writes of later
// stages (it would otherwise drain all loads before every read).  Completion
// is awaited explicitly with lgkm_wait(), which re-defines every result so no
// use can be scheduled before the wait.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }
__device__ __forceinline__ void ds_read128(u4_t& v, uint32_t a) { asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a)); }
__device__ __forceinline__ void ds_read32(uint32_t& v, uint32_t a) { asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(a)); }
// The same with a compile-time byte offset, carried in the instruction's
// 16-bit offset field when it fits.
template <int OFF>
__device__ __forceinline__ void ds_read128_at(u4_t& v, uint32_t a) {
  if constexpr (OFF < 65536) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
  else ds_read128(v, a + OFF);
}
// 8 bits, zero-extended
template <int OFF>
__device__ __forceinline__ void ds_read_u8_at(uint32_t& v, uint32_t a) {
  if constexpr (OFF < 65536) asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
  else asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(a + OFF));
}
// 16 bits, zero-extended
template <int OFF>
__device__ __forceinline__ void ds_read_u16_at(uint32_t& v, uint32_t a) {
  if constexpr (OFF < 65536) asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
  else asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(a + OFF));
}
__device__ __forceinline__ void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void pin(u4_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Multiply-accumulate one LDS stage into acc.  tm_active (uniform) limits the
// row blocks that are computed (grouped experts with few rows).  Per K-step
// only the A operands and one B operand are live, which keeps the 128x128
// wave tile of the large plan inside the register file.
// MXFP4 stage: per 64-element sub-step, one v_mfma_scale_f32_32x32x64_f8f6f4
// per (tm, tn).  Lane l supplies the 32 codes of row l % 32 in K block
// l / 32 of the sub-step (one 16-byte chunk, low nibble first, exactly the
// stored layout) and that block's E8M0 scale in the low byte of its scale
// operand; the hardware applies both scales and accumulates in fp32.
// The operands of sub-step ss + 1 are read from LDS while the MFMAs of
// sub-step ss run (two register slots): with no dequantisation between the
// reads and the MFMAs, the read latency is otherwise as long as a
// sub-step's MFMAs.

// Per-lane LDS read addresses of a tile, computed once per tile (stage buffer
// 0, first row block): the code chunk of each sub-step of this lane's K-group
// and the scales of its first sub-step.  Stage buffers, row
// blocks and later sub-steps' scales are compile-time offsets from these.
template <class C>
struct ReadAddr {
  static constexpr int kS = C::kSub / C::KS;  // sub-steps of one K-group per stage
  uint32_t a[kS], b[kS];
  uint32_t as, bs;
};

template <class C>
__device__ __forceinline__ ReadAddr<C> read_addr(const Smem<C>& sm) {
  ReadAddr<C> ra;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int gw = wave % C::kGroupWaves, kgrp = wave / C::kGroupWaves;
  const int wm = gw / C::WN, wn = gw % C::WN;
  const int r_in = lane % C::MF, g = lane / C::MF;
  const int ra_row = wm * C::kWM + r_in, rb_row = wn * C::kWN + r_in;
  // the swizzle depends on the row's low bits only, which row blocks keep
  static_assert(C::kWM % swz_period<C::CH, C::MF>() == 0 && C::kWN % swz_period<C::CH, C::MF>() == 0 &&
                    C::MF % swz_period<C::CH, C::MF>() == 0, "swizzle must not depend on the row block");
#pragma unroll
  for (int ss = 0; ss < ReadAddr<C>::kS; ++ss) {
    const int c = C::KG * (ss * C::KS + kgrp) + g;
    ra.a[ss] = lds_addr(sm.a[0]) + ra_row * C::RB + ((c ^ swz<C::CH, C::MF>(ra_row)) << 4);
    ra.b[ss] = lds_addr(sm.b[0]) + rb_row * C::RB + ((c ^ swz<C::CH, C::MF>(rb_row)) << 4);
    pin(ra.a[ss]);
    pin(ra.b[ss]);
  }
  // chunk c's scales: NVFP4 bytes 2c and 2c + 1 (blocks of 16), MXFP4 byte c
  constexpr int kScalePerChunk = 32 / C::SBLK;
  const int c0 = C::KG * kgrp + g;
  if constexpr (C::SFL == 2) {
    // chunk c's two scales: columns 2c, 2c + 1, in word c / 2 of the group's run
    const int word = (c0 >> 1) * 32 + 2 * (c0 & 1);
    ra.as = lds_addr(sm.asf[0]) + (ra_row >> 3) * 8 * C::SB + (ra_row & 7) * 4 + word;
    ra.bs = lds_addr(sm.bsf[0]) + (rb_row >> 3) * 8 * C::SB + (rb_row & 7) * 4 + word;
  } else {
    ra.as = lds_addr(sm.asf[0]) + ra_row * C::SB + kScalePerChunk * c0;
    ra.bs = lds_addr(sm.bsf[0]) + rb_row * C::SB + kScalePerChunk * c0;
  }
  pin(ra.as);
  pin(ra.bs);
  return ra;
}

template <class C>
struct MxFrags {
  u4_t ac[C::TM], bc[C::TN];
  uint32_t asw[C::TM], bsw[C::TN];  // the chunk's E8M0 scale byte
};

// LDS reads of MX sub-step SS of stage buffer BUF
template <class C, int BUF, int SS>
__device__ __forceinline__ void mx_read(MxFrags<C>& f, const ReadAddr<C>& ra) {
  constexpr int kScale = SS * C::KG * C::KS;  // one scale byte per chunk
  static_for<C::TM>([&](auto tmc) {
    constexpr int tm = decltype(tmc)::value;
    ds_read128_at<BUF * C::BM * C::RB + tm * 32 * C::RB>(f.ac[tm], ra.a[SS]);
    ds_read_u8_at<BUF * C::BM * C::SB + tm * 32 * C::SB + kScale>(f.asw[tm], ra.as);
  });
  static_for<C::TN>([&](auto tnc) {
    constexpr int tn = decltype(tnc)::value;
    ds_read128_at<BUF * C::BN * C::RB + tn * 32 * C::RB>(f.bc[tn], ra.b[SS]);
    ds_read_u8_at<BUF * C::BN * C::SB + tn * 32 * C::SB + kScale>(f.bsw[tn], ra.bs);
  });
}

// One MX stage (buffer BUF): the next sub-step's reads are issued into the
// other fragment set before this sub-step's MFMAs.
template <class C, int BUF>
__device__ __forceinline__ void compute_stage_mx(const ReadAddr<C>& ra, typename C::Acc (&acc)[C::TM][C::TN]) {
  typedef int v8i_t __attribute__((ext_vector_type(8)));
  constexpr int NS = C::kSub / C::KS;
  MxFrags<C> f[2];
  mx_read<C, BUF, 0>(f[0], ra);
  static_for<NS>([&](auto ssc) {
    constexpr int ss = decltype(ssc)::value;
    MxFrags<C>& cur = f[ss & 1];
    lgkm_wait();  // slot ss & 1 has landed (nothing else is in flight)
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      pin(cur.ac[tm]);
      pin(cur.asw[tm]);
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      pin(cur.bc[tn]);
      pin(cur.bsw[tn]);
    }
    if constexpr (ss + 1 < NS) mx_read<C, BUF, ss + 1>(f[(ss + 1) & 1], ra);
    v8i_t av[C::TM], bv[C::TN];
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
      av[tm] = v8i_t{(int)cur.ac[tm][0], (int)cur.ac[tm][1], (int)cur.ac[tm][2], (int)cur.ac[tm][3], 0, 0, 0, 0};
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
      bv[tn] = v8i_t{(int)cur.bc[tn][0], (int)cur.bc[tn][1], (int)cur.bc[tn][2], (int)cur.bc[tn][3], 0, 0, 0, 0};
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[tm], bv[tn], acc[tm][tn], 4, 4, 0,
                                                                       (int)cur.asw[tm], 0, (int)cur.bsw[tn]);
  });
}

// Multiply-accumulate one LDS stage (buffer BUF) into acc.
template <class C, int BUF>
__device__ __forceinline__ void compute_stage(const Smem<C>& sm, const ReadAddr<C>& ra, int tm_active,
                                              typename C::Acc (&acc)[C::TM][C::TN]) {
  if constexpr (C::kMx) {
    compute_stage_mx<C, BUF>(ra, acc);
    return;
  }
  // scale bytes between a K-group's sub-steps (KG KS chunks: 2 KG KS columns)
  constexpr int kScaleStep = C::SFL == 2 ? (C::KG * C::KS / 2) * 32 : 2 * C::KG * C::KS;
#pragma unroll
  for (int ss = 0; ss < ReadAddr<C>::kS; ++ss) {
    u4_t ac[C::TM], bc[C::TN];
    uint32_t asw[C::TM], bsw[C::TN];
    static_for<C::TM>([&](auto tmc) {
      constexpr int tm = decltype(tmc)::value;
      if (tm < tm_active) {
        ds_read128_at<BUF * C::BM * C::RB + tm * C::MF * C::RB>(ac[tm], ra.a[ss]);
        ds_read_u16_at<BUF * C::BM * C::SB + tm * C::MF * C::SB>(asw[tm], ra.as + ss * kScaleStep);
      }
    });
    static_for<C::TN>([&](auto tnc) {
      constexpr int tn = decltype(tnc)::value;
      ds_read128_at<BUF * C::BN * C::RB + tn * C::MF * C::RB>(bc[tn], ra.b[ss]);
      ds_read_u16_at<BUF * C::BN * C::SB + tn * C::MF * C::SB>(bsw[tn], ra.bs + ss * kScaleStep);
    });
    lgkm_wait();
    h2_t asp[C::TM], bsp[C::TN];
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      if (tm < tm_active) {
        pin(ac[tm]);
        pin(asw[tm]);
        asp[tm] = e4m3x2_to_h2(asw[tm]);
      }
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      pin(bc[tn]);
      pin(bsw[tn]);
      bsp[tn] = e4m3x2_to_h2(bsw[tn]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8_t af[C::TM];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
        if (tm < tm_active) af[tm] = dequant8(ac[tm][t], scale_pair(asp[tm], t >> 1));
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const h8_t bf = dequant8(bc[tn][t], scale_pair(bsp[tn], t >> 1));
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
          if (tm < tm_active) acc[tm][tn] = Mfma<C::MF>::run(af[tm], bf, acc[tm][tn]);
      }
    }
    if constexpr (C::IL > 0) {
#pragma unroll
      for (int i = 0; i < 4 * C::TM * C::TN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, C::IL, 0);  // then IL VALU
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void zero_acc(typename C::Acc (&acc)[C::TM][C::TN]) {
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int j = 0; j < Mfma<C::MF>::kAcc; ++j) acc[tm][tn][j] = 0.0f;
}

// Stages i0 + J, i0 + J + 1, ... (J < STAGES) of the main loop: issue the DMA
// of the stage STAGES - 1 ahead, compute this one, wait for the next.
template <class C, int J>
__device__ __forceinline__ void stage_steps(Smem<C>& sm, const ReadAddr<C>& ra, const Operand& A, const Operand& B,
                                            int i0, int n, int kt0, int wave, int lane, int a_rows_dma,
                                            int tm_active, typename C::Acc (&acc)[C::TM][C::TN]) {
  if constexpr (J < C::STAGES) {
    const int i = i0 + J;
    if (i >= n) return;
    const int pre = i + C::STAGES - 1;
    if (pre < n) issue_stage<C>(sm, (J + C::STAGES - 1) % C::STAGES, A, B, kt0 + pre, wave, lane, a_rows_dma);
    compute_stage<C, J>(sm, ra, tm_active, acc);
    if (i + 1 < n) stage_ready<C>(min(C::STAGES - 2, n - 2 - i));
    stage_steps<C, J + 1>(sm, ra, A, B, i0, n, kt0, wave, lane, a_rows_dma, tm_active, acc);
  }
}

// K-tiles [kt0, kt1) of the tile into acc (which is zeroed first).  Loads run
// STAGES - 1 stages ahead of the MFMAs; each wait only drains the stage needed
// next, so the later stages stay in flight across the barrier.
template <class C>
__device__ __forceinline__ void mainloop(Smem<C>& sm, const Operand& A, const Operand& B, int kt0, int kt1,
                                         int tm_active, typename C::Acc (&acc)[C::TM][C::TN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  zero_acc<C>(acc);
  const int n = kt1 - kt0;
  if (n <= 0) return;
  // the previous user of these buffers (an earlier tile of this work-group)
  // is done once every wave passes this barrier
  wait_vm_barrier<0>();
  // A rows whose products are used: fewer only when an expert has fewer rows
  // than the tile (grouped plans have one wave row, WM == 1)
  const int a_rows_dma = C::WM == 1 ? tm_active * C::MF : C::BM;
#pragma unroll
  for (int i = 0; i < C::STAGES - 1; ++i)
    if (i < n) issue_stage<C>(sm, i, A, B, kt0 + i, wave, lane, a_rows_dma);
  stage_ready<C>(min(C::STAGES - 2, n - 1));
  const ReadAddr<C> ra = read_addr<C>(sm);
  // unrolled by STAGES: each stage buffer's LDS offset is a constant
  for (int i0 = 0; i0 < n; i0 += C::STAGES)
    stage_steps<C, 0>(sm, ra, A, B, i0, n, kt0, wave, lane, a_rows_dma, tm_active, acc);
}

// alpha * acc -> bf16 stores; bounds checks only for partial tiles.
template <class C>
__device__ __forceinline__ void store_bf16(const typename C::Acc (&acc)[C::TM][C::TN], int tm_active, float alpha,
                                           uint16_t* out, int64_t ldo, int rows_valid, int cols_valid) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, gw = wave_id() % C::kGroupWaves;
  const int wm = gw / C::WN, wn = gw % C::WN;
  const int n_in = lane % C::MF, g = lane / C::MF;
  if (rows_valid >= C::BM && cols_valid >= C::BN) {  // full tile (uniform)
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      if (tm >= tm_active) continue;
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const int col = wn * C::kWN + tn * C::MF + n_in;
#pragma unroll
        for (int j = 0; j < Mfma<C::MF>::kAcc; ++j) {
          const int row = wm * C::kWM + tm * C::MF + Mfma<C::MF>::row(j, g);
          out[row * ldo + col] = f32_to_bf16_bits(alpha * acc[tm][tn][j]);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
    if (tm >= tm_active) continue;
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int col = wn * C::kWN + tn * C::MF + n_in;
#pragma unroll
      for (int j = 0; j < Mfma<C::MF>::kAcc; ++j) {
        const int row = wm * C::kWM + tm * C::MF + Mfma<C::MF>::row(j, g);
        if (row < rows_valid && col < cols_valid) out[row * ldo + col] = f32_to_bf16_bits(alpha * acc[tm][tn][j]);
      }
    }
  }
}

// Split-K exchange.  The partial tiles and the arrival counters are the only
// memory the work-groups of one call share.  They are written and read only
// with agent-coherent accesses (the sc1 cache policy: through to the level
// where the L2s of all XCDs agree), so the exchange needs no L2 write-back or
// invalidation of the whole cache, which costs microseconds while other
// work-groups still stream.  Ordering: every wave's partial stores complete
// (s_waitcnt vmcnt(0)) before the work-group barrier after which its arrival
// is counted, and the last split issues its partial loads only after it has
// read the count.  The accesses go through buffer descriptors bounded by the
// tile's partial block, so an index outside it reads zero and writes nothing.
constexpr int kCoherent = 16;  // buffer cache policy: sc1

__device__ __forceinline__ rsrc_t partial_rsrc(const float* block, int slots, int tile_floats) {
  return make_rsrc(block, (uint32_t)((int64_t)slots * tile_floats * 4));
}
__device__ __forceinline__ void store_coherent(const rsrc_t& r, uint32_t off, f4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ void store_coherent(const rsrc_t& r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ f4_t load_coherent4(const rsrc_t& r, uint32_t off) {
  return __builtin_bit_cast(f4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ float load_coherent(const rsrc_t& r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}

// Count one arrival at a tile's counter (thread 0 of the work-group, after
// the barrier that follows its partial stores); true for the last of S.
__device__ __forceinline__ bool count_arrival(int* counter, int S) {
  return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
}
// The last split leaves the counter at zero for the next call.
__device__ __forceinline__ void reset_counter(int* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K partials are kept in the accumulators' own register layout: float4
// chunk i of lane l of wave slot w (within a K-group) sits at index
// (w * kChunks + i) * 64 + l, so every store and every load of the reduction
// moves a contiguous 1 KB per wave.
template <class C>
struct PartLayout {
  static constexpr int kAccQ = Mfma<C::MF>::kAcc / 4;      // float4 per MFMA tile
  static constexpr int kChunks = C::TM * C::TN * kAccQ;     // float4 per lane
  static constexpr int kQ = C::kGroupWaves * kChunks * 64;  // float4 per tile
  static_assert(kQ * 4 == C::BM * C::BN, "partial tile size");
};

// Split z's partial tile into slot z of the tile's block (descriptor r).
template <class C>
__device__ __forceinline__ void store_partial(const typename C::Acc (&acc)[C::TM][C::TN], const rsrc_t& r, int z) {
  typedef PartLayout<C> P;
  const int lane = threadIdx.x & 63, gw = wave_id() % C::kGroupWaves;
  const uint32_t base = (uint32_t)(z * P::kQ + gw * P::kChunks * 64 + lane) * 16;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int q = 0; q < P::kAccQ; ++q) {
        f4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[tm][tn][4 * q + e];
        store_coherent(r, base + (uint32_t)(((tm * C::TN + tn) * P::kAccQ + q) * 64 * 16), v);
      }
}

// Sum the S partial tiles of one output tile in split order (((p0 + p1) + p2)
// + ...), scale by alpha and store bf16 with bounds checks.  Float4 position f
// of the layout above is handled by thread f mod kThreads; the S loads of
// kLoads / S positions are issued together (kLoads float4 in flight: 16, or 8
// where four waves per SIMD must fit), so a thread needs about
// ceil(positions * S / kLoads) memory round trips.
template <class C, int S>
__device__ __forceinline__ void reduce_partials_s(const rsrc_t& r, float alpha, uint16_t* out, int64_t ldo,
                                                  int rows_valid, int cols_valid) {
  typedef PartLayout<C> P;
  constexpr int kLoads = C::OCC >= 4 ? 8 : 16;
  constexpr int PB = S >= kLoads ? 1 : kLoads / S;  // positions per batch
  for (int f0 = threadIdx.x; f0 < P::kQ; f0 += C::kThreads * PB) {
    f4_t v[PB][S];
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      const int f = f0 + b * C::kThreads;
      if (f < P::kQ) {
#pragma unroll
        for (int z = 0; z < S; ++z) v[b][z] = load_coherent4(r, (uint32_t)(z * P::kQ + f) * 16);
      }
    }
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      const int f = f0 + b * C::kThreads;
      if (f >= P::kQ) continue;
      f4_t sum = v[b][0];
#pragma unroll
      for (int z = 1; z < S; ++z) sum += v[b][z];
      const int lane = f & 63, i = (f >> 6) % P::kChunks, gw = (f >> 6) / P::kChunks;
      const int q = i % P::kAccQ, tn = (i / P::kAccQ) % C::TN, tm = (i / P::kAccQ) / C::TN;
      const int wm = gw / C::WN, wn = gw % C::WN;
      const int col = wn * C::kWN + tn * C::MF + lane % C::MF, g = lane / C::MF;
      if (col >= cols_valid) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm * C::kWM + tm * C::MF + Mfma<C::MF>::row(4 * q + e, g);
        if (row < rows_valid) out[row * ldo + col] = f32_to_bf16_bits(alpha * sum[e]);
      }
    }
  }
}

constexpr int kMaxSplits = 16;

template <class C>
__device__ __forceinline__ void reduce_partials(const rsrc_t& r, int S, float alpha, uint16_t* out, int64_t ldo,
                                                int rows_valid, int cols_valid) {
  switch (S) {
#define NVFP4_RED(n) \
  case n: reduce_partials_s<C, n>(r, alpha, out, ldo, rows_valid, cols_valid); break;
    NVFP4_RED(2) NVFP4_RED(3) NVFP4_RED(4) NVFP4_RED(5) NVFP4_RED(6) NVFP4_RED(7) NVFP4_RED(8) NVFP4_RED(9)
    NVFP4_RED(10) NVFP4_RED(11) NVFP4_RED(12) NVFP4_RED(13) NVFP4_RED(14) NVFP4_RED(15) NVFP4_RED(16)
#undef NVFP4_RED
    default: break;
  }
}

// Sum the KS K-groups' accumulators into group 0's (pairwise tree through LDS:
// groups [h, 2h) store, groups [0, h) add).  Each wave stores its registers in
// its own lane-contiguous slice, so the paired wave reads them back with the
// same layout and no bank conflicts.  Called by every wave of the work-group
// after all LDS reads of the main loop.
template <class C>
struct GroupRed {
  static constexpr int kChunks = C::TM * C::TN * Mfma<C::MF>::kAcc / 4;  // f4 per lane
  static constexpr int kSlotFloats = C::kGroupWaves * kChunks * 64 * 4;  // = BM * BN
  static constexpr int kSlots = C::KS / 2;
  static constexpr int kFloats = C::KS > 1 ? kSlots * kSlotFloats : 1;
};

template <class C>
__device__ __forceinline__ void reduce_groups(float* red, typename C::Acc (&acc)[C::TM][C::TN]) {
  if constexpr (C::KS > 1) {
    typedef GroupRed<C> R;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int gw = wave % C::kGroupWaves, kgrp = wave / C::kGroupWaves;
    __syncthreads();  // every wave is past its last read of the stage buffers
#pragma unroll
    for (int h = C::KS / 2; h >= 1; h /= 2) {
      if (kgrp >= h && kgrp < 2 * h) {
        f4_t* dst = (f4_t*)(red + (int64_t)(kgrp - h) * R::kSlotFloats) + (int64_t)gw * R::kChunks * 64 + lane;
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
            for (int q = 0; q < Mfma<C::MF>::kAcc / 4; ++q) {
              f4_t v;
              for (int i = 0; i < 4; ++i) v[i] = acc[tm][tn][4 * q + i];
              dst[((tm * C::TN + tn) * (Mfma<C::MF>::kAcc / 4) + q) * 64] = v;
            }
      }
      __syncthreads();
      if (kgrp < h) {
        const f4_t* src = (const f4_t*)(red + (int64_t)kgrp * R::kSlotFloats) + (int64_t)gw * R::kChunks * 64 + lane;
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
            for (int q = 0; q < Mfma<C::MF>::kAcc / 4; ++q) {
              const f4_t v = src[((tm * C::TN + tn) * (Mfma<C::MF>::kAcc / 4) + q) * 64];
              for (int i = 0; i < 4; ++i) acc[tm][tn][4 * q + i] += v[i];
            }
      }
      __syncthreads();
    }
  }
}

template <class C>
union SharedGemm {
  Smem<C> pipe;
  float red[GroupRed<C>::kFloats];
};

// Map a linear work-group id to a logical id so that each XCD (work-groups
// are dispatched round-robin over 8 XCDs) gets one contiguous logical range.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8, r = G % 8, x = b % 8, i = b / 8;
  return x * q + min(x, r) + i;
}

template <class C, bool SPLITK>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gemm(GemmLaunch p) {
  __shared__ __attribute__((aligned(16))) SharedGemm<C> shm;
  Smem<C>& sm = shm.pipe;
  __shared__ int last_flag;
  const int S = p.splits;
  const int G = (int)(p.tiles_m * p.tiles_n) * S;
  const int L = xcd_remap(blockIdx.x, G);
  const int tile_l = L / S, z = L % S;
  // grouped raster: bands of GROUP_M tile rows, column by column inside a band
  const int tiles_m = (int)p.tiles_m, tiles_n = (int)p.tiles_n;
  const int band = p.group_m * tiles_n;
  const int first_m = (tile_l / band) * p.group_m;
  const int gm = min(p.group_m, tiles_m - first_m);
  const int tmi = first_m + (tile_l % band) % gm, tni = (tile_l % band) / gm;
  const int tile = tmi * tiles_n + tni;

  const int64_t m0 = (int64_t)tmi * C::BM, n0 = (int64_t)tni * C::BN;
  const int64_t ld = p.K / 2, lds = p.K / C::SBLK;
  Operand A{p.a + m0 * ld, p.a_sf + m0 * lds, ld, lds, (int)min<int64_t>(C::BM, p.M - m0)};
  Operand B{p.b + n0 * ld, p.b_sf + n0 * lds, ld, lds, (int)min<int64_t>(C::BN, p.N - n0)};
  const int nk = (int)(p.K / C::BK);
  const int kt0 = (int)((int64_t)z * nk / S), kt1 = (int)((int64_t)(z + 1) * nk / S);
  typename C::Acc acc[C::TM][C::TN];
  mainloop<C>(sm, A, B, kt0, kt1, C::TM, acc);
  reduce_groups<C>(shm.red, acc);
  const bool lead = C::KS == 1 || wave_id() < C::kGroupWaves;  // K-group 0 holds the sum
  const float alpha = p.alpha ? *p.alpha : 1.0f;
  uint16_t* out = p.d + m0 * p.N + n0;
  if (!SPLITK || S == 1) {
    if (lead) store_bf16<C>(acc, C::TM, alpha, out, p.N, A.rows, B.rows);
    return;
  }
  // split-K: publish this split's partial, count arrivals, last one reduces
  const int tid = threadIdx.x;
  constexpr int kTileFloats = C::BM * C::BN;
  int* counter = (int*)p.ws + tile;
  const rsrc_t part = partial_rsrc(p.ws + kCounterBytes / 4 + (int64_t)tile * S * kTileFloats, S, kTileFloats);
  if (lead) store_partial<C>(acc, part, z);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
  __syncthreads();
  if (tid == 0) last_flag = count_arrival(counter, S);
  __syncthreads();
  if (!last_flag) return;
  reduce_partials<C>(part, S, alpha, out, p.N, A.rows, B.rows);
  if (tid == 0) reset_counter(counter);
}

}  // namespace nvfp4
