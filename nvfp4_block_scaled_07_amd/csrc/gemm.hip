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
//  * Packed codes and scale bytes are staged HBM -> VGPR -> LDS with 16-byte
//    loads, double buffered: a stage covers 256 K elements, i.e. 128 code
//    bytes and 16 scale bytes per row.  LDS keeps the packed form (a quarter
//    of the bytes of f16), laid out [chunk][row][16 B] so that the 64 lanes
//    of a wave read contiguous 16-byte entries.
//  * Each lane turns one 16-byte chunk (32 consecutive K elements of one row)
//    into the f16 operands of 4 MFMA K-steps: hardware e2m1->f16 conversion
//    plus one packed f16 multiply by the e4m3 block scale (exact in f16).
//    A and B use the same lane->K map, so the order of K inside a chunk does
//    not change the sum's terms.
//  * The contraction runs on v_mfma_f32_32x32x16_f16 (large tiles) or
//    v_mfma_f32_16x16x32_f16 (skinny and grouped tiles) with fp32
//    accumulators; the e4m3 scales are not powers of two and come per 16
//    elements, so they cannot ride the E8M0-per-32 scaled FP4 MFMA exactly.
//  * Split-K writes fp32 partials to the caller's workspace and a second
//    kernel sums them in a fixed order (bitwise deterministic).
#include "device.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kBK = 256;             // K elements per LDS stage
constexpr int kChunks = kBK / 32;    // 16-byte chunks of codes per row per stage
constexpr int kBKBytes = kBK / 2;    // code bytes per row per stage
constexpr int kBKScales = kBK / 16;  // scale bytes per row per stage

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

template <int BM_, int BN_, int WM_, int WN_, int MF_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWM = BM / WM;        // rows per wave
  static constexpr int kWN = BN / WN;        // cols per wave
  static constexpr int TM = kWM / MF;        // MFMA tiles per wave along M
  static constexpr int TN = kWN / MF;
  static constexpr int KG = 64 / MF;         // lane groups along K in one MFMA
  static constexpr int kSub = kChunks / KG;  // MFMA sub-steps per stage (4 K-steps each)
  static_assert(BM % (WM * MF) == 0 && BN % (WN * MF) == 0, "tile shape");
  typedef typename Mfma<MF>::Acc Acc;
};

template <int BM, int BN>
struct Smem {
  u4_t a[2][kChunks][BM];
  u4_t b[2][kChunks][BN];
  u4_t asf[2][BM];
  u4_t bsf[2][BN];
};

// One operand tile: rows [0, rows) of `data` are valid; rows beyond are
// clamped to the last valid row on load (their results are never stored).
struct Operand {
  const uint8_t* data;
  const uint8_t* sf;
  int64_t ld;    // code bytes per row (K/2)
  int64_t lds;   // scale bytes per row (K/16)
  int rows;      // >= 1
};

template <class C>
struct Stage {
  static constexpr int NT = C::kThreads;
  static constexpr int kA = C::BM * kChunks;
  static constexpr int kB = C::BN * kChunks;
  static constexpr int kS = C::BM + C::BN;
  static constexpr int nA = (kA + NT - 1) / NT;
  static constexpr int nB = (kB + NT - 1) / NT;
  static constexpr int nS = (kS + NT - 1) / NT;
  u4_t ra[nA], rb[nB], rs[nS];

  __device__ __forceinline__ void load(const Operand& A, const Operand& B, int kt, int tid) {
#pragma unroll
    for (int i = 0; i < nA; ++i) {
      const int idx = tid + i * NT;
      if (kA % NT == 0 || idx < kA) {
        const int row = min(idx / kChunks, A.rows - 1), ch = idx % kChunks;
        ra[i] = *(const u4_t*)(A.data + row * A.ld + (int64_t)kt * kBKBytes + ch * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < nB; ++i) {
      const int idx = tid + i * NT;
      if (kB % NT == 0 || idx < kB) {
        const int row = min(idx / kChunks, B.rows - 1), ch = idx % kChunks;
        rb[i] = *(const u4_t*)(B.data + row * B.ld + (int64_t)kt * kBKBytes + ch * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < nS; ++i) {
      const int idx = tid + i * NT;
      if (idx < C::BM) {
        const int row = min(idx, A.rows - 1);
        rs[i] = *(const u4_t*)(A.sf + row * A.lds + (int64_t)kt * kBKScales);
      } else if (idx < kS) {
        const int row = min(idx - C::BM, B.rows - 1);
        rs[i] = *(const u4_t*)(B.sf + row * B.lds + (int64_t)kt * kBKScales);
      }
    }
  }

  __device__ __forceinline__ void store(Smem<C::BM, C::BN>& sm, int st, int tid) {
#pragma unroll
    for (int i = 0; i < nA; ++i) {
      const int idx = tid + i * NT;
      if (kA % NT == 0 || idx < kA) sm.a[st][idx % kChunks][idx / kChunks] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < nB; ++i) {
      const int idx = tid + i * NT;
      if (kB % NT == 0 || idx < kB) sm.b[st][idx % kChunks][idx / kChunks] = rb[i];
    }
#pragma unroll
    for (int i = 0; i < nS; ++i) {
      const int idx = tid + i * NT;
      if (idx < C::BM) sm.asf[st][idx] = rs[i];
      else if (idx < kS) sm.bsf[st][idx - C::BM] = rs[i];
    }
  }
};

// Scale pair (s, s) for half `hi` (0: first 16 elements of the chunk, 1:
// second) from the two scale bytes in bits 0-15 of w.
__device__ __forceinline__ h2_t scale_pair(uint32_t w, int hi) {
  h2_t sp = e4m3x2_to_h2(w);
  h2_t r;
  r[0] = sp[hi];
  r[1] = sp[hi];
  return r;
}

// Multiply-accumulate one LDS stage into acc.  tm_active (uniform) limits the
// row blocks that are computed (grouped experts with few rows).
template <class C>
__device__ __forceinline__ void compute_stage(const Smem<C::BM, C::BN>& sm, int st, int tid, int tm_active,
                                              typename C::Acc (&acc)[C::TM][C::TN]) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r_in = lane % C::MF, g = lane / C::MF;
#pragma unroll
  for (int s = 0; s < C::kSub; ++s) {
    const int c = C::KG * s + g;  // chunk of this lane: K offset 32c in the stage
    u4_t ac[C::TM], bc[C::TN];
    uint32_t asw[C::TM], bsw[C::TN];
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      if (tm < tm_active) {
        const int row = wm * C::kWM + tm * C::MF + r_in;
        ac[tm] = sm.a[st][c][row];
        asw[tm] = ((const uint32_t*)&sm.asf[st][row])[c >> 1] >> (16 * (c & 1));
      }
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int row = wn * C::kWN + tn * C::MF + r_in;
      bc[tn] = sm.b[st][c][row];
      bsw[tn] = ((const uint32_t*)&sm.bsf[st][row])[c >> 1] >> (16 * (c & 1));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8_t af[C::TM], bf[C::TN];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
        if (tm < tm_active) af[tm] = dequant8(ac[tm][t], scale_pair(asw[tm], t >> 1));
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) bf[tn] = dequant8(bc[tn][t], scale_pair(bsw[tn], t >> 1));
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
        if (tm < tm_active) {
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = Mfma<C::MF>::run(af[tm], bf[tn], acc[tm][tn]);
        }
    }
  }
}

template <class C>
__device__ __forceinline__ void mainloop(Smem<C::BM, C::BN>& sm, const Operand& A, const Operand& B, int kt0,
                                         int kt1, int tm_active, typename C::Acc (&acc)[C::TM][C::TN]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int j = 0; j < Mfma<C::MF>::kAcc; ++j) acc[tm][tn][j] = 0.0f;
  if (kt0 >= kt1) return;
  Stage<C> stg;
  stg.load(A, B, kt0, tid);
  stg.store(sm, 0, tid);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int st = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) stg.load(A, B, kt + 1, tid);
    compute_stage<C>(sm, st, tid, tm_active, acc);
    if (more) stg.store(sm, st ^ 1, tid);
    __syncthreads();
  }
}

// Store alpha * acc as bf16 (F32OUT = false) or acc as fp32 partials.
template <class C, bool F32OUT>
__device__ __forceinline__ void epilogue(const typename C::Acc (&acc)[C::TM][C::TN], int tm_active, float alpha,
                                         void* out, int64_t ldo, int rows_valid, int cols_valid) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n_in = lane % C::MF, g = lane / C::MF;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
    if (tm >= tm_active) continue;
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int col = wn * C::kWN + tn * C::MF + n_in;
      if (col >= cols_valid) continue;
#pragma unroll
      for (int j = 0; j < Mfma<C::MF>::kAcc; ++j) {
        const int row = wm * C::kWM + tm * C::MF + Mfma<C::MF>::row(j, g);
        if (row < rows_valid) {
          if (F32OUT)
            ((float*)out)[row * ldo + col] = acc[tm][tn][j];
          else
            ((uint16_t*)out)[row * ldo + col] = f32_to_bf16_bits(alpha * acc[tm][tn][j]);
        }
      }
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void k_gemm(GemmLaunch p) {
  __shared__ Smem<C::BM, C::BN> sm;
  const int tile = blockIdx.x;
  const int tmi = tile / p.tiles_n, tni = tile % p.tiles_n;
  const int z = blockIdx.y;
  const int64_t m0 = (int64_t)tmi * C::BM, n0 = (int64_t)tni * C::BN;
  const int64_t ld = p.K / 2, lds = p.K / 16;
  Operand A{p.a + m0 * ld, p.a_sf + m0 * lds, ld, lds, (int)min<int64_t>(C::BM, p.M - m0)};
  Operand B{p.b + n0 * ld, p.b_sf + n0 * lds, ld, lds, (int)min<int64_t>(C::BN, p.N - n0)};
  const int nk = (int)(p.K / kBK);
  const int kt0 = (int)((int64_t)z * nk / p.splits), kt1 = (int)((int64_t)(z + 1) * nk / p.splits);
  typename C::Acc acc[C::TM][C::TN];
  mainloop<C>(sm, A, B, kt0, kt1, C::TM, acc);
  if (p.splits == 1) {
    const float alpha = p.alpha ? *p.alpha : 1.0f;
    epilogue<C, false>(acc, C::TM, alpha, p.d + m0 * p.N + n0, p.N, A.rows, B.rows);
  } else {
    float* ws = p.ws + (int64_t)z * p.M * p.N;
    epilogue<C, true>(acc, C::TM, 1.0f, ws + m0 * p.N + n0, p.N, A.rows, B.rows);
  }
}

// Sum split-K partials in split order, scale by alpha, round to bf16.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int splits, int64_t mn,
                                                       const float* __restrict__ alpha_p, uint16_t* __restrict__ d) {
  const float alpha = alpha_p ? *alpha_p : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += ws[(int64_t)z * mn + i];
    d[i] = f32_to_bf16_bits(alpha * s);
  }
}

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

template <class C>
__global__ __launch_bounds__(C::kThreads) void k_grouped(GroupedLaunch p) {
  __shared__ Smem<C::BM, C::BN> sm;
  const int e = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * C::BN;
  const int64_t lo = p.offsets[e], hi = p.offsets[e + 1];
  if (lo < 0 || hi <= lo || hi > p.rows) return;  // empty or invalid expert
  const int64_t ld = p.K / 2, lds = p.K / 16;
  const float alpha = p.alpha ? p.alpha[e] : 1.0f;
  Operand B{p.b + ((int64_t)e * p.N + n0) * ld, p.b_sf + ((int64_t)e * p.N + n0) * lds, ld, lds,
            (int)min<int64_t>(C::BN, p.N - n0)};
  const int nk = (int)(p.K / kBK);
  for (int64_t mc = lo; mc < hi; mc += C::BM) {
    const int rows_c = (int)min<int64_t>(C::BM, hi - mc);
    const int tm_active = (rows_c + C::MF - 1) / C::MF;  // row blocks of this wave layout (WM == 1)
    Operand A{p.a + mc * ld, p.a_sf + mc * lds, ld, lds, rows_c};
    typename C::Acc acc[C::TM][C::TN];
    mainloop<C>(sm, A, B, 0, nk, tm_active, acc);
    epilogue<C, false>(acc, tm_active, alpha, p.d + mc * p.N + n0, p.N, rows_c, B.rows);
  }
}

// ---------------------------------------------------------------------------
// Plans and launchers.
// ---------------------------------------------------------------------------
typedef Cfg<128, 128, 2, 2, 32> CfgTile128;
typedef Cfg<16, 128, 1, 4, 16> CfgSkinny16;
typedef Cfg<32, 128, 1, 4, 16> CfgSkinny32;
typedef Cfg<64, 128, 1, 4, 16> CfgSkinny64;
typedef Cfg<64, 128, 1, 4, 16> CfgGrouped;
static_assert(CfgGrouped::WM == 1, "grouped row-block count assumes one wave row");

static const PlanInfo kPlans[] = {
    {"tile128x128_mfma32", 128, 128},
    {"skinny16x128_mfma16", 16, 128},
    {"skinny32x128_mfma16", 32, 128},
    {"skinny64x128_mfma16", 64, 128},
};

static int target_blocks() { return 512; }  // two work-groups per CU on 256 CUs

GemmPlan choose_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan pl;
  pl.kind = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 3 : 0;
  const PlanInfo& info = kPlans[pl.kind];
  pl.name = info.name;
  pl.tiles_m = (M + info.bm - 1) / info.bm;
  pl.tiles_n = (N + info.bn - 1) / info.bn;
  const int64_t tiles = pl.tiles_m * pl.tiles_n;
  const int64_t nk = K / kBK;
  int64_t s = 1;
  if (tiles > 0 && tiles < target_blocks()) s = (target_blocks() + tiles - 1) / tiles;
  if (s > nk) s = nk;
  if (s < 1) s = 1;
  pl.splits = (int)s;
  pl.workspace = s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
  return pl;
}

hipError_t launch_gemm(const GemmPlan& pl, GemmLaunch p, hipStream_t stream) {
  p.tiles_n = (int)pl.tiles_n;
  p.splits = pl.splits;
  dim3 grid((unsigned)(pl.tiles_m * pl.tiles_n), (unsigned)pl.splits);
  switch (pl.kind) {
    case 0: hipLaunchKernelGGL(k_gemm<CfgTile128>, grid, dim3(CfgTile128::kThreads), 0, stream, p); break;
    case 1: hipLaunchKernelGGL(k_gemm<CfgSkinny16>, grid, dim3(CfgSkinny16::kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(k_gemm<CfgSkinny32>, grid, dim3(CfgSkinny32::kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL(k_gemm<CfgSkinny64>, grid, dim3(CfgSkinny64::kThreads), 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.splits == 1) return err;
  const int64_t mn = p.M * p.N;
  int64_t blocks = (mn + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, stream, p.ws, pl.splits, mn, p.alpha,
                     p.d);
  return hipGetLastError();
}

hipError_t launch_grouped(GroupedLaunch p, int32_t* status, hipStream_t stream, bool compute) {
  if (status) {
    hipLaunchKernelGGL(k_check_offsets, dim3(1), dim3(64), 0, stream, p.offsets, p.E, p.rows, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!compute) return hipSuccess;
  dim3 grid((unsigned)((p.N + CfgGrouped::BN - 1) / CfgGrouped::BN), (unsigned)p.E);
  hipLaunchKernelGGL(k_grouped<CfgGrouped>, grid, dim3(CfgGrouped::kThreads), 0, stream, p);
  return hipGetLastError();
}

size_t grouped_workspace(int64_t, int64_t, int64_t, int32_t) { return 0; }

}  // namespace nvfp4
