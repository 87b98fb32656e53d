// The two unsplit large-M NVFP4 tiles (plan kinds 14 and 16), built in a
// source of their own so that they can take another instruction schedule
// than the rest of the library: the build compiles this file with the
// iterative ILP scheduler, which keeps more dequantisation work between the
// MFMAs of these 8-wave tiles (8192 x 6144 x 6144 on the 256x256 tile:
// about 3.5% faster; the same schedule doubles the time of the split 64x64
// K-group tile, so it is not applied library-wide).  Results are bitwise the
// same: the schedule reorders independent instructions only.
#include "gemm_tile.h"

namespace nvfp4 {

// Waves 0-3 (one per SIMD) issue each stage's loads; the other four go
// straight to their LDS reads and MFMAs (1-3% faster at 4096..16384 x 6144 x
// 6144 on two boxes, bitwise the same).
typedef Cfg<256, 256, 2, 4, 32, 256, 2, 0, 1, 2, 16, 4> CfgTile256w8k256;  // 8 waves of 128x64
typedef Cfg<256, 192, 4, 2, 32, 256, 2, 0, 1, 2, 16, 4> CfgTile256x192;    // 8 waves of 64x96, 126 KB LDS
// the same tiles on scales in the 8 x 4 tiled layout (nvfp4_gemm_sf)
typedef Cfg<256, 256, 2, 4, 32, 256, 2, 0, 1, 2, 16, 4, 2> CfgTile256w8k256Sf8;
typedef Cfg<256, 192, 4, 2, 32, 256, 2, 0, 1, 2, 16, 4, 2> CfgTile256x192Sf8;

void launch_large_tile(int kind, const GemmLaunch& p, unsigned grid, hipStream_t stream) {
  const bool sf8 = p.sf_layout == 2;
  if (kind == 14 && sf8)
    hipLaunchKernelGGL((k_gemm<CfgTile256w8k256Sf8, false>), dim3(grid), dim3(CfgTile256w8k256Sf8::kThreads), 0, stream,
                       p);
  else if (kind == 14)
    hipLaunchKernelGGL((k_gemm<CfgTile256w8k256, false>), dim3(grid), dim3(CfgTile256w8k256::kThreads), 0, stream, p);
  else if (kind == 16 && sf8)
    hipLaunchKernelGGL((k_gemm<CfgTile256x192Sf8, false>), dim3(grid), dim3(CfgTile256x192Sf8::kThreads), 0, stream, p);
  else if (kind == 16)
    hipLaunchKernelGGL((k_gemm<CfgTile256x192, false>), dim3(grid), dim3(CfgTile256x192::kThreads), 0, stream, p);
}

}  // namespace nvfp4
