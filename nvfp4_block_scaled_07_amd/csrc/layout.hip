// Scale-layout conversion for interop: between the library's linear
// [rows][K/16] e4m3 scales and the 128 x 4 tiled layout of the CUTLASS NVFP4
// path.  The pages only name the switch between scale layouts ("The Art of
// Reading the Manual: Debugging FP4 GEMM Kernels on Blackwell SM120", section
// "The Message": use_8x4_sf_layout=False) and never describe one; the tiled
// layout is read as: the scale matrix, padded with zeros to a multiple of 128
// rows and 4 columns, stored as 512-byte tiles of 128 rows x 4 columns in
// row-major tile order, the scale of row r and column c of a tile at byte
// (r % 32) * 16 + ((r % 128) / 32) * 4 + c % 4.  The 8 x 4 layout that the
// switch names is read the same way with 32-byte tiles of 8 rows x 4 columns
// (padding to multiples of 8 rows and 4 columns), the scale of row r and
// column c of a tile at byte (r % 8) * 4 + c % 4.  Byte moves only.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

// one thread per byte of the tiled layout (padding bytes written as zero)
__global__ __launch_bounds__(256) void k_scales_to_128x4(const uint8_t* __restrict__ sf, uint8_t* __restrict__ tiled,
                                                         int64_t rows, int64_t cols, int64_t total) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total) return;
  const int64_t tc = (cols + 3) / 4;
  const int64_t tile = p / 512, in = p % 512;
  const int64_t r = (tile / tc) * 128 + ((in % 16) / 4) * 32 + in / 16;
  const int64_t c = (tile % tc) * 4 + in % 4;
  tiled[p] = (r < rows && c < cols) ? sf[r * cols + c] : (uint8_t)0;
}

// one thread per linear scale byte
__global__ __launch_bounds__(256) void k_scales_from_128x4(const uint8_t* __restrict__ tiled,
                                                           uint8_t* __restrict__ sf, int64_t rows, int64_t cols) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= rows * cols) return;
  const int64_t tc = (cols + 3) / 4;
  const int64_t r = q / cols, c = q % cols;
  sf[q] = tiled[((r / 128) * tc + c / 4) * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + c % 4];
}

// 8 x 4 tiles: one thread per byte of the tiled layout (padding written as zero)
__global__ __launch_bounds__(256) void k_scales_to_8x4(const uint8_t* __restrict__ sf, uint8_t* __restrict__ tiled,
                                                       int64_t rows, int64_t cols, int64_t total) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total) return;
  const int64_t tc = (cols + 3) / 4;
  const int64_t tile = p / 32, in = p % 32;
  const int64_t r = (tile / tc) * 8 + in / 4;
  const int64_t c = (tile % tc) * 4 + in % 4;
  tiled[p] = (r < rows && c < cols) ? sf[r * cols + c] : (uint8_t)0;
}

// one thread per linear scale byte
__global__ __launch_bounds__(256) void k_scales_from_8x4(const uint8_t* __restrict__ tiled, uint8_t* __restrict__ sf,
                                                         int64_t rows, int64_t cols) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= rows * cols) return;
  const int64_t tc = (cols + 3) / 4;
  const int64_t r = q / cols, c = q % cols;
  sf[q] = tiled[((r / 8) * tc + c / 4) * 32 + (r % 8) * 4 + c % 4];
}

size_t tiled8x4_bytes(int64_t rows, int64_t K) {
  const int64_t cols = K / 16;
  return (size_t)(((rows + 7) / 8) * 8) * (size_t)(((cols + 3) / 4) * 4);
}

hipError_t launch_scales_to_8x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, hipStream_t stream) {
  const int64_t total = (int64_t)tiled8x4_bytes(rows, K);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_to_8x4, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, sf, tiled, rows,
                     K / 16, total);
  return hipGetLastError();
}

hipError_t launch_scales_from_8x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K, hipStream_t stream) {
  const int64_t n = rows * (K / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_from_8x4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, tiled, sf, rows,
                     K / 16);
  return hipGetLastError();
}

size_t tiled128x4_bytes(int64_t rows, int64_t K) {
  const int64_t cols = K / 16;
  return (size_t)(((rows + 127) / 128) * 128) * (size_t)(((cols + 3) / 4) * 4);
}

hipError_t launch_scales_to_128x4(const uint8_t* sf, uint8_t* tiled, int64_t rows, int64_t K, hipStream_t stream) {
  const int64_t total = (int64_t)tiled128x4_bytes(rows, K);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_to_128x4, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, sf, tiled,
                     rows, K / 16, total);
  return hipGetLastError();
}

hipError_t launch_scales_from_128x4(const uint8_t* tiled, uint8_t* sf, int64_t rows, int64_t K,
                                    hipStream_t stream) {
  const int64_t n = rows * (K / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_from_128x4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, tiled, sf, rows,
                     K / 16);
  return hipGetLastError();
}

}  // namespace nvfp4
