/* Device side of the seeded input generator (test/benchmark infrastructure).
 * Produces the same bf16 bits as dg_host.c for the same key and index. */
#include <hip/hip_runtime.h>
#include <stdint.h>
#define DG_FN __device__ static inline
#include "dg_core.h"

/* Block b of n_blocks: out + b * block_stride gets a rows x cols slice of the
 * tensor keyed keys[b]; element (r, c) has flat index (row0 + r) * ld_full + col0 + c.
 * Stored row-major (out[r * cols + c]) or, with `transposed`, column-major
 * (out[c * rows + r]). */
__global__ void dg_fill_kernel(uint16_t* __restrict__ out, const uint64_t* __restrict__ keys,
                               int64_t block_stride, int64_t row0, int64_t col0, int64_t rows,
                               int64_t cols, int64_t ld_full, float scale, int transposed) {
  const int64_t b = blockIdx.y;
  const uint64_t key = keys[b];
  const int64_t total = rows * cols;
  uint16_t* o = out + b * block_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r, c;
    if (transposed) {
      c = i / rows;
      r = i - c * rows;
    } else {
      r = i / cols;
      c = i - r * cols;
    }
    const uint64_t n = (uint64_t)(row0 + r) * (uint64_t)ld_full + (uint64_t)(col0 + c);
    o[i] = dg_value(key, n, scale);
  }
}

extern "C" int dg_fill_bf16_dev(uint16_t* out, const uint64_t* keys_dev, int n_blocks,
                                int64_t block_stride, int64_t row0, int64_t col0, int64_t rows,
                                int64_t cols, int64_t ld_full, float scale, int transposed,
                                void* stream) {
  if (n_blocks <= 0 || rows <= 0 || cols <= 0) return 0;
  if (n_blocks > 65535) return -1;
  const hipError_t before = hipGetLastError();  // an error left by an earlier call
  if (before != hipSuccess) return -(2000 + (int)before);
  const int threads = 256;
  int64_t per = (rows * cols + threads - 1) / threads;
  int gx = (int)(per < 4096 ? per : 4096);
  hipLaunchKernelGGL(dg_fill_kernel, dim3(gx, n_blocks), dim3(threads), 0, (hipStream_t)stream,
                     out, keys_dev, block_stride, row0, col0, rows, cols, ld_full, scale,
                     transposed);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : -(1000 + (int)e);
}

/* fp8 codes, laid out as dg_fill_kernel lays out bf16 values (row-major only). */
__global__ void dg_fill_fp8_kernel(uint8_t* __restrict__ out, const uint64_t* __restrict__ keys,
                                   int64_t block_stride, int64_t row0, int64_t col0, int64_t rows,
                                   int64_t cols, int64_t ld_full, int32_t mul) {
  const int64_t b = blockIdx.y;
  const uint64_t key = keys[b];
  const int64_t total = rows * cols;
  uint8_t* o = out + b * block_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    const uint64_t n = (uint64_t)(row0 + r) * (uint64_t)ld_full + (uint64_t)(col0 + c);
    o[i] = dg_value_fp8(key, n, mul);
  }
}

extern "C" int dg_fill_fp8_dev(uint8_t* out, const uint64_t* keys_dev, int n_blocks,
                               int64_t block_stride, int64_t row0, int64_t col0, int64_t rows,
                               int64_t cols, int64_t ld_full, int32_t mul, void* stream) {
  if (n_blocks <= 0 || rows <= 0 || cols <= 0) return 0;
  if (n_blocks > 65535) return -1;
  const hipError_t before = hipGetLastError();
  if (before != hipSuccess) return -(2000 + (int)before);
  const int threads = 256;
  int64_t per = (rows * cols + threads - 1) / threads;
  int gx = (int)(per < 4096 ? per : 4096);
  hipLaunchKernelGGL(dg_fill_fp8_kernel, dim3(gx, n_blocks), dim3(threads), 0,
                     (hipStream_t)stream, out, keys_dev, block_stride, row0, col0, rows, cols,
                     ld_full, mul);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : -(1000 + (int)e);
}

extern "C" const char* dg_error_string(int code) {
  int e = -code;
  if (e >= 2000) e -= 2000; else if (e >= 1000) e -= 1000;
  return hipGetErrorString((hipError_t)e);
}
