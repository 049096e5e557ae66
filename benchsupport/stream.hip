// Reference kernels for bench.py (measurement infrastructure, not the MoE path):
//  bs_stream_read: reads a buffer once, the way the layer kernel streams expert
//                  rows: each wave takes whole 16 KiB chunks, one 1 KiB
//                  non-temporal load per instruction (16 bytes a lane), all 16
//                  loads of a chunk in flight before any is consumed.  Its rate
//                  over a buffer far larger than the caches is the achievable
//                  streaming-read ceiling the layer kernel is held against;
//  bs_copy:        copies a buffer of known size (the reference against which
//                  rocprofv3 FETCH_SIZE / WRITE_SIZE are scaled to bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int bs_u32x4 __attribute__((ext_vector_type(4)));

constexpr int BS_LOADS = 16;                          // 1 KiB loads per chunk
constexpr size_t BS_CHUNK16 = (size_t)BS_LOADS * 64;  // chunk size in 16-byte units

__global__ __launch_bounds__(512) void bs_stream_read_kernel(const bs_u32x4* __restrict__ p,
                                                             size_t n16, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const size_t n_waves = (size_t)gridDim.x * (blockDim.x >> 6);
  const size_t n_chunks = n16 / BS_CHUNK16;
  uint32_t acc = 0;
  for (size_t c = wave; c < n_chunks; c += n_waves) {
    const bs_u32x4* q = p + c * BS_CHUNK16 + lane;   // last index read: c*1024 + 15*64 + 63
    bs_u32x4 v[BS_LOADS];
#pragma unroll
    for (int j = 0; j < BS_LOADS; ++j) v[j] = __builtin_nontemporal_load(q + j * 64);
#pragma unroll
    for (int j = 0; j < BS_LOADS; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // the tail past the last whole chunk, 16 bytes a thread
  for (size_t i = n_chunks * BS_CHUNK16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x) {
    const bs_u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never: keeps the loads alive
}

__global__ __launch_bounds__(256) void bs_copy_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// p: device buffer of `bytes` (a multiple of 16); sink: device array of at least
// `blocks` words, written only in the practically impossible case above.
extern "C" int bs_stream_read(const void* p, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!p || !sink || bytes % 16 || blocks <= 0) return -1;
  hipLaunchKernelGGL(bs_stream_read_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     (const bs_u32x4*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bs_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks <= 0) return -1;
  hipLaunchKernelGGL(bs_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
