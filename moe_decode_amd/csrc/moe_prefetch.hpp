// Speculative expert prefetch (gfx950).
//
// Consecutive decode steps route alike, so the experts a layer chose on the
// previous step can be pulled into the caches ahead of the layer's next call
// ("Muse Spark Open Ultrafast: Pushing beyond 1,000 Tokens per second",
// Megakernel internals: prefetching weights into every cache level, and
// speculative expert prefetching).  The kernel reads every byte of the listed
// experts' gate/up and down rows (and, for fp8 experts, their block scales) with
// the default, allocating cache policy, so the lines pass from HBM into the
// 256 MB Infinity Cache that all XCDs share, where the layer's own streaming
// reads of the same rows then hit.  It computes nothing and writes nothing.
//
// Grid: blockIdx.y is the position j in the id list, blockIdx.x strides over
// the expert's weight rows, 16 bytes per lane and kPrefetchBatch independent
// loads in flight per lane; a block whose id is outside [0, E+S) returns at
// once.
#pragma once

#include "moe_device.hpp"

namespace moe {

constexpr int kPrefetchWG = 256;
constexpr int kPrefetchBatch = 8;

struct PrefetchParams {
  const uint8_t* wgu;   // gate/up rows, [E+S] experts of gu_bytes each
  const uint8_t* wd;    // down rows, [E+S] experts of d_bytes each
  const uint8_t* sgu;   // fp8 block scales of gate/up, [E+S] x sgu_bytes (or null)
  const uint8_t* sd;    // fp8 block scales of down, [E+S] x sd_bytes (or null)
  uint64_t gu_bytes, d_bytes, sgu_bytes, sd_bytes;
  // per expert: 16-byte chunks of gate/up and of down rows, 4-byte words of the
  // two scale tensors (0 for bf16 experts)
  uint32_t u_gu, u_d, u_sgu, u_sd;
  const int32_t* ids;   // [gridDim.y] expert ids
  int n_valid;          // E + S
};

__global__ __launch_bounds__(kPrefetchWG) void moe_prefetch_kernel(PrefetchParams p) {
  const int e = p.ids[blockIdx.y];
  if (e < 0 || e >= p.n_valid) return;
  const uint8_t* gu = p.wgu + (size_t)e * p.gu_bytes;
  const uint8_t* dn = p.wd + (size_t)e * p.d_bytes;
  const uint32_t n_w = p.u_gu + p.u_d;  // 16-byte chunks of weight rows
  const uint32_t stride = gridDim.x * kPrefetchWG;
  uint32_t sink = 0;
  for (uint32_t o0 = blockIdx.x * kPrefetchWG + threadIdx.x; o0 < n_w;
       o0 += kPrefetchBatch * stride) {
    // the whole batch is requested before any of it is consumed; a lane past
    // the end re-reads the last chunk, so every load is unconditional
    uint4 v[kPrefetchBatch];
#pragma unroll
    for (int b = 0; b < kPrefetchBatch; ++b) {
      uint32_t o = o0 + (uint32_t)b * stride;
      o = o < n_w ? o : n_w - 1;
      const uint8_t* a = o < p.u_gu ? gu + ((size_t)o << 4) : dn + ((size_t)(o - p.u_gu) << 4);
      v[b] = *reinterpret_cast<const uint4*>(a);
    }
#pragma unroll
    for (int b = 0; b < kPrefetchBatch; ++b) sink ^= v[b].x ^ v[b].y ^ v[b].z ^ v[b].w;
  }
  // fp8 block scales: a few hundred words per expert, read by the first block
  if (blockIdx.x == 0) {
    const uint32_t n_s = p.u_sgu + p.u_sd;
    for (uint32_t o = threadIdx.x; o < n_s; o += kPrefetchWG) {
      const uint8_t* a = o < p.u_sgu ? p.sgu + (size_t)e * p.sgu_bytes + ((size_t)o << 2)
                                     : p.sd + (size_t)e * p.sd_bytes + ((size_t)(o - p.u_sgu) << 2);
      sink ^= *reinterpret_cast<const uint32_t*>(a);
    }
  }
  // consuming the folded bits keeps every load; nothing is stored
  asm volatile("" ::"v"(sink));
}

}  // namespace moe
