// bf16 lm_head GEMV with the greedy argmax folded in (gfx950).
//
// Every wave streams a contiguous range of vocabulary row pairs (one row per
// 32-lane half, 16-byte loads, v_dot2_f32_bf16) against the M hidden rows held
// in LDS and keeps, per token row, its best (logit, lowest index).  The
// workgroups' bests meet in a 64-bit atomic max on (order-preserving logit key
// << 32 | ~index), so the largest logit wins and equal logits go to the lowest
// vocabulary index; the last workgroup to finish writes the tokens and resets
// the keys for the next call ("bf16 router gate and lm_head", Ling-3.0-flash
// on 4 Blackwell GPUs; greedy decoding).
#pragma once

#include "moe_device.hpp"

namespace moe {

struct LmParams {
  int M, H, V;
  const uint16_t* h;
  const uint16_t* w;
  int32_t* token;
  float* max_logit;
  uint32_t* hdr;
};

template <int CPLH>
__global__ __launch_bounds__(MOE_LM_WG) void moe_lmhead_kernel(LmParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  const uint4* xs4 = reinterpret_cast<const uint4*>(xs);
  uint64_t* wbest = reinterpret_cast<uint64_t*>(lds + ((p.M * p.H * 2 + 15) & ~15));

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nwaves = MOE_LM_WG / 64;
  const int M = p.M, H = p.H, H8 = H >> 3;
  {
    const uint4* src = reinterpret_cast<const uint4*>(p.h);
    uint4* dst = reinterpret_cast<uint4*>(xs);
    for (int i = tid; i < (M * H) >> 3; i += MOE_LM_WG) dst[i] = src[i];
  }
  __syncthreads();

  const long long NRP = ((long long)p.V + 1) >> 1;
  const long long NW = (long long)gridDim.x * nwaves;
  const long long gw = (long long)blockIdx.x * nwaves + wv;
  const long long rp0 = gw * NRP / NW, rp1 = (gw + 1) * NRP / NW;
  const int grp = lane >> 5, li = lane & 31;

  float best[MOE_MAXM];
  int besti[MOE_MAXM];
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) { best[m] = 0.0f; besti[m] = -1; }

  for (long long rp = rp0; rp < rp1; ++rp) {
    const long long v = 2 * rp + grp;
    const bool valid = v < p.V;
    const uint4* row = reinterpret_cast<const uint4*>(p.w + (size_t)(valid ? v : 0) * H);
    uint4 w[CPLH];
#pragma unroll
    for (int q = 0; q < CPLH; ++q) w[q] = row[li + 32 * q];
#pragma unroll
    for (int m = 0; m < MOE_MAXM; ++m) {
      if (m < M) {
        float a = 0.0f;
#pragma unroll
        for (int q = 0; q < CPLH; ++q) a = dot8(w[q], xs4[m * H8 + li + 32 * q], a);
        a = group_sum(a, 32);
        if (valid && (besti[m] < 0 || a > best[m])) { best[m] = a; besti[m] = (int)v; }
      }
    }
  }
  // combine the two row groups of the wave, then the waves of the workgroup
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) {
    if (m < M) {
      const uint64_t key = besti[m] < 0 ? 0ull
                                        : (((uint64_t)f_key(best[m]) << 32) |
                                           (uint64_t)(0xFFFFFFFFu - (uint32_t)besti[m]));
      const uint64_t k0 = readlane_u64(key, 0), k1 = readlane_u64(key, 32);
      if (lane == 0) wbest[wv * MOE_MAXM + m] = k0 > k1 ? k0 : k1;
    }
  }
  __syncthreads();
  // One thread publishes the workgroup's keys and then counts itself done with
  // release ordering; the last workgroup's acquire sees every key.
  if (tid == 0) {
    uint64_t* keys = reinterpret_cast<uint64_t*>(p.hdr + HDR_LM_KEYS);
    for (int m = 0; m < M; ++m) {
      uint64_t k = 0;
      for (int w = 0; w < nwaves; ++w) {
        const uint64_t c = wbest[w * MOE_MAXM + m];
        k = c > k ? c : k;
      }
      if (k) __hip_atomic_fetch_max(keys + m, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t old = __hip_atomic_fetch_add(p.hdr + HDR_LM_DONE, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      for (int m = 0; m < M; ++m) {
        const uint64_t k = __hip_atomic_load(keys + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.token[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
        if (p.max_logit) p.max_logit[m] = key_f((uint32_t)(k >> 32));
        __hip_atomic_store(keys + m, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      st_u32(p.hdr + HDR_LM_DONE, 0u);
    }
  }
}

}  // namespace moe
