// bf16 lm_head GEMV with the greedy argmax folded in (gfx950).
//
// 512-thread workgroups, 8 waves each (about 144 VGPRs: one workgroup per CU at a
// time, the grid of two per CU runs in two rounds; holding the kernel to 128
// VGPRs for two resident workgroups spills in the row loop and is 18 % slower).
// Every wave streams a contiguous range of
// vocabulary row pairs (one row per 32-lane half, 16-byte loads,
// v_dot2_f32_bf16) against the M hidden rows held in LDS, with the next pair's
// loads in flight while the current pair is reduced, and keeps per token row
// its best (logit, lowest index).  A workgroup's bests are published as
// step-tagged words in its own slot of the workspace; the last workgroup to
// finish (two-level counters, so the finishing workgroups' atomics spread
// over eight addresses) collects every slot, takes the largest logit with the
// lowest index, writes the tokens and advances the step
// ("bf16 router gate and lm_head", Ling-3.0-flash on 4 Blackwell GPUs; greedy
// decoding).
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

// 64-bit order of (logit, index): larger logit first, then lower index
__device__ __forceinline__ uint64_t lm_key(float z, int v) {
  return ((uint64_t)f_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
}

// The grid-wide argmax once every wave has left its per-token-row best in
// wbest[wave][row]: each workgroup publishes its bests as step-tagged words in
// its own slot of the workspace and counts itself done in two levels of
// relaxed counters (8 group counters, then one); the last workgroup collects
// every slot (bounded wait), writes token and max logit, and advances the step.
__device__ __forceinline__ void lm_finish(const LmParams& p, uint64_t* wbest, int* flag,
                                          uint32_t tag, int tid) {
  const int G = gridDim.x, g = blockIdx.x, M = p.M;
  uint64_t* slots = reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(p.hdr) +
                                                HDR_LM_SLOT_BYTE);
  if (tid < M) {
    uint64_t k = 0;
    for (int w = 0; w < MOE_LM_WAVES; ++w) {
      const uint64_t c = wbest[w * MOE_MAXM + tid];
      k = c > k ? c : k;
    }
    uint64_t* s = slots + ((size_t)g * MOE_MAXM + tid) * 2;
    st_tag(s, (uint32_t)(k >> 32), tag);
    st_tag(s + 1, (uint32_t)k, tag);
  }
  __syncthreads();
  // count this workgroup done: its group of g % 8, then the groups
  if (tid == 0) {
    const int grp8 = g & 7, in_grp = (G - grp8 + 7) >> 3;
    bool last = false;
    if (add_u32(p.hdr + HDR_LM_DONE_GRP + 32 * grp8, 1u) == (uint32_t)(in_grp - 1))
      last = add_u32(p.hdr + HDR_LM_DONE, 1u) == (uint32_t)((G < 8 ? G : 8) - 1);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;

  // last workgroup: every slot carries this call's tag (bounded wait)
  if (tid < MOE_MAXM) wbest[tid] = 0ull;
  __syncthreads();
  const uint32_t budget = ld_u32(p.hdr + HDR_DEADLINE);
  Waiter wt{p.hdr, now_ticks() + (budget ? budget : kDefaultDeadlineTicks)};
  for (int s = tid; s < G * M; s += MOE_LM_WG) {
    const int gg = s / M, m = s - gg * M;
    const uint64_t* src = slots + ((size_t)gg * MOE_MAXM + m) * 2;
    uint64_t hi = ld_tag(src), lo = ld_tag(src + 1);
    while ((uint32_t)(hi >> 32) != tag || (uint32_t)(lo >> 32) != tag) {
      if (wt.expired()) { record_status(p.hdr, -6 /* MOE_E_TIMEOUT */); break; }
      __builtin_amdgcn_s_sleep(1);
      hi = ld_tag(src);
      lo = ld_tag(src + 1);
    }
    const uint64_t k = ((hi & 0xFFFFFFFFull) << 32) | (lo & 0xFFFFFFFFull);
    atomicMax(reinterpret_cast<unsigned long long*>(wbest + m), (unsigned long long)k);
  }
  __syncthreads();
  if (tid < M) {
    const uint64_t k = wbest[tid];
    p.token[tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    if (p.max_logit) p.max_logit[tid] = key_f((uint32_t)(k >> 32));
  }
  if (tid == 0) {
    for (int c = 0; c < 8; ++c) st_u32(p.hdr + HDR_LM_DONE_GRP + 32 * c, 0u);
    st_u32(p.hdr + HDR_LM_DONE, 0u);
    st_u32(p.hdr + HDR_LM_EPOCH, tag);
  }
}

// MM: token rows the kernel is built for (up to 8; wider calls take the
// matrix-core kernel below)
template <int CPLH, int MM>
__global__ __launch_bounds__(MOE_LM_WG, 2) void moe_lmhead_kernel(LmParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  const uint4* xs4 = reinterpret_cast<const uint4*>(xs);
  uint64_t* wbest = reinterpret_cast<uint64_t*>(lds + ((p.M * p.H * 2 + 15) & ~15));
  int* flag = reinterpret_cast<int*>(wbest + MOE_LM_WAVES * MOE_MAXM);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int M = p.M, H = p.H, H8 = H >> 3;
  const uint32_t tag = ld_u32(p.hdr + HDR_LM_EPOCH) + 1u;
  {
    const uint4* src = reinterpret_cast<const uint4*>(p.h);
    uint4* dst = reinterpret_cast<uint4*>(xs);
    for (int i = tid; i < (M * H) >> 3; i += MOE_LM_WG) dst[i] = src[i];
  }
  __syncthreads();

  const long long NRP = ((long long)p.V + 1) >> 1;
  const long long NW = (long long)G * MOE_LM_WAVES;
  const long long gw = (long long)g * MOE_LM_WAVES + wv;
  const long long rp0 = gw * NRP / NW, rp1 = (gw + 1) * NRP / NW;
  const int grp = lane >> 5, li = lane & 31;

  float best[MM];
  int besti[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) { best[m] = 0.0f; besti[m] = -1; }

  auto load = [&](uint4 (&w)[CPLH], long long rp) __attribute__((always_inline)) {
    const long long v = 2 * rp + grp;
    const uint4* row = reinterpret_cast<const uint4*>(p.w + (size_t)(v < p.V ? v : 0) * H);
#pragma unroll
    for (int q = 0; q < CPLH; ++q) w[q] = ld_weight(row + li + 32 * q);
  };
  auto reduce = [&](const uint4 (&w)[CPLH], long long rp) __attribute__((always_inline)) {
    const long long v = 2 * rp + grp;
    const bool valid = v < p.V;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      if (m < M) {
        float a = 0.0f;
#pragma unroll
        for (int q = 0; q < CPLH; ++q) a = dot8(w[q], xs4[m * H8 + li + 32 * q], a);
        a = group_sum(a, 32);
        if (valid && (besti[m] < 0 || a > best[m])) { best[m] = a; besti[m] = (int)v; }
      }
    }
  };
  // two row pairs in flight per wave: the next pair's loads are issued before
  // the current pair is reduced, unconditionally in the steady-state loop (a
  // load behind a condition would make the waits count only the loads of the
  // path without it, and so wait for the pair in flight too)
  uint4 wa[CPLH], wb[CPLH];
  long long rp = rp0;
  if (rp0 < rp1) load(wa, rp0);
  for (; rp + 2 < rp1; rp += 2) {
    load(wb, rp + 1);
    reduce(wa, rp);
    load(wa, rp + 2);
    reduce(wb, rp + 1);
  }
  if (rp + 1 < rp1) {
    load(wb, rp + 1);
    reduce(wa, rp);
    reduce(wb, rp + 1);
  } else if (rp < rp1) {
    reduce(wa, rp);
  }

  // the wave's best per token row (both halves), then the workgroup's
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    if (m < M) {
      const uint64_t key = besti[m] < 0 ? 0ull : lm_key(best[m], besti[m]);
      const uint64_t k0 = readlane_u64(key, 0), k1 = readlane_u64(key, 32);
      if (lane == 0) wbest[wv * MOE_MAXM + m] = k0 > k1 ? k0 : k1;
    }
  }
  __syncthreads();
  lm_finish(p, wbest, flag, tag, tid);
}

// The same GEMV and argmax on the matrix cores, for several token rows: the
// logits of M token rows over V vocabulary rows are a dense [V x H] x [H x M]
// contraction, M FLOP per weight byte, which at M >= 6 keeps the vector ALUs
// busier than the weight stream allows.  One workgroup per CU, 8 waves; each
// wave takes a contiguous range of 16-row vocabulary tiles and multiplies
// each tile by the token rows with v_mfma_f32_16x16x32_bf16: the tile's rows
// are the 16 rows of A (lane l: vocabulary row l % 16), the token rows the 16
// columns of B (lane l: token row l % 16, repeating row 0 past M; those
// columns are ignored).  A row is read in 64-element super-chunks, one 128-byte
// line: lane group q = l / 16 loads its 16 bytes at elements 8q and 32 + 8q,
// which feed two MFMAs; B is read from LDS at the same elements, so both
// operands sum over the same k in the same order for every row.  NB
// super-chunks form one batch of loads, and the next batch is in flight while
// the current one is multiplied.  x sits in LDS with a row stride of H + 8
// elements, which keeps the 16 token rows' 16-byte reads on distinct banks.
template <int NB>
__global__ __launch_bounds__(MOE_LM_WG, 1) void moe_lmhead_mfma_kernel(LmParams p) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __align__(16) unsigned char lds[];
  const int M = p.M, H = p.H, V = p.V, XS = H + 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  uint64_t* wbest = reinterpret_cast<uint64_t*>(lds + ((M * XS * 2 + 15) & ~15));
  int* flag = reinterpret_cast<int*>(wbest + MOE_LM_WAVES * MOE_MAXM);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const uint32_t tag = ld_u32(p.hdr + HDR_LM_EPOCH) + 1u;
  {
    const int H8 = H >> 3;
    const uint4* src = reinterpret_cast<const uint4*>(p.h);
    for (int i = tid; i < M * H8; i += MOE_LM_WG) {
      const int m = i / H8, c = i - m * H8;
      *reinterpret_cast<uint4*>(xs + m * XS + 8 * c) = src[i];
    }
  }
  __syncthreads();

  const int NT = (V + 15) >> 4;            // 16-row tiles
  const int NBT = (H >> 6) / NB;           // batches per tile
  const long long NW = (long long)G * MOE_LM_WAVES;
  const long long gw = (long long)g * MOE_LM_WAVES + wv;
  const int t0 = (int)(gw * NT / NW), t1 = (int)((gw + 1) * NT / NW);
  const int S = (t1 - t0) * NBT;           // batches of this wave
  // Loads read whole 128-byte lines: lane l takes row l & 7 of a half tile and
  // 16-byte chunk l >> 3 of each 128-byte super-chunk (w[2c]: rows 0-7 of the
  // tile, w[2c + 1]: rows 8-15).  In the matrix instruction lane l is row
  // l % 16 of k-group l / 16, so that register holds, for matrix rows i < 8,
  // row i at chunk 2g and, for i >= 8, row i - 8 at chunk 2g + 1.  Each
  // register therefore feeds two products, one with x at the even chunks
  // (valid in matrix rows 0-7) and one at the odd chunks (valid in rows 8-15);
  // the two halves of a row are added at the end of the tile.  Every row sums
  // the same chunks in the same order.
  const int i8 = lane & 7, c8 = lane >> 3;
  const int i16 = lane & 15, q = lane >> 4;
  const uint16_t* xr = xs + (i16 < M ? i16 : 0) * XS + 16 * q;

  auto load = [&](uint4 (&w)[2 * NB], int s) __attribute__((always_inline)) {
    const int tl = s / NBT, bt = s - tl * NBT;
    const int va = 16 * (t0 + tl) + i8, vb = va + 8;
    const uint4* ra = reinterpret_cast<const uint4*>(p.w + (size_t)(va < V ? va : V - 1) * H) +
                      (size_t)bt * NB * 8 + c8;
    const uint4* rb = reinterpret_cast<const uint4*>(p.w + (size_t)(vb < V ? vb : V - 1) * H) +
                      (size_t)bt * NB * 8 + c8;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      w[2 * c] = ld_weight(ra + 8 * c);
      w[2 * c + 1] = ld_weight(rb + 8 * c);
    }
  };
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 ae = zero4, ao = zero4, be = zero4, bo = zero4;
  uint64_t best = 0ull;
  auto mul = [&](const uint4 (&w)[2 * NB], int s) __attribute__((always_inline)) {
    const int tl = s / NBT, bt = s - tl * NBT;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const uint16_t* xb = xr + 64 * (bt * NB + c);
      const bf16x8 xe = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb));
      const bf16x8 xo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb + 8));
      const bf16x8 wa = __builtin_bit_cast(bf16x8, w[2 * c]);
      const bf16x8 wb = __builtin_bit_cast(bf16x8, w[2 * c + 1]);
      ae = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xe, ae, 0, 0, 0);
      ao = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xo, ao, 0, 0, 0);
      be = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xe, be, 0, 0, 0);
      bo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xo, bo, 0, 0, 0);
    }
    if (bt == NBT - 1) {
      // tile done.  Lane l holds matrix rows 4q .. 4q + 3 of column l % 16:
      // even-chunk sums of half-tile rows 4q + j for q < 2, odd-chunk sums of
      // rows 4(q - 2) + j for q >= 2; lanes l and l ^ 32 add their halves.
      // Lanes q < 2 then report tile rows 4q + j, lanes q >= 2 rows 8 + 4(q - 2) + j.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pa = q < 2 ? ae[j] : ao[j];
        const float pb = q < 2 ? be[j] : bo[j];
        const float za = pa + __shfl_xor(pa, 32);
        const float zb = pb + __shfl_xor(pb, 32);
        const float z = q < 2 ? za : zb;
        const int v = 16 * (t0 + tl) + (q < 2 ? 4 * q + j : 8 + 4 * (q - 2) + j);
        if (i16 < M && v < V) {
          const uint64_t k = lm_key(z, v);
          best = k > best ? k : best;
        }
      }
      ae = zero4;
      ao = zero4;
      be = zero4;
      bo = zero4;
    }
  };
  // two batches in flight: the steady-state loop issues its loads
  // unconditionally (a load behind a condition would make every wait in the
  // loop count only the loads of the path without it, and so wait for the
  // batch in flight too); the last one or two batches follow it
  uint4 wa[2 * NB], wb[2 * NB];
  int s = 0;
  if (S > 0) load(wa, 0);
  for (; s + 2 < S; s += 2) {
    load(wb, s + 1);
    mul(wa, s);
    load(wa, s + 2);
    mul(wb, s + 1);
  }
  if (s + 1 < S) {
    load(wb, s + 1);
    mul(wa, s);
    mul(wb, s + 1);
  } else if (s < S) {
    mul(wa, s);
  }

  // the wave's best per token row: lanes r, r + 16, r + 32, r + 48 hold row r
  {
    uint64_t o = __shfl_xor(best, 16);
    best = o > best ? o : best;
    o = __shfl_xor(best, 32);
    best = o > best ? o : best;
    if (lane < M) wbest[wv * MOE_MAXM + lane] = best;
  }
  __syncthreads();
  lm_finish(p, wbest, flag, tag, tid);
}

}  // namespace moe
