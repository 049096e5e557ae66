// Device-side building blocks for the gfx950 kernels of libmoedecode.
//
// Wave64 throughout.  Weight rows are streamed with 16-byte loads, eight bf16
// values per lane per load, and reduced with v_dot2_f32_bf16 (two bf16
// products accumulated in fp32 per instruction).  Partial sums are combined
// across the lanes of a row with DPP row operations and ds_swizzle, never
// through LDS.  Values that cross workgroups carry a step tag in the same
// 64-bit word ("step-tagged values", SGLang Low-Latency Mode, AMD Low-Latency
// Kernels): a consumer accepts a word once its tag equals the current step, so
// no flag, fence or reset is needed between steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WG 512                  // threads per workgroup of the fused layer kernel
#define MOE_WAVES (MOE_WG / 64)
#define MOE_MAXM 16                 // at most sixteen token rows (a 16-token tree verify)
#define MOE_LM_WG 512               // threads per workgroup of the lm_head kernel
#define MOE_LM_WAVES (MOE_LM_WG / 64)
#define MOE_LM_MAX_GRID 512         // lm_head workgroups, at most (one result slot each)

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- workspace header (uint32 word offsets; hot words on separate 128 B lines)
enum : int {
  HDR_XREAD0 = 32,      // layer calls with an even tag: workgroups that finished reading x_in
  HDR_XREAD1 = 64,      // the same for odd tags (each call clears the other one for the next)
  HDR_STATUS = 96,      // sticky device status (moe_status)
  HDR_FLAGS = 128,      // debug flags
  HDR_DEADLINE = 129,   // wait budget in 100 MHz ticks (0 = default)
  HDR_LM_DONE = 160,    // lm_head: groups of workgroups finished
  HDR_LM_EPOCH = 192,   // lm_head: calls completed; tag of a call = epoch + 1
  HDR_LM_DONE_GRP = 512,  // lm_head: workgroups finished per group of g % 8 (8 words, 32 apart)
  HDR_WORDS = 1024,     // control words: 4 KiB
  HDR_STAMPS = 1024,    // phase stamps: [256 workgroups][32] u64 after the control words
  STAMP_WG = 256,
  STAMP_SLOTS = 32,
  // lm_head result slots after the stamps: [MOE_LM_MAX_GRID][MOE_MAXM] x 2 tagged words
  HDR_LM_SLOT_BYTE = HDR_WORDS * 4 + STAMP_WG * STAMP_SLOTS * 8,
  HDR_BYTES = HDR_LM_SLOT_BYTE + MOE_LM_MAX_GRID * MOE_MAXM * 2 * 8
};

// debug flags of a workspace (moe_workspace_debug); DBG_NOT_RESIDENT is seen by
// the host only: the layer kernel's occupancy check then reports no room
enum : uint32_t { DBG_NO_ROUTER_PUBLISH = 1u, DBG_STAMPS = 2u, DBG_NOT_RESIDENT = 4u };

constexpr uint32_t kDefaultDeadlineTicks = 20000000u;  // 200 ms at 100 MHz

// ---- bf16 <-> fp32
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> one word of two bf16 (lo in bits 0-15), round to nearest even
// (finite inputs): one v_cvt_pk_bf16_f32.
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf(float lo, float hi) {
  const moe_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, moe_bf16x2));
}

// acc + sum_{i<8} w_i * x_i over eight bf16 pairs packed in two uint4.
__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x),
                                        __builtin_bit_cast(bf16x2, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y),
                                        __builtin_bit_cast(bf16x2, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z),
                                        __builtin_bit_cast(bf16x2, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w),
                                        __builtin_bit_cast(bf16x2, x.w), acc, false);
  return acc;
}

// ---- cross-lane primitives
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// exchange with lane ^ 16 inside each 32-lane half (ds_swizzle bitmask mode)
__device__ __forceinline__ float swz16_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ uint32_t swz16_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_u<CTRL>((uint32_t)u), hi = dpp_u<CTRL>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint64_t)lo);
}
__device__ __forceinline__ double swz16_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = swz16_u((uint32_t)u), hi = swz16_u((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint64_t)lo);
}
// Sum of a double over the 64 lanes (the same butterfly as group_sum); the
// result is wave-uniform.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  v += swz16_d(v);
  const uint64_t u = readlane_u64(__builtin_bit_cast(uint64_t, v), 0);
  const uint64_t w = readlane_u64(__builtin_bit_cast(uint64_t, v), 32);
  return __builtin_bit_cast(double, u) + __builtin_bit_cast(double, w);
}

// Sum over each group of `lpr` consecutive lanes (lpr = 8, 16, 32 or 64);
// every lane of a group receives the group's sum.  lpr is wave-uniform.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  if (lpr >= 16) v += dpp_f<0x140>(v);
  if (lpr >= 32) v += swz16_f(v);
  if (lpr >= 64) v = readlane_f(v, 0) + readlane_f(v, 32);
  return v;
}

// Wave-wide maximum of an unsigned key; the result is wave-uniform.  All in
// DPP (quad swaps, half-row and row mirrors, then the row broadcasts that
// carry row 0 into row 1, row 2 into row 3 and rows 0-1 into rows 2-3), so lane
// 63 ends with the maximum; one readlane makes it uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving map of an fp32 value to an unsigned key (-0 maps as +0).
__device__ __forceinline__ uint32_t f_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---- step-tagged words (agent-scope relaxed atomics: coherent across XCDs)
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t lo, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)lo, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Weight rows are read once per call, so their 16-byte loads carry the
// non-temporal (streaming) policy: tens of megabytes of weights then go by
// without displacing the few lines that are reused from L2 within and between
// calls, the kernel's own code first among them, then the tagged exchange
// words.  The megakernel of "Muse Spark Open Ultrafast: Pushing beyond 1,000
// Tokens per second", section "Megakernel internals", marks its weight
// streams evict-first for the same reason and reports the cost of code
// refetches in its instruction-cache part.
#ifndef MOE_WEIGHT_NT
#define MOE_WEIGHT_NT 1
#endif
__device__ __forceinline__ uint4 ld_weight(const uint4* p) {
#if MOE_WEIGHT_NT
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Deadline of every wait in one call ("every wait has a deadline", SGLang
// Low-Latency Mode, AMD Low-Latency Kernels).  A missed deadline records
// MOE_E_TIMEOUT in the workspace and makes the waiter give up; all later
// waits of the call then give up at once, so every wave reaches the end.
struct Waiter {
  uint32_t* hdr;
  uint64_t deadline;
  __device__ bool expired() const { return now_ticks() > deadline; }
};

__device__ __forceinline__ void record_status(uint32_t* hdr, int st) {
  // first error wins
  uint32_t expected = 0u;
  __hip_atomic_compare_exchange_strong(hdr + HDR_STATUS, &expected, (uint32_t)st,
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the word at p carries `tag`; returns false on a missed deadline.
__device__ __forceinline__ bool wait_tag(const uint64_t* p, uint32_t tag, const Waiter& w,
                                         uint64_t& out) {
  uint64_t v = ld_tag(p);
  if ((uint32_t)(v >> 32) == tag) { out = v; return true; }
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    v = ld_tag(p);
    if ((uint32_t)(v >> 32) == tag) { out = v; return true; }
    if (w.expired()) {
      record_status(w.hdr, -6 /* MOE_E_TIMEOUT */);
      out = 0;
      return false;
    }
  }
}

}  // namespace moe
