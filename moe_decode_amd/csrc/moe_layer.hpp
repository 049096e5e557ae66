// The fused MoE layer / chain kernel for gfx950.
//
// One persistent launch runs one or several MoE layers; one workgroup per CU,
// all resident for the whole call.  Per layer:
//
//   P0  stage the layer input x [M][H] in LDS (layer 0 from the caller's
//       buffer, later layers from step-tagged residual words); under the
//       pre-norm chain keep this workgroup's rows of h_l for the residual and
//       replace x by bf16(RMSNorm(h_l)).
//   P1  router GEMV rows, spread over the waves of the GPU; logits are
//       published as step-tagged words.  The first rows are requested before x
//       arrives ("weights that do not depend on routing load before their
//       inputs arrive", SGLang Low-Latency Mode, AMD Low-Latency Kernels).
//   P4  every workgroup reads all logits and computes the softmax top-k
//       itself, so no second device-wide hop is needed.
//   P5  union of the rows' choices: a bitmap over experts plus population
//       counts gives each selected expert its slot with no scan over experts or
//       sort (SGLang Low-Latency Mode, item 3: at most eight rows); the shared
//       expert joins as one more slot that every row selects with gate 1.
//   P6  every slot's gate/up rows, cut into one equal, contiguous share of
//       (slot, intermediate pair) units per workgroup: gate/up GEMV + SwiGLU,
//       the results kept in LDS.
//   P7  the same workgroup's share of the down projection: over its own
//       intermediate indices, for all H outputs (split-K; the down weights are
//       stored transposed so each intermediate index is one contiguous row),
//       scaled by the row's gate and published as tagged fp32 partial sums.
//       No SwiGLU value crosses workgroups, and each workgroup streams its
//       gate/up and down weights back to back.
//   P8  each workgroup owns a slice of output rows: it sums every partial for
//       those rows in a fixed order and rounds once (or adds the residual with
//       one rounding, or writes the fp32 partial).
//
// Every selected expert's weights stream from HBM exactly once per call, for
// all the token rows that chose it; no two workgroups read the same weights.
#pragma once

#include "moe_device.hpp"

namespace moe {

#ifndef MOE_MAX_LAYERS
#define MOE_MAX_LAYERS 64
#endif

constexpr int kMaxPK = MOE_MAXM * 16;  // max (routed expert, row) pairs = M * K
constexpr int kMaxSlots = kMaxPK + 1;  // routed slots plus the shared expert
constexpr int kMaxWG = 256;            // workgroups of the layer kernel, at most

struct LayerW {
  const uint16_t* wr;   // [E][H]
  const uint16_t* wgu;  // [E+S][2I][H]
  const uint16_t* wd;   // [E+S][I][H]: each expert's down projection, transposed
};

enum : uint32_t {
  F_RESIDUAL = 1u,     // chain: h_{l+1} = bf16(h_l + acc)
  F_OUT_F32 = 2u,      // write the unrounded fp32 acc
  F_TOPK_IN = 4u,      // routing comes from the caller (experts only)
  F_ROUTER_ONLY = 8u,  // router + top-k only
  F_ALIAS = 16u,       // out overlaps x_in: wait until every workgroup has read x_in
  F_PRENORM = 32u,     // chain: each layer's MoE input is bf16(RMSNorm(h_l)), unit gain
};

constexpr float kRmsEps = 1e-6f;

// NL: layer weight slots carried in the kernel arguments (1 for single-layer
// calls keeps the argument block small; the chain takes MOE_MAX_LAYERS).
template <int NL>
struct ParamsT {
  int H, E, K, I, S, M, L;
  uint32_t flags;
  int nr_max;         // output rows owned by one workgroup, at most
  int uw_max;         // gate/up units of one workgroup, at most
  int zcap;           // contributions staged in LDS per round
  // LDS byte offsets
  int lds_xs, lds_lg, lds_hw, lds_z, lds_small;
  const uint16_t* x_in;
  void* out;
  const int32_t* tk_idx_in;
  const float* tk_gate_in;
  int32_t* tk_idx_out;   // [L][M][K] (or [M][K])
  float* tk_gate_out;    // [M][K]
  float* logits_out;     // [M][E]
  uint16_t* h_all;       // [L+1][M][H] residual stream per layer (optional)
  uint32_t* hdr;
  uint64_t* lg_buf;      // [L][M][E]              tagged fp32 logits
  uint64_t* part_buf;    // [L][kMaxWG][2][M][H]   tagged fp32 gate-scaled partial down outputs
  uint64_t* res_buf;     // [L+1][M][H/2]          tagged bf16 pairs, residual stream
  LayerW lw[NL];
};

struct Small {
  int nU, nP, abort_flag, ncontrib;
  int tk_idx[kMaxPK];
  float tk_gate[kMaxPK];
  int upos[kMaxPK];          // routed slot of (row, rank), -1 if skipped
  int uexp[kMaxSlots];       // expert id of slot r (slot U: the shared expert, id E)
  uint32_t umask[kMaxSlots]; // rows that chose slot r
  uint32_t bm[32];           // expert bitmap (E <= 1024)
  int bpre[32];              // population-count prefix per bitmap word
  float rn[MOE_MAXM];        // RMSNorm scale per token row
  alignas(16) uint32_t gmax[MOE_MAXM * MOE_WAVES];  // top-k: group maxima per row
  int ccount[MOE_MAXM];                 // top-k: candidates per row
  alignas(16) uint64_t cand[MOE_MAXM * 64];  // top-k: (key << 32 | ~expert) candidates
  float slot_gate[kMaxSlots * MOE_MAXM];     // gate of (slot, token row); 1 for the shared expert
  int wtot[MOE_WAVES * MOE_MAXM];            // contribution counts per wave and row
  int cstart[MOE_MAXM + 1];                  // first contribution of each token row
  uint16_t clist[kMaxWG * 2 * MOE_MAXM];     // contributions: workgroup << 4 | piece << 3 | row
  float osum[MOE_MAXM * 64];                 // combined outputs of the owned rows
  uint16_t hres[MOE_MAXM * 64];  // residual input h_l of this workgroup's output rows
};

__device__ __forceinline__ float swiglu(float a, float b) {
  const float s = a / (1.0f + expf(-a));
  return s * b;
}

// Inclusive prefix sum over the 64 lanes, all in DPP: shifts by 1, 2, 4 and
// 8 inside each 16-lane row, then row 0's total broadcast into row 1 (and row
// 2's into row 3), then row 1's running total into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Copy n tagged words into LDS (low 32 bits) once each carries `tag`.  Each
// thread requests a whole batch of B independent words before checking any,
// and re-requests every word of the batch still carrying an older tag together,
// so a stage costs about one load latency per poll round rather than one per
// word.  addr(i) gives the source word of element i.  Returns false on a
// missed deadline (recorded in the workspace status).
template <int B, typename Addr>
__device__ __forceinline__ bool stage_tagged(int n, uint32_t* dst32, uint32_t tag,
                                             const Waiter& wt, int tid, Addr addr) {
  const uint64_t ready = (uint64_t)tag << 32;
  for (int base = tid; base < n; base += B * MOE_WG) {
    uint64_t v[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = base + b * MOE_WG;
      v[b] = i < n ? ld_tag(addr(i)) : ready;
    }
    for (;;) {
      bool all = true;
#pragma unroll
      for (int b = 0; b < B; ++b) all = all && (uint32_t)(v[b] >> 32) == tag;
      if (all) break;
      if (wt.expired()) {
        record_status(wt.hdr, -6 /* MOE_E_TIMEOUT */);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int b = 0; b < B; ++b)
        if ((uint32_t)(v[b] >> 32) != tag) v[b] = ld_tag(addr(base + b * MOE_WG));
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = base + b * MOE_WG;
      if (i < n) dst32[i] = (uint32_t)v[b];
    }
  }
  return true;
}

// ---------------------------------------------------------------- streaming units
//
// A row unit is two weight rows of H bf16 values, the first on lanes 0-31 and
// the second on lanes 32-63, CPLH 16-byte loads per lane; every unit requests
// all its weights before using any, and the first router unit of a layer is
// requested before the layer waits for its input.

template <int CPLH>
struct RowRegs {
  uint4 w[CPLH];
};

template <int CPLH>
__device__ __forceinline__ void load_rows(RowRegs<CPLH>& r, const uint16_t* row0,
                                          const uint16_t* row1, int lane) {
  const uint4* src = reinterpret_cast<const uint4*>((lane >> 5) ? row1 : row0);
  const int li = lane & 31;
#pragma unroll
  for (int q = 0; q < CPLH; ++q) r.w[q] = src[li + 32 * q];
}

// Dot product of each half-wave's row with token row m (all lanes of a half
// receive the sum).
template <int CPLH>
__device__ __forceinline__ float dot_rows(const RowRegs<CPLH>& r, const uint4* xs4, int H8, int m,
                                          int lane) {
  const int li = lane & 31;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < CPLH; ++q) acc = dot8(r.w[q], xs4[m * H8 + li + 32 * q], acc);
  return group_sum(acc, 32);
}

// P1 item `it`: router rows 2it and 2it + 1 (the first on lanes 0-31, the
// second on lanes 32-63).
template <int CPLH, class P>
__device__ __forceinline__ void p1_load(const P& p, int l, int it, RowRegs<CPLH>& A, int lane) {
  const int e0 = 2 * it, e1 = (2 * it + 1 < p.E) ? 2 * it + 1 : 2 * it;
  load_rows<CPLH>(A, p.lw[l].wr + (size_t)e0 * p.H, p.lw[l].wr + (size_t)e1 * p.H, lane);
}

template <int CPLH, class P>
__device__ __forceinline__ void p1_compute(const P& p, int l, int it, const RowRegs<CPLH>& A,
                                           const uint4* xs4, uint32_t tag, int lane,
                                           uint32_t dbg) {
  const int H8 = p.H >> 3;
  const int e = 2 * it + (lane >> 5);
  const bool publish = e < p.E && (lane & 31) == 0 && !(dbg & DBG_NO_ROUTER_PUBLISH);
#pragma unroll 1
  for (int m = 0; m < p.M; ++m) {
    const float acc = dot_rows<CPLH>(A, xs4, H8, m, lane);
    if (publish) st_tag(p.lg_buf + ((size_t)l * p.M + m) * p.E + e, __float_as_uint(acc), tag);
  }
}

// acc[k] += h * w_k for the eight bf16 values of w (each product exact in fp32).
__device__ __forceinline__ void fma8(float* acc, const uint4& w, float h) {
  acc[0] = __builtin_fmaf(h, bf_lo(w.x), acc[0]);
  acc[1] = __builtin_fmaf(h, bf_hi(w.x), acc[1]);
  acc[2] = __builtin_fmaf(h, bf_lo(w.y), acc[2]);
  acc[3] = __builtin_fmaf(h, bf_hi(w.y), acc[3]);
  acc[4] = __builtin_fmaf(h, bf_lo(w.z), acc[4]);
  acc[5] = __builtin_fmaf(h, bf_hi(w.z), acc[5]);
  acc[6] = __builtin_fmaf(h, bf_lo(w.w), acc[6]);
  acc[7] = __builtin_fmaf(h, bf_hi(w.w), acc[7]);
}

// ---------------------------------------------------------------- P4 / P5

// Softmax top-k ("softmax top-k with renormalised gates", Low-Latency MoE
// Decode, routing step).  The selection order is: larger logit first, lower
// expert index first among equal logits.
//
// Fast path (E <= 512 experts, one per thread, and K no larger than the number
// of 64-expert groups): every wave takes the maximum of its group of 64
// experts for each row; the smallest of a row's group maxima, tau, has at
// least (groups) >= K experts at or above it, so the row's K winners are among
// the experts with key >= tau.  Those candidates (typically 10-20 of 512) are
// compacted into LDS and each one's rank is counted directly against the
// others; ranks below K are the selection.  No step is a serial round over K.
// A row with more than 64 candidates, and every row outside the fast path's
// shapes, takes the plain method: K rounds of a wave-wide maximum.
//
// K rounds over one row held by one wave, PER keys per lane in lane-major
// blocks (lane L holds experts L*PER .. L*PER+PER-1); key 0 marks "no expert".
template <int PER>
__device__ __forceinline__ void select_rounds(const float* lr, int E, int K, int* out, int lane) {
  uint32_t keys[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * PER + i;
    keys[i] = e < E ? f_key(lr[e]) : 0u;
  }
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    uint32_t lb = 0u;
    int li = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (keys[i] > lb) { lb = keys[i]; li = i; }
    const uint32_t wmax = wave_max_u32(lb);
    const uint64_t ball = __ballot(lb == wmax && lb != 0u);
    const int wl = ball ? (int)__builtin_ctzll(ball) : 0;
    const int wi = __builtin_amdgcn_readlane(li, wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == wi) keys[i] = 0u;
    }
    if (lane == 0) out[k] = wmax ? wl * PER + wi : -1;
  }
}

__device__ __forceinline__ void select_row_plain(const float* lr, int E, int K, int* out,
                                                 int lane) {
  const int per = (E + 63) >> 6;
  if (per <= 1) select_rounds<1>(lr, E, K, out, lane);
  else if (per <= 2) select_rounds<2>(lr, E, K, out, lane);
  else if (per <= 4) select_rounds<4>(lr, E, K, out, lane);
  else if (per <= 8) select_rounds<8>(lr, E, K, out, lane);
  else select_rounds<16>(lr, E, K, out, lane);
}

// Gates of row m from its K selected experts (tk_idx written by this wave):
// p_k = exp(l_k - l_max) renormalised over the K (the full softmax
// denominator cancels in the renormalisation); lane k holds rank k.
__device__ __forceinline__ void gates_from_idx(const float* lr, int K, Small* sm, int m,
                                               int lane) {
  const int ek = lane < K ? sm->tk_idx[m * K + lane] : 0;
  const float v0 = lr[sm->tk_idx[m * K]];
  const float pk = lane < K ? expf(lr[ek] - v0) : 0.0f;
  const float s = group_sum(pk, 64);
  if (lane < K) sm->tk_gate[m * K + lane] = pk / s;
}

// Fast path for exactly MM token rows (see above).
template <int MM>
__device__ __forceinline__ void topk_fast(const float* lgs, Small* sm, int E, int K, int nW,
                                          int tid, int wv, int lane) {
  // (a) every wave: its group maximum, for every row
  uint32_t key[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) key[m] = tid < E ? f_key(lgs[m * E + tid]) : 0u;
  uint32_t mine = 0u;
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    const uint32_t gm = wave_max_u32(key[m]);
    mine = lane == m ? gm : mine;
  }
  if (lane < MM) sm->gmax[lane * MOE_WAVES + wv] = mine;
  if (tid < MOE_MAXM) sm->ccount[tid] = 0;
  __syncthreads();
  // (b) lane m: tau of row m = its smallest group maximum; every row's
  //     candidates (key >= tau) are packed as (key << 32 | ~expert), so that
  //     one unsigned 64-bit comparison orders them as the selection does
  uint32_t tau_l = 0u;
  if (lane < MM) {
    const uint4 ga = *reinterpret_cast<const uint4*>(sm->gmax + lane * MOE_WAVES);
    const uint4 gb = *reinterpret_cast<const uint4*>(sm->gmax + lane * MOE_WAVES + 4);
    const uint32_t g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
    tau_l = g8[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) tau_l = w < nW ? min(tau_l, g8[w]) : tau_l;
  }
  uint64_t ball[MM];
  int cnt = 0;
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane((int)tau_l, m);
    ball[m] = __ballot(key[m] != 0u && key[m] >= tau);
    cnt = lane == m ? (int)__builtin_popcountll(ball[m]) : cnt;
  }
  const int base = lane < MM ? atomicAdd(&sm->ccount[lane], cnt) : 0;
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    const int pos = __builtin_amdgcn_readlane(base, m) +
                    (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ball[m] >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ball[m], 0u));
    if (((ball[m] >> lane) & 1ull) && pos < 64)
      sm->cand[m * 64 + pos] = ((uint64_t)key[m] << 32) | (uint64_t)(uint32_t)~tid;
  }
  __syncthreads();
}

template <class P>
__device__ __forceinline__ void topk_rows(const P& p, const float* lgs, Small* sm, int tid,
                                          int wv, int lane) {
  const int M = p.M, E = p.E, K = p.K;
  const int nW = (E + 63) >> 6;
  const bool fast = E <= MOE_WG && K <= nW;
  if (fast) {
    switch (M) {
      case 1: topk_fast<1>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 2: topk_fast<2>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 3: topk_fast<3>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 4: topk_fast<4>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 5: topk_fast<5>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 6: topk_fast<6>(lgs, sm, E, K, nW, tid, wv, lane); break;
      case 7: topk_fast<7>(lgs, sm, E, K, nW, tid, wv, lane); break;
      default: topk_fast<8>(lgs, sm, E, K, nW, tid, wv, lane); break;
    }
  }
  // (c) one wave per row: rank the candidates, or K plain rounds
  for (int m = wv; m < M; m += MOE_WAVES) {
    const int n = fast ? sm->ccount[m] : 0;
    if (n >= K && n <= 64) {
      const uint64_t* cr = sm->cand + m * 64;
      const uint64_t mine = lane < n ? cr[lane] : 0ull;
      int rank = 0;
#pragma unroll 1
      for (int j = 0; j < n; j += 8) {
        const ulonglong2 c0 = *reinterpret_cast<const ulonglong2*>(cr + j);
        const ulonglong2 c1 = *reinterpret_cast<const ulonglong2*>(cr + j + 2);
        const ulonglong2 c2 = *reinterpret_cast<const ulonglong2*>(cr + j + 4);
        const ulonglong2 c3 = *reinterpret_cast<const ulonglong2*>(cr + j + 6);
        const uint64_t c8[8] = {c0.x, c0.y, c1.x, c1.y, c2.x, c2.y, c3.x, c3.y};
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += (j + q < n && c8[q] > mine) ? 1 : 0;
      }
      if (lane < n && rank < K) sm->tk_idx[m * K + rank] = (int)~(uint32_t)mine;
      // gates in rank order (the candidates' lane order depends on timing)
      gates_from_idx(lgs + m * E, K, sm, m, lane);
    } else {
      select_row_plain(lgs + m * E, E, K, sm->tk_idx + m * K, lane);
      gates_from_idx(lgs + m * E, K, sm, m, lane);
    }
  }
}

// Routed slots in ascending expert order and their row masks, then the shared
// expert as slot U (every row), and the gate of every (slot, row).  Built by
// wave 0 alone (its LDS operations execute in order), then one workgroup
// barrier publishes the tables.
template <class P>
__device__ __forceinline__ void build_union(const P& p, Small* sm, int wv, int lane) {
  if (wv == 0) {
    const int M = p.M, K = p.K;
    const int MK = M * K;  // <= 128: entries (row, rank) i = lane and lane + 64
    if (lane < 32) sm->bm[lane] = 0u;
    sm->umask[lane] = 0u;
    sm->umask[lane + 64] = 0u;
    if (lane == 0) sm->umask[kMaxPK] = 0u;
    const int ea = lane < MK ? sm->tk_idx[lane] : -1;
    const int eb = lane + 64 < MK ? sm->tk_idx[lane + 64] : -1;
    if (ea >= 0) atomicOr(&sm->bm[ea >> 5], 1u << (ea & 31));
    if (eb >= 0) atomicOr(&sm->bm[eb >> 5], 1u << (eb & 31));
    const uint32_t w = lane < 32 ? sm->bm[lane] : 0u;
    const int c = __builtin_popcount(w);
    const int incl = wave_incl_scan(c);
    const int U = __builtin_amdgcn_readlane(incl, 63);
    if (lane < 32) sm->bpre[lane] = incl - c;
    if (lane == 0) sm->nU = U;
    // routed slot of each entry = number of selected experts below it
    int ra = -1, rb = -1;
    // gate of (slot, row): a row that lists one expert more than once (possible
    // only for caller-provided routing) weights it by the sum of those gates,
    // added in rank order by the entry that lists it first
    auto row_gate = [&](int i, int e) __attribute__((always_inline)) -> float {
      const int m0 = (i / K) * K;
      for (int k = m0; k < i; ++k)
        if (sm->tk_idx[k] == e) return -1.0f;  // not the first listing
      float gsum = 0.0f;
      for (int k = i; k < m0 + K; ++k)
        if (sm->tk_idx[k] == e) gsum += sm->tk_gate[k];
      return gsum;
    };
    if (ea >= 0) {
      ra = sm->bpre[ea >> 5] + __builtin_popcount(sm->bm[ea >> 5] & ((1u << (ea & 31)) - 1u));
      sm->uexp[ra] = ea;
      atomicOr(&sm->umask[ra], 1u << (lane / K));
      const float gs = row_gate(lane, ea);
      if (gs >= 0.0f) sm->slot_gate[ra * MOE_MAXM + lane / K] = gs;
    }
    if (eb >= 0) {
      rb = sm->bpre[eb >> 5] + __builtin_popcount(sm->bm[eb >> 5] & ((1u << (eb & 31)) - 1u));
      sm->uexp[rb] = eb;
      atomicOr(&sm->umask[rb], 1u << ((lane + 64) / K));
      const float gs = row_gate(lane + 64, eb);
      if (gs >= 0.0f) sm->slot_gate[rb * MOE_MAXM + (lane + 64) / K] = gs;
    }
    if (lane < MK) sm->upos[lane] = ra;
    if (lane + 64 < MK) sm->upos[lane + 64] = rb;
    if (p.S) {
      if (lane == 0) {
        sm->uexp[U] = p.E;
        sm->umask[U] = (1u << M) - 1u;
      }
      if (lane < M) sm->slot_gate[U * MOE_MAXM + lane] = 1.0f;
    }
  }
  __syncthreads();
}

// Piece q (0 or 1) of a workgroup's gate/up units [us0, us1): slot r and its
// units [a, b).  A range of at most I/2 units spans at most two slots.
__device__ __forceinline__ bool piece_of(int us0, int us1, int I2, int q, int& r, int& a,
                                         int& b) {
  if (us0 >= us1) return false;
  const int r0 = us0 / I2, e0 = (r0 + 1) * I2;
  if (q == 0) {
    r = r0;
    a = us0;
    b = us1 < e0 ? us1 : e0;
    return true;
  }
  if (us1 <= e0) return false;
  r = r0 + 1;
  a = e0;
  b = us1;
  return true;
}

// The contribution list of the combine: for each token row m, in order of
// workgroup g, piece q and row index t within the piece's slot, one entry
// (g << 4 | q << 3 | t) for every piece whose slot row m selected.  Workgroup
// g's units are the same equal share [g*NU/G, (g+1)*NU/G) the producer took.
// Thread g describes workgroup g; per-wave ballots and one barrier place the
// entries.
__device__ __forceinline__ void build_contributions(Small* sm, int G, int NU, int I2, int M,
                                                    int tid, int wv, int lane) {
  const int gg = tid;
  int r0 = 0, r1 = 0;
  uint32_t m0 = 0u, m1 = 0u;  // rows of piece 0 / piece 1 of workgroup gg
  if (gg < G) {
    const int us0 = (int)(((long long)gg * NU) / G), us1 = (int)(((long long)(gg + 1) * NU) / G);
    int a, b;
    if (piece_of(us0, us1, I2, 0, r0, a, b)) m0 = sm->umask[r0];
    if (piece_of(us0, us1, I2, 1, r1, a, b)) m1 = sm->umask[r1];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  int pre[MOE_MAXM];
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) {
    const uint64_t b0 = __ballot((m0 >> m) & 1u);
    const uint64_t b1 = __ballot((m1 >> m) & 1u);
    pre[m] = __builtin_popcountll(b0 & lt) + __builtin_popcountll(b1 & lt);
    if (lane == 0 && m < M)
      sm->wtot[wv * MOE_MAXM + m] = __builtin_popcountll(b0) + __builtin_popcountll(b1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int m = 0; m < M; ++m) {
      sm->cstart[m] = acc;
      for (int w = 0; w < MOE_WAVES; ++w) acc += sm->wtot[w * MOE_MAXM + m];
    }
    sm->cstart[M] = acc;
    sm->ncontrib = acc;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) {
    if (m < M && (((m0 | m1) >> m) & 1u)) {
      int pos = sm->cstart[m] + pre[m];
      for (int w = 0; w < wv; ++w) pos += sm->wtot[w * MOE_MAXM + m];
      if ((m0 >> m) & 1u)
        sm->clist[pos++] = (uint16_t)((gg << 4) | (0 << 3) |
                                      __builtin_popcount(m0 & ((1u << m) - 1u)));
      if ((m1 >> m) & 1u)
        sm->clist[pos] = (uint16_t)((gg << 4) | (1 << 3) |
                                    __builtin_popcount(m1 & ((1u << m) - 1u)));
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- the kernel

template <int CPLH, int NL>
__global__ __launch_bounds__(MOE_WG, 1) void moe_layer_kernel(ParamsT<NL> p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + p.lds_xs);
  const uint4* xs4 = reinterpret_cast<const uint4*>(xs);
  float* lgs = reinterpret_cast<float*>(lds + p.lds_lg);
  uint32_t* hw = reinterpret_cast<uint32_t*>(lds + p.lds_hw);  // [M][uw_max] SwiGLU pairs
  float* zs = reinterpret_cast<float*>(lds + p.lds_z);         // [zcap][nr_max] contributions
  Small* sm = reinterpret_cast<Small*>(lds + p.lds_small);

  const int G = gridDim.x, g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int NW = G * MOE_WAVES;
  const int gw = wv * G + g;  // consecutive wave ids land on different CUs
  const uint32_t tag = ld_u32(p.hdr + HDR_EPOCH) + 1u;
  const uint32_t dbg = ld_u32(p.hdr + HDR_FLAGS);
  const uint32_t budget = ld_u32(p.hdr + HDR_DEADLINE);
  Waiter wt{p.hdr, now_ticks() + (budget ? budget : kDefaultDeadlineTicks)};
  const int M = p.M, H = p.H, I = p.I, K = p.K, S = p.S, E = p.E;
  const int I2 = I >> 1, H2 = H >> 1, I8 = I >> 3;
  const int MK = M * K;
  const bool router_only = (p.flags & F_ROUTER_ONLY) != 0u;
  const bool topk_in = (p.flags & F_TOPK_IN) != 0u;

  if (tid == 0) sm->abort_flag = 0;
  uint64_t* stamps = ((dbg & DBG_STAMPS) && g < STAMP_WG)
                         ? reinterpret_cast<uint64_t*>(p.hdr + HDR_STAMPS) + (size_t)g * STAMP_SLOTS
                         : nullptr;
  int sbase = 0;
#define MOE_STAMP(ev)                                                          \
  do {                                                                         \
    if (stamps && tid == 0 && sbase >= 0) stamps[sbase + (ev)] = now_ticks(); \
  } while (0)

  // output rows owned by this workgroup (whole row pairs)
  const int r0 = (int)(((long long)g * H2) / G), r1 = (int)(((long long)(g + 1) * H2) / G);
  const int n0 = 2 * r0, NR = 2 * (r1 - r0);

  for (int l = 0; l < p.L; ++l) {
    sbase = l == 0 ? 0 : (l == 1 ? 10 : (l == p.L - 1 ? 20 : -1));
    MOE_STAMP(0);
    // ---------------- P1 prefetch: this wave's first router rows do not
    // depend on x, so their loads fly while x is staged
    const int NRI = topk_in ? 0 : (E + 1) >> 1;
    RowRegs<CPLH> A, B;
    if (gw < NRI) p1_load<CPLH>(p, l, gw, A, lane);

    // ---------------- P0: layer input -> LDS
    if (l == 0) {
      const uint4* src = reinterpret_cast<const uint4*>(p.x_in);
      uint4* dst = reinterpret_cast<uint4*>(xs);
      for (int i = tid; i < (M * H) >> 3; i += MOE_WG) dst[i] = src[i];
    } else {
      const uint64_t* src = p.res_buf + (size_t)l * M * H2;
      if (!stage_tagged<8>(M * H2, reinterpret_cast<uint32_t*>(xs), tag, wt, tid,
                           [&](int i) { return src + i; }))
        sm->abort_flag = 1;
    }
    __syncthreads();
    if (l == 0 && tid == 0 && (p.flags & F_ALIAS)) add_u32(p.hdr + HDR_XREAD, 1u);
    if (sm->abort_flag) break;
    if (p.flags & F_RESIDUAL) {
      for (int i = tid; i < M * NR; i += MOE_WG) {
        const int m = i / NR, nl = i - m * NR;
        sm->hres[m * p.nr_max + nl] = xs[m * H + n0 + nl];
      }
    }
    if (l == 0 && g == 0 && p.h_all) {
      uint4* dst = reinterpret_cast<uint4*>(p.h_all);
      for (int i = tid; i < (M * H) >> 3; i += MOE_WG) dst[i] = xs4[i];
    }
    if (p.flags & F_PRENORM) {
      // Sum of squares per row in double: every bf16 square is exact in fp32 and,
      // over the value range of a residual stream, every partial sum is exact in
      // double, so the sum (and the scale) does not depend on the order.
      const uint32_t* xr32 = reinterpret_cast<const uint32_t*>(xs);
      for (int m = wv; m < M; m += MOE_WAVES) {
        double ss = 0.0;
        for (int c = lane; c < H2; c += 64) {
          const uint32_t w = xr32[m * H2 + c];
          const float a = bf_lo(w), b = bf_hi(w);
          ss += (double)(a * a);
          ss += (double)(b * b);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        if (lane == 0) sm->rn[m] = (float)(1.0 / sqrt(ss / (double)H + (double)kRmsEps));
      }
      __syncthreads();
      uint32_t* x32 = reinterpret_cast<uint32_t*>(xs);
      for (int i = tid; i < M * H2; i += MOE_WG) {
        const float r = sm->rn[i / H2];
        const uint32_t w = x32[i];
        x32[i] = f_to_bf(bf_lo(w) * r) | (f_to_bf(bf_hi(w) * r) << 16);
      }
    }
    __syncthreads();
    MOE_STAMP(1);

    // ---------------- P1: router rows
    for (int it = gw; it < NRI; it += NW) {
      if (it != gw) p1_load<CPLH>(p, l, it, A, lane);
      p1_compute<CPLH>(p, l, it, A, xs4, tag, lane, dbg);
    }
    MOE_STAMP(2);

    if (router_only) {
      // the last workgroup to finish its rows computes the top-k
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = add_u32(p.hdr + HDR_DONE, 1u);
        sm->abort_flag = (old == (uint32_t)(G - 1)) ? 2 : 3;
      }
      __syncthreads();
      if (sm->abort_flag != 2) return;
    }

    // ---------------- P4: routing
    if (topk_in) {
      for (int i = tid; i < MK; i += MOE_WG) {
        int e = p.tk_idx_in[i];
        if (e < 0 || e >= E) {
          record_status(p.hdr, -7 /* MOE_E_INDEX */);
          e = -1;
        }
        sm->tk_idx[i] = e;
        sm->tk_gate[i] = p.tk_gate_in[i];
      }
      __syncthreads();
    } else {
      const uint64_t* src = p.lg_buf + (size_t)l * M * E;
      if (!stage_tagged<8>(M * E, reinterpret_cast<uint32_t*>(lgs), tag, wt, tid,
                           [&](int i) { return src + i; }))
        sm->abort_flag = 1;
      __syncthreads();
      MOE_STAMP(3);
      if (sm->abort_flag == 1) break;
      topk_rows(p, lgs, sm, tid, wv, lane);
      __syncthreads();
      MOE_STAMP(9);
      if (g == 0 || router_only) {
        int32_t* oi = p.tk_idx_out ? p.tk_idx_out + (size_t)l * MK : nullptr;
        for (int i = tid; i < MK; i += MOE_WG) {
          if (oi) oi[i] = sm->tk_idx[i];
          if (p.tk_gate_out && l == 0) p.tk_gate_out[i] = sm->tk_gate[i];
        }
        if (p.logits_out && l == 0)
          for (int i = tid; i < M * E; i += MOE_WG) p.logits_out[i] = lgs[i];
      }
      if (router_only) break;
    }

    // ---------------- P5: routed slots (+ the shared expert as slot U)
    build_union(p, sm, wv, lane);
    const int U = sm->nU;
    const int US = U + S;
    MOE_STAMP(4);

    // ---------------- P6: this workgroup's gate/up units
    // Units u = (slot r, intermediate pair jp), slot-major (u = r * I/2 + jp);
    // the workgroup takes the contiguous range [us0, us1), an equal share of
    // all units, which spans at most two slots ("pieces").  A wave's unit is
    // gate/up rows 2jp and 2jp + 1 of slot r, all requested before any is
    // used; the SwiGLU pair of every selecting row stays in LDS.
    const int NU = US * I2;
    const int us0 = (int)(((long long)g * NU) / G), us1 = (int)(((long long)(g + 1) * NU) / G);
    const int UW = us1 - us0;
    {
      const int H8 = H >> 3;
      for (int u = us0 + wv; u < us1; u += MOE_WAVES) {
        const int rr = u / I2, jp = u - rr * I2;
        const uint16_t* base = p.lw[l].wgu + (size_t)sm->uexp[rr] * (2 * (size_t)I) * H;
        const size_t j0 = 2 * (size_t)jp;
        load_rows<CPLH>(A, base + j0 * H, base + ((size_t)I + j0) * H, lane);
        load_rows<CPLH>(B, base + (j0 + 1) * H, base + ((size_t)I + j0 + 1) * H, lane);
        uint32_t bits = sm->umask[rr];
        int t = 0;
#pragma unroll 1
        while (bits) {
          const int m = __builtin_ctz(bits);
          bits &= bits - 1u;
          const float a0 = dot_rows<CPLH>(A, xs4, H8, m, lane);
          const float a1 = dot_rows<CPLH>(B, xs4, H8, m, lane);
          const uint32_t word = f_to_bf(swiglu(readlane_f(a0, 0), readlane_f(a0, 32))) |
                                (f_to_bf(swiglu(readlane_f(a1, 0), readlane_f(a1, 32))) << 16);
          if (lane == 0) hw[t * p.uw_max + (u - us0)] = word;
          ++t;
        }
      }
    }
    __syncthreads();
    MOE_STAMP(5);

    // ---------------- P7: down projection, split over the intermediate dim
    // For each piece (slot r, units [a, b)) this workgroup computes the partial
    // down projection over its own 2(b - a) intermediate indices for ALL H
    // outputs, y_t[n] = sum_j h_t[j] * Wd[e][n][j] (Wd stored transposed, so
    // row j is contiguous), scales it by the gate of the row, and publishes it
    // as tagged fp32 words.  No SwiGLU value crosses workgroups.  Thread c
    // owns output columns 8c .. 8c+7 and streams DB intermediate rows at a time.
    uint64_t* part_l = p.part_buf + (size_t)l * kMaxWG * 2 * M * H;
    {
      const int H8 = H >> 3;
      const int c = tid;
      for (int q = 0; q < 2; ++q) {
        int r, a, b;
        if (!piece_of(us0, us1, I2, q, r, a, b)) break;
        const int e = sm->uexp[r];
        const uint32_t mask = sm->umask[r];
        const int nt = __builtin_popcount(mask);
        float acc[MOE_MAXM][8];
#pragma unroll
        for (int t = 0; t < MOE_MAXM; ++t)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[t][k] = 0.0f;
        const uint16_t* wd = p.lw[l].wd + (size_t)e * I * H;
        constexpr int DB = 4;  // intermediate pairs per batch (2 rows each)
        for (int u = a; u < b; u += DB) {
          uint4 w[2 * DB];
#pragma unroll
          for (int k = 0; k < DB; ++k) {
            const int uu = (u + k < b) ? u + k : u;
            const size_t j = 2 * (size_t)(uu - r * I2);
            const uint4* r0p = reinterpret_cast<const uint4*>(wd + j * H);
            const uint4* r1p = reinterpret_cast<const uint4*>(wd + (j + 1) * H);
            w[2 * k] = c < H8 ? r0p[c] : make_uint4(0, 0, 0, 0);
            w[2 * k + 1] = c < H8 ? r1p[c] : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int k = 0; k < DB; ++k) {
            if (u + k < b) {
#pragma unroll
              for (int t = 0; t < MOE_MAXM; ++t) {
                if (t < nt) {
                  const uint32_t hword = hw[t * p.uw_max + (u + k - us0)];
                  const float h0 = bf_lo(hword), h1 = bf_hi(hword);
                  fma8(acc[t], w[2 * k], h0);
                  fma8(acc[t], w[2 * k + 1], h1);
                }
              }
            }
          }
        }
        // publish gate * partial for each selecting row
        if (c < H8) {
          uint32_t bits = mask;
#pragma unroll
          for (int t = 0; t < MOE_MAXM; ++t) {
            if (t < nt) {
              const int m = __builtin_ctz(bits);
              bits &= bits - 1u;
              const float gt = sm->slot_gate[r * MOE_MAXM + m];
              uint64_t* dst = part_l + (((size_t)g * 2 + q) * M + t) * H + 8 * c;
#pragma unroll
              for (int k = 0; k < 8; ++k) st_tag(dst + k, __float_as_uint(gt * acc[t][k]), tag);
            }
          }
        }
      }
    }
    MOE_STAMP(6);

    // ---------------- P8: combine (+ residual) and hand off
    // This workgroup owns output rows [n0, n0 + NR).  Its contributions are
    // every workgroup's published partials for the rows of the token rows they
    // cover, listed by token row, then workgroup, piece and row (a fixed order,
    // so the sum is deterministic); they are staged in LDS in chunks and summed.
    const bool last = (l == p.L - 1);
    if (last && (p.flags & F_ALIAS)) {
      if (tid == 0) {
        for (;;) {
          if (ld_u32(p.hdr + HDR_XREAD) >= (uint32_t)G) break;
          if (wt.expired()) { record_status(p.hdr, -6); sm->abort_flag = 1; break; }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
      if (sm->abort_flag == 1) break;
    }
    build_contributions(sm, G, NU, I2, M, tid, wv, lane);
    MOE_STAMP(7);
    {
      const int NC = sm->ncontrib;
      for (int i = tid; i < M * NR; i += MOE_WG) sm->osum[i] = 0.0f;
      __syncthreads();
      for (int c0 = 0; c0 < NC; c0 += p.zcap) {
        const int nc = (NC - c0 < p.zcap) ? NC - c0 : p.zcap;
        if (NR > 0 && !stage_tagged<8>(nc * NR, reinterpret_cast<uint32_t*>(zs), tag, wt, tid,
                                       [&](int i) {
                                         const int ci = i / NR;
                                         const uint32_t cd = sm->clist[c0 + ci];
                                         const int cg = (int)(cd >> 4), cq = (int)((cd >> 3) & 1u),
                                                   ct = (int)(cd & 7u);
                                         return part_l + (((size_t)cg * 2 + cq) * M + ct) * H + n0 +
                                                (i - ci * NR);
                                       }))
          sm->abort_flag = 1;
        __syncthreads();
        if (sm->abort_flag == 1) break;
        // output o = (m, nl): its contributions in this chunk are list entries
        // [cstart[m], cstart[m+1]) clipped to [c0, c0 + nc); one wave per
        // output, lanes strided over the entries, a fixed DPP tree at the end
        for (int o = wv; o < M * NR; o += MOE_WAVES) {
          const int m = o / NR, nl = o - m * NR;
          const int ka = max(sm->cstart[m], c0), kb = min(sm->cstart[m + 1], c0 + nc);
          float v = 0.0f;
          for (int k = ka + lane; k < kb; k += 64) v += zs[(k - c0) * NR + nl];
          v = group_sum(v, 64);
          if (lane == 0) sm->osum[o] += v;
        }
        __syncthreads();
      }
      if (sm->abort_flag == 1) break;
      for (int i = tid; i < (NR >> 1) * M; i += MOE_WG) {
        const int np = i / M, m = i - np * M;
        const int nl = 2 * np, n = n0 + nl;
        const float a0 = sm->osum[m * NR + nl];
        const float a1 = sm->osum[m * NR + nl + 1];
        if (p.flags & F_RESIDUAL) {
          const float h0 = bf_to_f(sm->hres[m * p.nr_max + nl]);
          const float h1 = bf_to_f(sm->hres[m * p.nr_max + nl + 1]);
          const uint32_t word = f_to_bf(h0 + a0) | (f_to_bf(h1 + a1) << 16);
          if (last)
            reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = word;
          else
            st_tag(p.res_buf + (size_t)(l + 1) * M * H2 + ((m * H + n) >> 1), word, tag);
          if (p.h_all)
            reinterpret_cast<uint32_t*>(p.h_all)[((size_t)(l + 1) * M * H + (size_t)m * H + n) >> 1] =
                word;
        } else if (p.flags & F_OUT_F32) {
          reinterpret_cast<float2*>(p.out)[(m * H + n) >> 1] = make_float2(a0, a1);
        } else {
          reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = f_to_bf(a0) | (f_to_bf(a1) << 16);
        }
      }
    }
    __syncthreads();
    MOE_STAMP(8);
    if (sm->abort_flag == 1) break;
  }

  // ---------------- end of call: the last workgroup advances the step
  __syncthreads();
  sbase = 0;
  MOE_STAMP(31);
#undef MOE_STAMP
  if (tid == 0) {
    const bool counted = router_only;  // router-only already counted itself
    uint32_t old = 0;
    if (!counted) old = add_u32(p.hdr + HDR_DONE, 1u);
    if (counted || old == (uint32_t)(G - 1)) {
      st_u32(p.hdr + HDR_DONE, 0u);
      st_u32(p.hdr + HDR_XREAD, 0u);
      st_u32(p.hdr + HDR_EPOCH, tag);
    }
  }
}

}  // namespace moe
