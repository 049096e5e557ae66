// The fused MoE layer / chain kernel for gfx950.
//
// One persistent launch runs one or several MoE layers; one workgroup per CU,
// all resident for the whole call.  Per layer:
//
//   P0  stage the layer input x [M][H] in LDS (layer 0 from the caller's
//       buffer, later layers from step-tagged residual words); under the
//       pre-norm chain keep this workgroup's rows of h_l for the residual and
//       replace x by bf16(RMSNorm(h_l) * gain).
//   P1  router GEMV rows and the shared expert's gate/up rows, spread over every
//       wave of the GPU.  Neither depends on the routing, so their loads are
//       issued before the input is even staged, and the shared expert's rows
//       stream while the logits travel between workgroups (the AMD kernels of
//       "SGLang Low-Latency Mode: Kernels and Runtime", section "AMD Low-Latency
//       Kernels", request routing-independent weights ahead of their inputs in
//       the same way).  Logits and the shared expert's SwiGLU output are
//       published as step-tagged words.
//   P4  every workgroup reads all logits and computes the softmax top-k
//       itself, so no second device-wide hop is needed.
//   P5  routed slots: the union of the rows' choices, from a bitmap over experts
//       plus population counts, with no scan over experts or sort (SGLang
//       Low-Latency Mode, item 3).  One token row needs no union: slot r is
//       rank r, and every wave keeps its own slot table.
//   P6  routed gate/up + SwiGLU: the tasks (one intermediate row pair of one
//       slot) of the whole union are dealt round-robin over every wave of the
//       GPU, so each workgroup streams from every selected expert; SwiGLU
//       outputs are published as tagged bf16 pairs.
//   P7  down projection: the (slot, output row) space is cut into one equal
//       slice per workgroup (pieces of at most two slots); each workgroup stages
//       the SwiGLU rows of its pieces and of the shared expert in LDS with one
//       batched wait, then streams the shared expert's down rows for its own
//       output rows and its pieces' routed down rows, published as tagged fp32.
//   P8  each workgroup owns a slice of output rows and combines
//       y_shared + s * sum_k g_k y_k in fp32 in rank order, then rounds once (or
//       adds the residual with one rounding, or writes the fp32 partial).
//
// Every selected expert's weights stream from HBM exactly once per call, for
// all the token rows that chose it, with the non-temporal policy (read once,
// they pass through L2 without evicting the kernel's code).
#pragma once

#include <type_traits>

#include "moe_device.hpp"

namespace moe {

// Pause between polling rounds of a tagged stage (units of 64 clocks).
#ifndef MOE_POLL_SLEEP
#define MOE_POLL_SLEEP 1
#endif

#ifndef MOE_MAX_LAYERS
#define MOE_MAX_LAYERS 64
#endif

constexpr int kMaxPK = MOE_MAXM * 16;  // max (routed expert, row) pairs = M * K
// Words that every workgroup reads (the logits, the shared expert's SwiGLU
// row, the next layer's input) are published in kCopies copies; workgroup g
// reads copy g % kCopies, the one of its own XCD.  When all workgroups poll
// one copy, their reads of the same lines queue at the memory side and a
// wave sees the last word about 0.4 us later than with one copy per XCD.
constexpr int kCopies = 8;

// Lane 0's value of v, whatever lanes are active, held in a scalar register
// from here on (a ticket taken by lane 0 and used by the whole wave: the
// compiler may not recompute it from the lane's register under another
// exec mask).
__device__ __forceinline__ int lane0_scalar(int v) {
  int s = __builtin_amdgcn_readlane(v, 0);
  asm volatile("" : "+s"(s));
  return s;
}
constexpr int kOwnSlots = kMaxPK + 1;  // first per-wave slot table entry (one token row)

struct LayerW {
  const uint16_t* wr;    // [E][H]
  const void* wgu;       // [E+S][2I][H] bf16, or fp8 e4m3 codes
  const void* wd;        // [E+S][H][I]  bf16, or fp8 e4m3 codes
  const float* bias;     // [E] selection bias, or null
  const uint16_t* gain;  // [H] RMSNorm gain (bf16), or null for unit gain
  const float* sgu;      // fp8: [E+S][2I/128][H/128] block scales of wgu
  const float* sd;       // fp8: [E+S][H/128][I/128] block scales of wd
};

enum : uint32_t {
  F_RESIDUAL = 1u,     // chain: h_{l+1} = bf16(h_l + acc)
  F_OUT_F32 = 2u,      // write the unrounded fp32 acc
  F_TOPK_IN = 4u,      // routing comes from the caller (experts only)
  F_ROUTER_ONLY = 8u,  // router + top-k only
  F_ALIAS = 16u,       // out overlaps x_in: wait until every workgroup has read x_in
  F_PRENORM = 32u,     // each layer's MoE input is bf16(RMSNorm(h_l) * gain_l)
};

constexpr float kRmsEps = 1e-6f;

// NL: layer weight slots carried in the kernel arguments (1 for single-layer
// calls keeps the argument block small; the chain takes MOE_MAX_LAYERS).
template <int NL>
struct ParamsT {
  int H, E, K, I, S, M, L;
  uint32_t flags;
  int nr_max;         // output rows owned by one workgroup, at most
  float scale;        // routed scaling factor of the combine
  uint32_t tag;       // this call's step tag (never 0; the host counts the calls on a workspace)
  uint32_t dbg;       // debug flags (DBG_*)
  uint32_t budget;    // wait deadline, 100 MHz ticks
  // LDS byte offsets
  int lds_xs, lds_lg, lds_hs, lds_ysh, lds_ysr, lds_small;  // lds_hs: [3*M][I] bf16
  int lds_gn;         // [H] bf16 norm gain
  int fold;           // down slices folded: half from the first slots, half from the last (see P6)
  int lds_p1w;        // the router / shared rows of waves 0-2 (see P1, P4), or -1
  const uint16_t* x_in;
  void* out;
  const int32_t* tk_idx_in;
  const float* tk_gate_in;
  int32_t* tk_idx_out;   // [L][M][K] (or [M][K])
  float* tk_gate_out;    // [M][K]
  float* logits_out;     // [M][E]
  uint16_t* h_all;       // [L+1][M][H] residual stream per layer (optional)
  uint32_t* hdr;
  uint64_t* lg_buf;      // [L][kCopies][M][E]   tagged fp32 logits
  uint64_t* hs_buf;      // [L][kCopies][M][I/2] tagged bf16 pairs, shared expert
  uint64_t* hr_buf;      // [L][M*K][I/2]   tagged bf16 pairs, routed (expert, row) pairs
  uint64_t* y_buf;       // [L][M*K][H]     tagged fp32 down outputs of routed pairs
  uint64_t* res_buf;     // [L+1][kCopies][M][H/2] tagged bf16 pairs, residual stream
  LayerW lw[NL];
};

// eight bf16 ones (the RMSNorm gain of a layer without one)
__device__ const uint4 kBf16OnesChunk = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
typedef __attribute__((address_space(3))) void* LdsPtr;
// cache-policy operand of a direct-to-LDS load: non-temporal, as the weight
// loads into registers
constexpr int kNtAux = MOE_WEIGHT_NT ? 2 : 0;

struct Small {
  int nU, nP, abort_flag, sel_ok;  // sel_ok: one token row selected on the fast path
  int gu_next, dn_next;      // the workgroup's task tickets (gate/up, down)
  int st_next, pad2;         // staging chunks of the down inputs: next to claim
  uint64_t st_done;          // and the chunks staged (bit c)
  int tk_idx[kMaxPK];
  float tk_gate[kMaxPK];
  int upos[kMaxPK];          // routed slot of (row, rank), -1 if skipped
  // Slot tables: entries [0, kMaxPK] are the workgroup's; with one token row,
  // each wave also keeps its own copy of its slots at kOwnSlots + 8 * wave
  int uexp[kOwnSlots + MOE_WAVES * 8];        // expert id of routed slot r
  uint32_t umask[kOwnSlots + MOE_WAVES * 8];  // rows that chose routed slot r
  int pbase[kOwnSlots + MOE_WAVES * 8];       // first (slot, row) pair of slot r
  uint32_t bm[32];           // expert bitmap (E <= 1024)
  int bpre[32];              // population-count prefix per bitmap word
  float rn[MOE_MAXM];        // RMSNorm scale per token row
  alignas(16) uint64_t cand[MOE_WAVES * 128];  // top-k: each wave's candidates + spare slots
  uint16_t hres[MOE_MAXM * 64];  // residual input h_l of this workgroup's output rows
  // this workgroup's down tasks (P7): per piece k < 4 its slot, rows [n0, n1),
  // blocks, token rows and first (slot, row) pair; per segment (shared |
  // pieces) its first staged word and first staging chunk (entry 5: the ends)
  int dk_r[4], dk_n0[4], dk_n1[4], dk_nb[4], dk_nrow[4], dk_pb[4];
  int dk_ws[6], dk_nc[6];
  int dk_ntask;
  int dn_done;  // waves that have left the down loop, in order
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
// NT threads take part (tid < NT: the workgroup, or one wave with tid = lane).
template <int B, int NT = MOE_WG, typename Addr>
__device__ __forceinline__ bool stage_tagged(int n, uint32_t* dst32, uint32_t tag,
                                             const Waiter& wt, int tid, Addr addr) {
  const uint64_t ready = (uint64_t)tag << 32;
  for (int base = tid; base < n; base += B * NT) {
    uint64_t v[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = base + b * NT;
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
      __builtin_amdgcn_s_sleep(MOE_POLL_SLEEP);
#pragma unroll
      for (int b = 0; b < B; ++b)
        if ((uint32_t)(v[b] >> 32) != tag) v[b] = ld_tag(addr(base + b * NT));
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = base + b * NT;
      if (i < n) dst32[i] = (uint32_t)v[b];
    }
  }
  return true;
}

// ---------------------------------------------------------------- streaming units
//
// A row unit is two weight rows of H bf16 values, the first on lanes 0-31 and
// the second on lanes 32-63, CPLH 16-byte loads per lane.  A down unit is
// DBLK blocks of 8 down-projection rows (8 lanes per row, CPLI loads per lane).
// Every task requests all its weights before using any, and the first task of
// a phase is requested before the phase waits on its inputs.

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
  for (int q = 0; q < CPLH; ++q) r.w[q] = ld_weight(src + li + 32 * q);
}

// Dot product of each half-wave's row with token row m (all lanes of a half
// receive the sum); wat(q) gives this lane's 16-byte chunk q of its row (from
// registers or from LDS).
template <int CPLH, typename WAt>
__device__ __forceinline__ float dot_rows_w(WAt wat, const uint4* xs4, int H8, int m, int lane) {
  const int li = lane & 31;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < CPLH; ++q) acc = dot8(wat(q), xs4[m * H8 + li + 32 * q], acc);
  return group_sum(acc, 32);
}

template <int CPLH>
__device__ __forceinline__ float dot_rows(const RowRegs<CPLH>& r, const uint4* xs4, int H8, int m,
                                          int lane) {
  return dot_rows_w<CPLH>([&](int q) { return r.w[q]; }, xs4, H8, m, lane);
}

// ---- fp8 e4m3 weights with 128 x 128 block scales
//
// A row of H codes takes H/16 16-byte chunks; lane li of a half-wave takes
// chunks li + 32q (q < C8 = ceil(CPLH / 2)), all of them when H is a multiple
// of 512.  Chunk c lies in column block c / 8, so its partial dot product is
// multiplied by that block's scale before it joins the lane's sum.  Codes
// become bf16 pairs in one conversion each (every e4m3 value is a bf16 value)
// and meet the bf16 activations in v_dot2.

// sum_{k<16} dec(w_k) * x_k for 16 codes and 16 bf16 activations (xa: 0-7, xb: 8-15)
__device__ __forceinline__ float dot16_fp8(const uint4 w, const uint4 xa, const uint4 xb) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  const uint32_t xx[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[i], 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[i], 1.0f, true);
    acc = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2_t, xx[2 * i]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2_t, xx[2 * i + 1]), acc,
                                          false);
  }
  return acc;
}

template <int CPLH>
struct Fp8Row {
  static constexpr int C = (CPLH + 1) / 2;            // chunks per lane
  static constexpr bool ragged = (CPLH & 1) != 0;     // H/16 < 32 C: some lanes idle
  __device__ static bool valid(int c, int H) { return !ragged || c < (H >> 4); }
};

template <int CPLH>
__device__ __forceinline__ void load_rows8(RowRegs<CPLH>& r, const uint8_t* row0,
                                           const uint8_t* row1, int H, int lane) {
  const uint4* src = reinterpret_cast<const uint4*>((lane >> 5) ? row1 : row0);
  const int li = lane & 31;
#pragma unroll
  for (int q = 0; q < Fp8Row<CPLH>::C; ++q) {
    const int c = li + 32 * q;
    r.w[q] = Fp8Row<CPLH>::valid(c, H) ? ld_weight(src + c) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Block scales of this lane's chunks; srow0 / srow1: the scale rows of the
// half-waves' weight rows.
template <int CPLH>
__device__ __forceinline__ void load_scales8(float (&sc)[Fp8Row<CPLH>::C], const float* srow0,
                                             const float* srow1, int H, int lane) {
  const float* srow = (lane >> 5) ? srow1 : srow0;
  const int li = lane & 31;
#pragma unroll
  for (int q = 0; q < Fp8Row<CPLH>::C; ++q) {
    const int c = li + 32 * q;
    sc[q] = Fp8Row<CPLH>::valid(c, H) ? srow[c >> 3] : 0.0f;
  }
}

template <int CPLH>
__device__ __forceinline__ float dot_rows8(const RowRegs<CPLH>& r,
                                           const float (&sc)[Fp8Row<CPLH>::C], const uint4* xs4,
                                           int H, int m, int lane) {
  const int li = lane & 31, H8 = H >> 3;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < Fp8Row<CPLH>::C; ++q) {
    const int c = Fp8Row<CPLH>::valid(li + 32 * q, H) ? li + 32 * q : 0;
    // convert at the point of use: hoisting the conversions out of the caller's
    // token-row loop would double the registers the codes occupy
    uint4 w = r.w[q];
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    const float part = dot16_fp8(w, xs4[m * H8 + 2 * c], xs4[m * H8 + 2 * c + 1]);
    acc = fmaf(sc[q], part, acc);
  }
  return group_sum(acc, 32);
}

// The same with the codes and scales in LDS ([chunk][lane]); same order of
// additions as dot_rows8.
template <int CPLH>
__device__ __forceinline__ float dot_rows8_lds(const uint4* sl, const float* ss, const uint4* xs4,
                                               int H, int m, int lane) {
  const int li = lane & 31, H8 = H >> 3;
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < Fp8Row<CPLH>::C; ++q) {
    const int c = Fp8Row<CPLH>::valid(li + 32 * q, H) ? li + 32 * q : 0;
    const float part = dot16_fp8(sl[q * 64 + lane], xs4[m * H8 + 2 * c], xs4[m * H8 + 2 * c + 1]);
    acc = fmaf(ss[q * 64 + lane], part, acc);
  }
  return group_sum(acc, 32);
}

// P1 item `it`: router rows (it < NRI) or a shared-expert gate/up row pair.
// The first unit goes to A; a gate/up item's second unit goes to B when
// `second` is set.
template <int CPLH, bool W8, class P>
__device__ __forceinline__ void p1_load(const P& p, int l, int it, int NRI,
                                        RowRegs<CPLH>& A, RowRegs<CPLH>& B,
                                        float (&SC)[Fp8Row<CPLH>::C], int lane, bool second) {
  if constexpr (W8) {
    if (it >= NRI) {  // shared expert: fp8 rows and their block scales
      const size_t H = (size_t)p.H, I = (size_t)p.I, HB = H >> 7;
      const size_t j0 = 2 * (size_t)(it - NRI);
      const uint8_t* base =
          static_cast<const uint8_t*>(p.lw[l].wgu) + (size_t)p.E * (2 * I) * H;
      const float* sb = p.lw[l].sgu + (size_t)p.E * ((2 * I) >> 7) * HB;
      load_rows8<CPLH>(A, base + j0 * H, base + (I + j0) * H, p.H, lane);
      if (second) load_rows8<CPLH>(B, base + (j0 + 1) * H, base + (I + j0 + 1) * H, p.H, lane);
      load_scales8<CPLH>(SC, sb + (j0 >> 7) * HB, sb + ((I + j0) >> 7) * HB, p.H, lane);
      return;
    }
  }
  // Row pointers are chosen first and the loads issued unconditionally after,
  // so the two register buffers never meet in one pointer (which would force
  // them out of registers).
  const size_t H = (size_t)p.H, I = (size_t)p.I;
  const uint16_t *a0, *a1, *b0, *b1;
  const bool router = it < NRI;
  if (router) {
    const int e0 = 2 * it, e1 = (2 * it + 1 < p.E) ? 2 * it + 1 : 2 * it;
    a0 = p.lw[l].wr + (size_t)e0 * H;
    a1 = p.lw[l].wr + (size_t)e1 * H;
    b0 = a0;
    b1 = a1;
  } else {
    const size_t j0 = 2 * (size_t)(it - NRI);
    const uint16_t* base = static_cast<const uint16_t*>(p.lw[l].wgu) + (size_t)p.E * (2 * I) * H;
    a0 = base + j0 * H;
    a1 = base + (I + j0) * H;
    b0 = base + (j0 + 1) * H;
    b1 = base + (I + j0 + 1) * H;
  }
  load_rows<CPLH>(A, a0, a1, lane);
  if (!router && second) load_rows<CPLH>(B, b0, b1, lane);
}

template <int CPLH, bool W8, class P>
__device__ __forceinline__ void p1_load_second(const P& p, int l, int it, int NRI,
                                               RowRegs<CPLH>& B, int lane) {
  const size_t H = (size_t)p.H, I = (size_t)p.I;
  const size_t j1 = 2 * (size_t)(it - NRI) + 1;
  if constexpr (W8) {
    const uint8_t* base = static_cast<const uint8_t*>(p.lw[l].wgu) + (size_t)p.E * (2 * I) * H;
    load_rows8<CPLH>(B, base + j1 * H, base + (I + j1) * H, p.H, lane);
  } else {
    const uint16_t* base = static_cast<const uint16_t*>(p.lw[l].wgu) + (size_t)p.E * (2 * I) * H;
    load_rows<CPLH>(B, base + j1 * H, base + (I + j1) * H, lane);
  }
}

// bf16 shared-expert item `it` copied from HBM straight into a wave's LDS slot
// (unit A [CPLH][64] = gate | up of unit 2j, then unit B = those of unit
// 2j + 1; 16-byte chunks in the register layout of load_rows), without
// passing through registers.  The copy has landed once the wave's vmcnt is
// zero; only the issuing wave reads the slot.
template <int CPLH, class P>
__device__ __forceinline__ void p1_shared_to_lds(const P& p, int l, int it, int NRI,
                                                 uint4* slot, int lane) {
  const size_t H = (size_t)p.H, I = (size_t)p.I;
  const size_t j0 = 2 * (size_t)(it - NRI);
  const uint16_t* base = static_cast<const uint16_t*>(p.lw[l].wgu) + (size_t)p.E * (2 * I) * H;
  const size_t r0 = (lane >> 5) ? I + j0 : j0;
  const uint4* sa = reinterpret_cast<const uint4*>(base + r0 * H) + (lane & 31);
  const uint4* sb = reinterpret_cast<const uint4*>(base + (r0 + 1) * H) + (lane & 31);
#pragma unroll
  for (int q = 0; q < CPLH; ++q)
    __builtin_amdgcn_global_load_lds(sa + 32 * q, (LdsPtr)(slot + q * 64), 16, 0, kNtAux);
#pragma unroll
  for (int q = 0; q < CPLH; ++q)
    __builtin_amdgcn_global_load_lds(sb + 32 * q, (LdsPtr)(slot + (CPLH + q) * 64), 16, 0, kNtAux);
}

// Router item it, token row m: the logit of expert 2 it + (lane >> 5), which
// every lane of the half-wave holds; lane c < kCopies of the half writes copy c.
template <class P>
__device__ __forceinline__ void publish_logit(const P& p, int l, int it, int m, float acc,
                                              uint32_t tag, int lane, uint32_t dbg) {
  const int e = 2 * it + (lane >> 5), c = lane & 31;
  if (e < p.E && c < kCopies && !(dbg & DBG_NO_ROUTER_PUBLISH))
    st_tag(p.lg_buf + (((size_t)l * kCopies + c) * p.M + m) * p.E + e, __float_as_uint(acc), tag);
}

// Shared-expert pair jp, token row m: a0 holds gate (lanes 0-31) and up (lanes
// 32-63) of unit 2jp, a1 those of unit 2jp + 1; lane c < kCopies writes copy c.
template <class P>
__device__ __forceinline__ void publish_shared(const P& p, int l, int jp, int m, float a0, float a1,
                                               uint32_t tag, int lane) {
  const int I2 = p.I >> 1;
  const uint32_t word = pk_bf(swiglu(readlane_f(a0, 0), readlane_f(a0, 32)),
                              swiglu(readlane_f(a1, 0), readlane_f(a1, 32)));
  if (lane < kCopies)
    st_tag(p.hs_buf + (size_t)l * kCopies * p.M * I2 + jp + ((size_t)lane * p.M + m) * I2, word, tag);
}

template <int CPLH, bool W8, class P>
__device__ __forceinline__ void p1_compute(const P& p, int l, int it, int NRI,
                                           const RowRegs<CPLH>& A, const RowRegs<CPLH>& B,
                                           const float (&SC)[Fp8Row<CPLH>::C], const uint4* xs4,
                                           uint32_t tag, int lane, uint32_t dbg) {
  const int H8 = p.H >> 3;
  if (it < NRI) {
#pragma unroll 1
    for (int m = 0; m < p.M; ++m)
      publish_logit(p, l, it, m, dot_rows<CPLH>(A, xs4, H8, m, lane), tag, lane, dbg);
  } else {
#pragma unroll 1
    for (int m = 0; m < p.M; ++m) {
      float a0, a1;
      if constexpr (W8) {
        a0 = dot_rows8<CPLH>(A, SC, xs4, p.H, m, lane);
        a1 = dot_rows8<CPLH>(B, SC, xs4, p.H, m, lane);
      } else {
        a0 = dot_rows<CPLH>(A, xs4, H8, m, lane);
        a1 = dot_rows<CPLH>(B, xs4, H8, m, lane);
      }
      publish_shared(p, l, it - NRI, m, a0, a1, tag, lane);
    }
  }
}

template <int CPLI, int DBLK>
struct DownRegs {
  uint4 w[DBLK][CPLI];
};

// Down rows [n, min(n + 8*DBLK, n_end)) of expert e: row n + 8b + (lane >> 3)
// on the 8-lane group of lane in block b.
template <int CPLI, int DBLK, class P>
__device__ __forceinline__ void load_down(DownRegs<CPLI, DBLK>& r, const P& p, int l, int e,
                                          int n, int n_end, int lane) {
  const int gl = lane >> 3, li = lane & 7;
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int row = n + 8 * b + gl;
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(p.lw[l].wd) + ((size_t)e * p.H + (row < n_end ? row : n)) * p.I);
#pragma unroll
    for (int q = 0; q < CPLI; ++q) r.w[b][q] = ld_weight(src + li + 8 * q);
  }
}

// y(t, row) = sum_j h_t[j] * W[row][j] for the nrows token rows whose SwiGLU
// outputs sit in LDS at hv4 (row t at hv4 + t * I8); emit(t, row, y).
template <int CPLI, int DBLK, typename Emit>
__device__ __forceinline__ void compute_down(const DownRegs<CPLI, DBLK>& r, int I8, int n,
                                             int n_end, int nrows, const uint4* hv4, int lane,
                                             Emit emit) {
  const int gl = lane >> 3, li = lane & 7;
#pragma unroll 1
  for (int t = 0; t < nrows; ++t) {
    // each 16-byte chunk of h is read once and serves every block
    float acc[DBLK];
#pragma unroll
    for (int b = 0; b < DBLK; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int q = 0; q < CPLI; ++q) {
      const uint4 x = hv4[t * I8 + li + 8 * q];
#pragma unroll
      for (int b = 0; b < DBLK; ++b) acc[b] = dot8(r.w[b][q], x, acc[b]);
    }
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const float y = group_sum(acc[b], 8);
      const int row = n + 8 * b + gl;
      if (li == 0 && row < n_end) emit(t, row, y);
    }
  }
}

// fp8 down rows: 8 lanes per row, lane li takes chunks li + 8q (q < C = I/128),
// so chunk q lies in column block q; the row's scale row is (row / 128).
template <int C, int DB>
struct DownRegs8 {
  uint4 w[DB][C];
  float s[DB][C];
};

template <int C, int DB, class P>
__device__ __forceinline__ void load_down8(DownRegs8<C, DB>& r, const P& p, int l, int e, int n,
                                           int n_end, int lane) {
  const int gl = lane >> 3, li = lane & 7;
  const size_t IB = (size_t)(p.I >> 7), HB = (size_t)(p.H >> 7);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const int row = n + 8 * b + gl < n_end ? n + 8 * b + gl : n;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.lw[l].wd) +
                                                      ((size_t)e * p.H + row) * p.I);
    const float* srow = p.lw[l].sd + ((size_t)e * HB + (size_t)(row >> 7)) * IB;
#pragma unroll
    for (int q = 0; q < C; ++q) {
      r.w[b][q] = ld_weight(src + li + 8 * q);
      r.s[b][q] = srow[q];
    }
  }
}

template <int C, int DB, typename Emit>
__device__ __forceinline__ void compute_down8(const DownRegs8<C, DB>& r, int I8, int n, int n_end,
                                              int nrows, const uint4* hv4, int lane, Emit emit) {
  const int gl = lane >> 3, li = lane & 7;
#pragma unroll 1
  for (int t = 0; t < nrows; ++t) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < C; ++q) {
        const int c = li + 8 * q;
        uint4 w = r.w[b][q];  // converted at the point of use (see dot_rows8)
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
        const float part = dot16_fp8(w, hv4[t * I8 + 2 * c], hv4[t * I8 + 2 * c + 1]);
        acc = fmaf(r.s[b][q], part, acc);
      }
      acc = group_sum(acc, 8);
      const int row = n + 8 * b + gl;
      if (li == 0 && row < n_end) emit(t, row, acc);
    }
  }
}

// ---------------------------------------------------------------- P4 / P5

// Softmax top-k with gates renormalised over the chosen experts: the router's
// second step in "Ling-3.0-flash on 4 Blackwell GPUs", section "PDL: stacking
// the latency floors of small kernels" (the router chain ends in a top-k), with
// K = 8 from section "The model".  The selection order is: larger logit first,
// lower expert index first among equal logits.
//
// Fast path (E = 512, K <= 8): one wave selects a row alone, with no barrier
// and no atomic (select_row_wave below).  Every other shape, and a row whose
// candidates do not fit one per lane, takes the plain method: K rounds of a
// wave-wide maximum.
//
// K rounds over one row held by one wave, PER keys per lane in lane-major
// blocks (lane L holds experts L*PER .. L*PER+PER-1); key 0 marks "no expert".
template <int PER>
__device__ __forceinline__ void select_rounds(const float* lr, const float* bias, int E, int K,
                                              int* out, int lane) {
  uint32_t keys[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * PER + i;
    keys[i] = e < E ? f_key(lr[e] + (bias ? bias[e] : 0.0f)) : 0u;
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

__device__ __forceinline__ void select_row_plain(const float* lr, const float* bias, int E, int K,
                                                 int* out, int lane) {
  const int per = (E + 63) >> 6;
  if (per <= 1) select_rounds<1>(lr, bias, E, K, out, lane);
  else if (per <= 2) select_rounds<2>(lr, bias, E, K, out, lane);
  else if (per <= 4) select_rounds<4>(lr, bias, E, K, out, lane);
  else if (per <= 8) select_rounds<8>(lr, bias, E, K, out, lane);
  else select_rounds<16>(lr, bias, E, K, out, lane);
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

// One row's selection by one wave, with no barrier and no atomic.  Lane l holds
// the scores of experts 8l .. 8l+7 (E = 512), so an 8-lane group holds 64
// experts.  The smallest of the eight group maxima, tau, has at least eight
// scores at or above it, so for K <= 8 the row's K winners are among the scores
// >= tau.  Those candidates (typically 20-30 of 512) are packed into this wave's
// LDS area as (key << 32 | ~expert), an order in which no two are equal and the
// larger comes first in the selection (higher score, then lower index).  Lane c
// takes candidate c and counts the candidates above it: its rank.  Returns false,
// having changed nothing but the wave's LDS area, when the candidates do not
// fit one per lane or are fewer than K (only NaN scores make them fewer); the
// caller then takes the plain rounds.  On success lane k < K holds the rank-k
// expert in e_k.  cw: 128 entries of this wave (the candidates, then one spare
// slot per lane).
__device__ __forceinline__ bool select_row_wave(const float* lr, const float (&bl)[8], int K,
                                                uint64_t* cw, int lane, int& e_k) {
  const float4 a = reinterpret_cast<const float4*>(lr)[2 * lane];
  const float4 b = reinterpret_cast<const float4*>(lr)[2 * lane + 1];
  const float s[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t key[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) key[i] = f_key(s[i] + bl[i]);
  uint32_t lm = key[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) lm = max(lm, key[i]);
  // maximum of the 8-lane group (quad swaps, then the half-row mirror)
  lm = max(lm, dpp_u<0xB1>(lm));
  lm = max(lm, dpp_u<0x4E>(lm));
  lm = max(lm, dpp_u<0x141>(lm));
  const uint32_t tau = ~wave_max_u32(~lm);  // the smallest group maximum
  uint32_t bits = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) bits |= (key[i] != 0u && key[i] >= tau) ? (1u << i) : 0u;
  const int c = __builtin_popcount(bits);
  const int incl = wave_incl_scan(c);
  const int n = __builtin_amdgcn_readlane(incl, 63);
  if (n < K || n > 64) return false;
  const int base = incl - c;
  // every lane stores all eight keys: candidates at their packed place, the
  // others into the lane's spare slot (no branch per key)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool cnd = (bits >> i) & 1u;
    const int at = cnd ? base + __builtin_popcount(bits & ((1u << i) - 1u)) : 64 + lane;
    cw[at] = ((uint64_t)key[i] << 32) | (uint64_t)(uint32_t)~(8 * lane + i);
  }
  const int n8 = (n + 7) & ~7;
  if (lane >= n && lane < n8) cw[lane] = 0ull;  // zero padding: never above a candidate
  const uint64_t mine = lane < n ? cw[lane] : 0ull;
  // rank: candidates above this one, eight at a time, the next eight in flight
  int rank = 0;
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cw);
  ulonglong2 q0 = c2[0], q1 = c2[1], q2 = c2[2], q3 = c2[3];
#pragma unroll 1
  for (int j = 0; j < n8; j += 8) {
    const uint64_t c8[8] = {q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
    if (j + 8 < n8) {
      q0 = c2[(j >> 1) + 4];
      q1 = c2[(j >> 1) + 5];
      q2 = c2[(j >> 1) + 6];
      q3 = c2[(j >> 1) + 7];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += c8[q] > mine ? 1 : 0;
  }
  // rank-k expert -> lane k, through the spare slots (free again)
  int* ek = reinterpret_cast<int*>(cw + 64);
  if (lane < n && rank < K) ek[rank] = (int)~(uint32_t)mine;
  e_k = lane < K ? ek[lane] : -1;
  return true;
}

// Gate of the rank-k expert held by lane k < K, computed as gates_from_idx
// computes it from the LDS table (shift by the rank-0 logit, sum over the K
// lanes, divide); 0 on the other lanes.
__device__ __forceinline__ float gate_of_rank(const float* lr, int K, int e_k, int lane) {
  const float lk = lane < K ? lr[e_k] : 0.0f;
  const float v0 = readlane_f(lk, 0);
  const float pk = lane < K ? expf(lk - v0) : 0.0f;
  const float s = group_sum(pk, 64);
  return lane < K ? pk / s : 0.0f;
}

// Every row's selection and gates: wave w takes rows w, w + 8, ...  bl: this
// lane's selection biases of experts 8 * lane .. 8 * lane + 7 (zeros without a
// bias), loaded before the logits arrive; bias: the bias vector for the plain
// path (or null).
template <class P>
__device__ __forceinline__ void topk_rows(const P& p, const float* lgs, const float (&bl)[8],
                                          const float* bias, Small* sm, int wv, int lane) {
  const int M = p.M, E = p.E, K = p.K;
  const bool fast = E == 512 && K <= 8;
  for (int m = wv; m < M; m += MOE_WAVES) {
    const float* lr = lgs + m * E;
    int ek;
    if (fast && select_row_wave(lr, bl, K, sm->cand + wv * 128, lane, ek)) {
      const float gk = gate_of_rank(lr, K, ek, lane);
      if (lane < K) {
        sm->tk_idx[m * K + lane] = ek;
        sm->tk_gate[m * K + lane] = gk;
      }
    } else {
      select_row_plain(lr, bias, E, K, sm->tk_idx + m * K, lane);
      gates_from_idx(lr, K, sm, m, lane);
    }
  }
}

// Routed slots in ascending expert order, their row masks and pair numbering.
// Built by wave 0 alone (its LDS operations execute in order), then one
// workgroup barrier publishes the tables.
template <class P>
__device__ __forceinline__ void build_union(const P& p, Small* sm, int wv, int lane) {
  constexpr int NE = kMaxPK / 64;  // entries (row, rank) per lane: i = lane + 64 j
  if (wv == 0) {
    // the lane number, opaque to the compiler: the lane-dependent values below
    // are made here, not hoisted out of the layer loop and held in registers
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int MK = p.M * p.K;
    // passes of 64 entries that hold any (row, rank) entry: one up to M * K = 64
    const int NJ = (MK + 63) >> 6;
    if (lane < 32) sm->bm[lane] = 0u;
#pragma unroll
    for (int j = 0; j < NE; ++j)
      if (j < NJ) sm->umask[lane + 64 * j] = 0u;
    int e[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      e[j] = -1;
      if (j < NJ) {
        e[j] = lane + 64 * j < MK ? sm->tk_idx[lane + 64 * j] : -1;
        if (e[j] >= 0) atomicOr(&sm->bm[e[j] >> 5], 1u << (e[j] & 31));
      }
    }
    const uint32_t w = lane < 32 ? sm->bm[lane] : 0u;
    const int c = __builtin_popcount(w);
    const int incl = wave_incl_scan(c);
    const int U = __builtin_amdgcn_readlane(incl, 63);
    if (lane < 32) sm->bpre[lane] = incl - c;
    if (lane == 0) sm->nU = U;
    // routed slot of each entry = number of selected experts below it
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      if (j >= NJ) break;
      int r = -1;
      if (e[j] >= 0) {
        r = sm->bpre[e[j] >> 5] + __builtin_popcount(sm->bm[e[j] >> 5] & ((1u << (e[j] & 31)) - 1u));
        sm->uexp[r] = e[j];
        atomicOr(&sm->umask[r], 1u << ((lane + 64 * j) / p.K));
      }
      if (lane + 64 * j < MK) sm->upos[lane + 64 * j] = r;
    }
    // first (slot, row) pair of every slot (U <= M * K: no more passes than above)
    int run = 0;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      if (j >= NJ) break;
      const int cj = lane + 64 * j < U ? __builtin_popcount(sm->umask[lane + 64 * j]) : 0;
      const int ij = wave_incl_scan(cj);
      sm->pbase[lane + 64 * j] = run + ij - cj;
      run += __builtin_amdgcn_readlane(ij, 63);
    }
    if (lane == 63) {
      sm->nP = run;
      sm->pbase[kMaxPK] = run;
    }
  }
  __syncthreads();
}

// Piece q (0 or 1) of this workgroup's slice of the routed work: expert slot r,
// intermediate range [j0, j1) and down rows [n0, n1).  Returns false if none.
struct Piece {
  int r, j0, j1, n0, n1;
};

// Piece q (0 or 1) of the range [s0, s1) of the (slot, output row) space, in
// units of 1/SG slot; a range of at most one slot lies in at most two slots.
// (32-bit arithmetic: s0, s1 <= 512 U, U <= 256, and a, b <= SG <= 512, so
// every product stays below 2^31)
__device__ __forceinline__ bool range_piece(int s0, int s1, int SG, int U, int I, int H, int q,
                                            Piece& pc) {
  if (U <= 0) return false;
  const int r = (int)((uint32_t)s0 / (uint32_t)SG) + q;
  if (r * SG >= s1 || r >= U) return false;
  int a = s0 - r * SG, b = s1 - r * SG;
  if (a < 0) a = 0;
  if (b > SG) b = SG;
  if (b <= a) return false;
  const uint32_t I2 = (uint32_t)I >> 1, H2 = (uint32_t)H >> 1, uG = (uint32_t)SG;
  pc.r = r;
  pc.j0 = 2 * (int)(((uint32_t)a * I2 + uG / 2) / uG);
  pc.j1 = 2 * (int)(((uint32_t)b * I2 + uG / 2) / uG);
  pc.n0 = 2 * (int)(((uint32_t)a * H2 + uG / 2) / uG);
  pc.n1 = 2 * (int)(((uint32_t)b * H2 + uG / 2) / uG);
  return true;
}

// Routed part of the combine for token row m and output rows (nl, nl + 1):
// q = sum over k < K, in order, of gate_k * y(slot of rank k), skipping a rank
// with no slot.  Every index is read before any value is summed (ranks past K
// repeat rank K - 1 and are not summed), so the three dependent LDS reads of a
// rank overlap across the ranks instead of following one another.
template <int KM>
__device__ __forceinline__ void routed_sum(const Small* sm, const float* ysr, int K, int m, int NR,
                                           int nl, float& q0, float& q1) {
  int pr[KM];
  float gk[KM];
  bool ok[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int kk = k < K ? k : K - 1;
    const int r = sm->upos[m * K + kk];
    ok[k] = k < K && r >= 0;
    const int rr = r >= 0 ? r : 0;
    const int pv = sm->pbase[rr] + __builtin_popcount(sm->umask[rr] & ((1u << m) - 1u));
    pr[k] = ok[k] ? pv : 0;
    gk[k] = sm->tk_gate[m * K + kk];
  }
  q0 = 0.0f;
  q1 = 0.0f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const float y0 = ysr[pr[k] * NR + nl], y1 = ysr[pr[k] * NR + nl + 1];
    q0 = ok[k] ? q0 + gk[k] * y0 : q0;
    q1 = ok[k] ? q1 + gk[k] * y1 : q1;
  }
}

// ---------------------------------------------------------------- the kernel

// W8: expert weights are fp8 e4m3 codes with 128 x 128 block scales (the
// router stays bf16); C8I fp8 chunks per down-row lane, DB8 down blocks per task.
template <int CPLH, int CPLI, int DBLK, int NL, bool W8 = false>
__global__ __launch_bounds__(MOE_WG, 1) void moe_layer_kernel(ParamsT<NL> p) {
  constexpr int C8I = CPLI / 2 > 0 ? CPLI / 2 : 1;
  constexpr int DB8 = 6 / C8I < 1 ? 1 : (6 / C8I > 4 ? 4 : 6 / C8I);
  constexpr int DB = W8 ? DB8 : DBLK;
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + p.lds_xs);
  const uint4* xs4 = reinterpret_cast<const uint4*>(xs);
  float* lgs = reinterpret_cast<float*>(lds + p.lds_lg);
  uint32_t* hs32 = reinterpret_cast<uint32_t*>(lds + p.lds_hs);
  const uint4* hs4 = reinterpret_cast<const uint4*>(lds + p.lds_hs);
  float* ysh = reinterpret_cast<float*>(lds + p.lds_ysh);
  float* ysr = reinterpret_cast<float*>(lds + p.lds_ysr);
  uint4* gn4 = reinterpret_cast<uint4*>(lds + p.lds_gn);
  static_assert(CPLH * 32 <= MOE_WG, "one 16-byte gain chunk per thread");
  Small* sm = reinterpret_cast<Small*>(lds + p.lds_small);

  const int G = gridDim.x, g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cp = g % kCopies;  // the copy this workgroup reads (see kCopies)
  const int NW = G * MOE_WAVES;
  const int gw = wv * G + g;  // consecutive wave ids land on different CUs
  // The step tag, debug flags and deadline come with the launch: no word of
  // the workspace is read before the first weight loads are issued, and no
  // end-of-call counting is needed to advance the step.
  const uint32_t tag = p.tag;
  const uint32_t dbg = p.dbg;
  Waiter wt{p.hdr, now_ticks() + p.budget};
  const int M = p.M, H = p.H, I = p.I, K = p.K, S = p.S, E = p.E;
  const int I2 = I >> 1, H2 = H >> 1, I8 = I >> 3;
  const int MK = M * K;
  const bool router_only = (p.flags & F_ROUTER_ONLY) != 0u;
  const bool topk_in = (p.flags & F_TOPK_IN) != 0u;

  if (tid == 0) sm->abort_flag = 0;
  // the input-read counter of this call's tag parity; the other one, which the
  // next call on this workspace uses, is cleared now (the previous call that
  // used it has completed)
  const int xread = (tag & 1u) ? HDR_XREAD1 : HDR_XREAD0;
  if (g == 0 && tid == 0) st_u32(p.hdr + ((tag & 1u) ? HDR_XREAD0 : HDR_XREAD1), 0u);
  uint64_t* stamps = ((dbg & DBG_STAMPS) && g < STAMP_WG)
                         ? reinterpret_cast<uint64_t*>(p.hdr + HDR_STAMPS) + (size_t)g * STAMP_SLOTS
                         : nullptr;
  int sbase = 0;
#define MOE_STAMP(ev)                                                          \
  do {                                                                         \
    if (stamps && tid == 0 && sbase >= 0) stamps[sbase + (ev)] = now_ticks(); \
  } while (0)

  // output rows owned by this workgroup (whole row pairs)
  const int r0 = (int)((uint32_t)(g * H2) / (uint32_t)G);
  const int r1 = (int)((uint32_t)((g + 1) * H2) / (uint32_t)G);
  const int n0 = 2 * r0, NR = 2 * (r1 - r0);

  // A single-layer launch (one weight slot) has no layer loop: the compiler
  // then tracks every load and store of the call exactly and waits only for
  // the ones a value depends on, where a loop's back edge makes it wait for all
  // of them (stores included) at many points.  (A `for` loop of one iteration
  // kept its back edge, taken when the abort flag is clear, so the loop's
  // condition is written into the `while` itself: with one slot the body has no
  // way back.)
  const int L = NL == 1 ? 1 : p.L;
  int l = 0;
  do {
    // the thread number, opaque to the compiler: values derived from it are
    // made again in every layer instead of being hoisted out of the layer loop
    // and held in registers through every phase
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o;
    const int lane = tid & 63;
    sbase = l == 0 ? 0 : (l == 1 ? 10 : (l == L - 1 ? 20 : -1));
    MOE_STAMP(0);
    // ---------------- P1 prefetch: this wave's first router / shared gate-up rows
    // do not depend on x, so their loads fly while x is staged
    const int NRI = topk_in ? 0 : (E + 1) >> 1;
    // One token row (fast selection shape): the shared expert's gate/up items
    // wait for the selection window (see P4), so that the first loads of the
    // call are the router rows and x alone.
    // In the layer loop the bf16 items go through the LDS slots of waves 1-2,
    // at most one per wave (see P4); where those do not fit they stay in P1.
    const bool sh_late = M == 1 && K <= 8 && !topk_in && !router_only && E == 512 && S &&
                         (NL == 1 || W8 || (p.lds_p1w >= 0 && I2 <= 2 * G));
    const int NSI = (router_only || !S || sh_late) ? 0 : I2;
    // bf16, two token rows on (where LDS has room): the token rows of a P1 item
    // are spread over all eight waves.  The item's wave (0-2) loads its rows as
    // before and copies them into its LDS slot, [unit][chunk][lane]; each wave
    // then computes whole token rows from LDS.  One wave would otherwise take
    // M dependent dot products per item (about 1.9 us for a router pair at
    // M = 6, twice that for a shared item), which the logits wait for.
    // (made again where used, from the launch's values, not held through P0)
    auto p1s_on = [&]() __attribute__((always_inline)) {
      return p.M >= 2 && p.lds_p1w >= 0 && NRI + NSI <= 3 * (int)gridDim.x;
    };
    auto p1w_at = [&]() __attribute__((always_inline)) {
      return reinterpret_cast<uint4*>(lds + p.lds_p1w);
    };
    // one slot, in 16-byte units: unit A [CPLH][64], unit B [CPLH][64], then
    // an fp8 shared item's scales [C][64] fp32
    constexpr int kP1Slot = 2 * CPLH * 64 + 16 * Fp8Row<CPLH>::C;
    RowRegs<CPLH> A, B;
    float SC[Fp8Row<CPLH>::C];
    if constexpr (NL > 1) {
      // left undefined on the waves without an item, the rows would be values
      // that the layer loop carries from one layer to the next, held in
      // registers through every phase
      A = {};
      B = {};
    }
    if (gw < NRI + NSI) p1_load<CPLH, W8>(p, l, gw, NRI, A, B, SC, lane, false);

    // ---------------- P0: layer input -> LDS
    // The norm's gain does not depend on the input: its load flies during the
    // stage.  It is loaded straight into LDS (lane l's 16 bytes land 16 l bytes past
    // the wave's base): no registers hold it, and no default value is written
    // into registers that the previous layer's loads may still be filling (the
    // layer loop would wait there for every load in flight).  A layer without
    // a gain reads a chunk of bf16 ones in every lane.
    if ((p.flags & F_PRENORM) && tid < (H >> 3)) {
      const uint16_t* gain = p.lw[l].gain;
      const uint4* src = gain ? reinterpret_cast<const uint4*>(gain) + tid : &kBf16OnesChunk;
      const int wvu = __builtin_amdgcn_readfirstlane(tid >> 6);
      __builtin_amdgcn_global_load_lds(src, (LdsPtr)(gn4 + 64 * wvu), 16, 0, 0);
    }
    if (tid == 0) {
      sm->gu_next = 0;  // read after the barriers of the routing phase
      sm->dn_next = 0;
      sm->dn_done = 0;
      sm->st_next = 0;
      sm->st_done = 0ull;
    }
    if (l == 0) {
      const uint4* src = reinterpret_cast<const uint4*>(p.x_in);
      uint4* dst = reinterpret_cast<uint4*>(xs);
      for (int i = tid; i < (M * H) >> 3; i += MOE_WG) dst[i] = src[i];
    } else {
      // One token row: waves 1-7 poll, three words per lane.  Wave 0's router
      // rows are in flight and a wave's loads return in order, so its polls
      // would wait behind them; fewer polling lanes also load the exchange
      // less.  (From two token rows on, where waves 0-2 hold P1 items, polling
      // from the other five waves measured slower.)
      const uint64_t* src = p.res_buf + ((size_t)l * kCopies + cp) * M * H2;
      if (M == 1 && H2 <= 3 * (MOE_WG - 64)) {
        if (tid >= 64 && !stage_tagged<3, MOE_WG - 64>(H2, reinterpret_cast<uint32_t*>(xs), tag, wt,
                                                       tid - 64, [&](int i) { return src + i; }))
          sm->abort_flag = 1;
      } else if (!stage_tagged<8>(M * H2, reinterpret_cast<uint32_t*>(xs), tag, wt, tid,
                                  [&](int i) { return src + i; })) {
        sm->abort_flag = 1;
      }
    }
    // (the gain's direct loads have landed: vmcnt(0), expcnt and lgkmcnt left free)
    if (p.flags & F_PRENORM) __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (l == 0 && tid == 0 && (p.flags & F_ALIAS)) add_u32(p.hdr + xread, 1u);
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
      // Sum of squares per row in double: every bf16 value and its square are
      // exact in double and, over the value range of a residual stream, every
      // partial sum is exact in double, so the sum (and the scale) does not
      // depend on the order.  A wave's chunks are all requested before any is
      // used, into four partial sums.
      const int H8 = H >> 3;
      constexpr int J = (CPLH + 1) / 2;  // chunks per lane (H8 = 32 CPLH)
      for (int m = wv; m < M; m += MOE_WAVES) {
        uint4 v[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int c = lane + 64 * j;
          v[j] = xs4[m * H8 + (c < H8 ? c : 0)];
        }
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t mk = lane + 64 * j < H8 ? 0xFFFFFFFFu : 0u;
          const uint32_t w4[4] = {v[j].x & mk, v[j].y & mk, v[j].z & mk, v[j].w & mk};
#pragma unroll
          for (int q = 0; q < 4; q += 2) {
            const double a = bf_lo(w4[q]), b = bf_hi(w4[q]);
            const double c = bf_lo(w4[q + 1]), d = bf_hi(w4[q + 1]);
            s0 = __builtin_fma(a, a, s0);
            s1 = __builtin_fma(b, b, s1);
            s2 = __builtin_fma(c, c, s2);
            s3 = __builtin_fma(d, d, s3);
          }
        }
        const double ss = wave_sum_f64((s0 + s1) + (s2 + s3));
        if (lane == 0) sm->rn[m] = (float)(1.0 / sqrt(ss / (double)H + (double)kRmsEps));
      }
      __syncthreads();
      // u = bf16((h * r) * gain): two fp32 products, one rounding; (row,
      // 16-byte chunk) units over all threads
      for (int i = tid; i < M * H8; i += MOE_WG) {
        const int m = i / H8, c = i - m * H8;
        const uint4 xv = xs4[i], gv = gn4[c];
        const float r = sm->rn[m];
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w}, g4[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o4[e] = pk_bf((bf_lo(w4[e]) * r) * bf_lo(g4[e]), (bf_hi(w4[e]) * r) * bf_hi(g4[e]));
        reinterpret_cast<uint4*>(xs)[i] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
      }
    }
    if (p1s_on() && gw < NRI + NSI) {
      // slot: unit A [CPLH][64], unit B [CPLH][64] (16-byte chunks); fp8 shared
      // items use C chunks of each and keep their scales [C][64] after B
      uint4* sl = p1w_at() + (size_t)wv * kP1Slot;
      if (W8 && gw >= NRI) {
#pragma unroll
        for (int q = 0; q < Fp8Row<CPLH>::C; ++q) {
          sl[q * 64 + lane] = A.w[q];
          reinterpret_cast<float*>(sl + 2 * CPLH * 64)[q * 64 + lane] = SC[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < CPLH; ++q) sl[q * 64 + lane] = A.w[q];
      }
    }
    __syncthreads();
    MOE_STAMP(1);

    // ---------------- P1: router rows + shared expert gate/up rows
    if (!p1s_on()) {
      for (int it = gw; it < NRI + NSI; it += NW) {
        if (it != gw)
          p1_load<CPLH, W8>(p, l, it, NRI, A, B, SC, lane, true);
        else if (it >= NRI)  // the prefetched gate/up item still needs its second row
          p1_load_second<CPLH, W8>(p, l, it, NRI, B, lane);
        p1_compute<CPLH, W8>(p, l, it, NRI, A, B, SC, xs4, tag, lane, dbg);
      }
    } else {
      // items of waves 0-2: router items first (w G + g < NRI), then shared ones
      const int H8 = H >> 3;
      int nri = 0, nsi = 0;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const int it = w * G + g;
        nri += it < NRI ? 1 : 0;
        nsi += (it >= NRI && it < NRI + NSI) ? 1 : 0;
      }
      const bool own_sh = gw >= NRI && gw < NRI + NSI;
      uint4* p1w = p1w_at();
      if (own_sh) p1_load_second<CPLH, W8>(p, l, gw, NRI, B, lane);  // flies during the router rows
      for (int u = wv; u < nri * M; u += MOE_WAVES) {
        const int w = u / M, m = u - w * M;
        const uint4* sl = p1w + (size_t)w * kP1Slot;
        publish_logit(p, l, w * G + g, m,
                      dot_rows_w<CPLH>([&](int q) { return sl[q * 64 + lane]; }, xs4, H8, m, lane),
                      tag, lane, dbg);
      }
      if (own_sh) {
        uint4* sl = p1w + (size_t)wv * kP1Slot + CPLH * 64;
        constexpr int NB = W8 ? Fp8Row<CPLH>::C : CPLH;
#pragma unroll
        for (int q = 0; q < NB; ++q) sl[q * 64 + lane] = B.w[q];
      }
      __syncthreads();
      for (int u = wv; u < nsi * M; u += MOE_WAVES) {
        const int w = nri + u / M, m = u - (u / M) * M;
        const uint4* sl = p1w + (size_t)w * kP1Slot;
        float a0, a1;
        if constexpr (W8) {
          const float* ss = reinterpret_cast<const float*>(sl + 2 * CPLH * 64);
          a0 = dot_rows8_lds<CPLH>(sl, ss, xs4, H, m, lane);
          a1 = dot_rows8_lds<CPLH>(sl + CPLH * 64, ss, xs4, H, m, lane);
        } else {
          a0 = dot_rows_w<CPLH>([&](int q) { return sl[q * 64 + lane]; }, xs4, H8, m, lane);
          a1 = dot_rows_w<CPLH>([&](int q) { return sl[(CPLH + q) * 64 + lane]; }, xs4, H8, m, lane);
        }
        publish_shared(p, l, w * G + g - NRI, m, a0, a1, tag, lane);
      }
    }
    MOE_STAMP(2);

    // router only: workgroup 0 gathers every workgroup's logits and computes
    // the top-k; the others are done
    if (router_only && g != 0) return;

    // ---------------- P4: routing
    // one token row (K <= 8): the routed slots are the ranks (see P5)
    const bool one_row = M == 1 && K <= 8 && !topk_in && !router_only;
    bool ranked = false;  // one row selected on the fast path, slot tables filled
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
      // the selection bias does not depend on the logits: this lane's eight
      // (experts 8 * lane .. 8 * lane + 7) are loaded before waiting
      const float* bias = p.lw[l].bias;
      float bl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bl[i] = (bias && E == 512) ? bias[8 * lane + i] : 0.0f;
      const uint64_t* src = p.lg_buf + ((size_t)l * kCopies + cp) * M * E;
      // One token row: a single wave polls the 512 logit words (eight per
      // lane, in flight together); 512 polling lanes in each of 256
      // workgroups slowed the exchange they waited on.
      if (one_row && E <= 512) {
        if (wv == 1 && !stage_tagged<8, 64>(M * E, reinterpret_cast<uint32_t*>(lgs), tag, wt, lane,
                                            [&](int i) { return src + i; }))
          sm->abort_flag = 1;
      } else if (!stage_tagged<8>(M * E, reinterpret_cast<uint32_t*>(lgs), tag, wt, tid,
                                  [&](int i) { return src + i; })) {
        sm->abort_flag = 1;
      }
      __syncthreads();
      MOE_STAMP(3);
      if (sm->abort_flag == 1) break;
      // One token row: wave 0 selects alone and fills the workgroup's slot
      // tables (slot r = rank r); one barrier publishes them.  The selection is
      // a chain of dependent wave-wide steps, and a second wave on the same
      // SIMD would only halve its issue rate.  A row whose candidates do not
      // fit one per lane takes the plain path below.
      if (one_row && E == 512) {
        if (wv == 0) {
          int ln = lane;  // opaque lane number (no hoisted lane-dependent addresses)
          asm volatile("" : "+v"(ln));
          int ek;
          const bool ok = select_row_wave(lgs, bl, K, sm->cand, ln, ek);
          if (ok) {
            const float gk = gate_of_rank(lgs, K, ek, ln);
            if (ln < K) {
              sm->tk_idx[ln] = ek;
              sm->tk_gate[ln] = gk;
              sm->uexp[ln] = ek;
              sm->umask[ln] = 1u;
              sm->pbase[ln] = ln;
              sm->upos[ln] = ln;
            }
            if (ln == 0) {
              sm->nU = K;
              sm->nP = K;
            }
            if (g == 0 && ln < K) {
              if (p.tk_idx_out) p.tk_idx_out[(size_t)l * MK + ln] = ek;
              if (p.tk_gate_out && l == 0) p.tk_gate_out[ln] = gk;
            }
          }
          if (ln == 0) sm->sel_ok = ok ? 1 : 0;
        } else if (sh_late && wv <= 2) {
          // the shared expert's gate/up items.  The first one's rows are
          // requested while wave 0 selects and used after the barrier, so that
          // the barrier does not wait for their memory latency: in the
          // single-layer kernel into registers, in the layer loop (which has
          // no registers to hold them across the barrier) straight into the
          // wave's LDS slot; fp8 items in the loop are computed before it.
          const int j0 = (wv - 1) * G + g;
          if (NL == 1) {
            if (j0 < I2) p1_load<CPLH, W8>(p, l, NRI + j0, NRI, A, B, SC, lane, true);
          } else if constexpr (!W8) {
            const int wvu = __builtin_amdgcn_readfirstlane(wv);
            if (j0 < I2) p1_shared_to_lds<CPLH>(p, l, NRI + j0, NRI, p1w_at() + (size_t)wvu * kP1Slot, lane);
          } else {
            for (int j = j0; j < I2; j += 2 * G) {
              p1_load<CPLH, W8>(p, l, NRI + j, NRI, A, B, SC, lane, true);
              p1_compute<CPLH, W8>(p, l, NRI + j, NRI, A, B, SC, xs4, tag, lane, dbg);
            }
          }
        }
        __syncthreads();
        if (NL == 1 && sh_late && wv >= 1 && wv <= 2) {
          for (int j = (wv - 1) * G + g; j < I2; j += 2 * G) {
            if (j != (wv - 1) * G + g) p1_load<CPLH, W8>(p, l, NRI + j, NRI, A, B, SC, lane, true);
            p1_compute<CPLH, W8>(p, l, NRI + j, NRI, A, B, SC, xs4, tag, lane, dbg);
          }
        } else if (NL > 1 && !W8 && sh_late && wv >= 1 && wv <= 2) {
          const int j0 = (wv - 1) * G + g;
          if (j0 < I2) {
            const int wvu = __builtin_amdgcn_readfirstlane(wv);
            const uint4* sl = p1w_at() + (size_t)wvu * kP1Slot;
            // the slot's direct loads have landed (they are the wave's only
            // loads in flight since the barrier)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const int H8 = H >> 3;
            const float a0 = dot_rows_w<CPLH>([&](int q) { return sl[q * 64 + lane]; }, xs4, H8, 0, lane);
            const float a1 =
                dot_rows_w<CPLH>([&](int q) { return sl[(CPLH + q) * 64 + lane]; }, xs4, H8, 0, lane);
            publish_shared(p, l, j0, 0, a0, a1, tag, lane);
          }
        }
        ranked = sm->sel_ok != 0;
        if (ranked) {
          if (g == 0 && p.logits_out && l == 0)
            for (int i = tid; i < E; i += MOE_WG) p.logits_out[i] = lgs[i];
          MOE_STAMP(9);
        }
      }
      if (!ranked) {
        topk_rows(p, lgs, bl, bias, sm, wv, lane);
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
    }

    // ---------------- P5: routed slots
    // One token row (K <= 8): the routed slots are the ranks (slot r = rank r,
    // one row each), so there is nothing to merge.  On the fast path wave 0 has
    // filled the workgroup's tables already.  After the plain path each wave
    // copies the selection into its own slot table, which only it reads, so no
    // barrier stands between the selection and the routed gate/up stream; wave 0
    // fills the workgroup's tables, which the down projection and the combine
    // read after the barrier that opens the down projection.
    int U;
    if (ranked) {
      U = K;
    } else if (one_row) {
      // the lane number, opaque to the compiler: the addresses built from it
      // are made here, not hoisted out of the layer loop and held in registers
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int e = ln < K ? sm->tk_idx[ln] : -1;  // valid ranks form a prefix
      U = (int)__builtin_popcountll(__ballot(e >= 0));
      if (ln < U) {
        sm->uexp[kOwnSlots + wv * 8 + ln] = e;
        sm->umask[kOwnSlots + wv * 8 + ln] = 1u;
        sm->pbase[kOwnSlots + wv * 8 + ln] = ln;
      }
      if (wv == 0) {
        if (ln < U) {
          sm->uexp[ln] = e;
          sm->umask[ln] = 1u;
          sm->pbase[ln] = ln;
        }
        if (ln < K) sm->upos[ln] = ln < U ? ln : -1;
        if (ln == 0) {
          sm->nU = U;
          sm->nP = U;
        }
      }
    } else {
      build_union(p, sm, wv, lane);
      U = sm->nU;
    }
    MOE_STAMP(4);

    // ---------------- P6: routed gate/up rows
    // A task is one intermediate pair jp of one routed slot: gate/up rows
    // j = 2jp (unit A) and 2jp + 1 (unit B), both requested before either is
    // used.  This workgroup's slice (pieces of at most two slots) still fixes
    // its down-projection work below.
    uint64_t* hr_l = p.hr_buf + (size_t)l * MK * I2;

    {
      const int H8 = H >> 3;
      // one task: SwiGLU of gate/up row pairs (2jp, 2jp + 1) for every row that chose slot rr
      // the slot tables: the workgroup's, or with one token row off the fast
      // path this wave's own
      const int so = (one_row && !ranked) ? kOwnSlots + wv * 8 : 0;
      auto emit_task = [&](const RowRegs<CPLH>& X, const RowRegs<CPLH>& Y,
                           const float (&S)[Fp8Row<CPLH>::C], int jp, int rr)
                           __attribute__((always_inline)) {
        uint64_t* dst = hr_l + (size_t)sm->pbase[so + rr] * I2 + jp;
        uint32_t bits = sm->umask[so + rr];
        int t = 0;
#pragma unroll 1
        while (bits) {
          const int m = __builtin_ctz(bits);
          bits &= bits - 1u;
          float a0, a1;
          if constexpr (W8) {
            a0 = dot_rows8<CPLH>(X, S, xs4, H, m, lane);
            a1 = dot_rows8<CPLH>(Y, S, xs4, H, m, lane);
          } else {
            a0 = dot_rows<CPLH>(X, xs4, H8, m, lane);
            a1 = dot_rows<CPLH>(Y, xs4, H8, m, lane);
          }
          const uint32_t word = pk_bf(swiglu(readlane_f(a0, 0), readlane_f(a0, 32)),
                                      swiglu(readlane_f(a1, 0), readlane_f(a1, 32)));
          if (lane == 0) st_tag(dst + (size_t)t * I2, word, tag);
          ++t;
        }
      };
      // Tasks t = (slot, pair) over the whole union, dealt round-robin: workgroup
      // g takes t = g, g + G, ...  Every workgroup then streams from every
      // selected expert, which evens out the per-workgroup finish times far
      // better than contiguous slices.  Inside the workgroup the waves take
      // those tasks in order from a ticket counter in LDS: the two waves that
      // share a SIMD do not issue at the same rate (the older one goes first),
      // so a fixed deal per wave leaves half the waves a task or more behind.
      // The next ticket is taken while the current task's rows are in flight.
      const int T = U * I2;
      // Workgroups 2i (on an even XCD) and 2i + 1 (on an odd one) hold the
      // tasks 2i + G k and 2i + 1 + G k.  The odd XCDs stream a few percent
      // slower (their workgroups end the phase about 4.5 us later at M = 6),
      // so the even partner also takes the odd one's task of every
      // k = XW - 1 (mod XW), right after its own of the same k: the tasks
      // still complete in slot order, and the even side does 16/15 of the
      // odd side's tasks.  Only for bf16 and at least 32 tasks per workgroup
      // (fewer, as at one token row or the TP4 shard, measured no gain).
      // Ticket j of this workgroup -> task:
      constexpr int XW = 16;
      const bool xw_on = !W8 && (G & 1) == 0 && T >= 32 * G;
      auto task_of = [&](int j) __attribute__((always_inline)) {
        if (xw_on && (g & 1) == 0) {
          const int b = j / (XW + 1), r = j - b * (XW + 1);
          return r == XW ? g + 1 + G * (XW * b + XW - 1) : g + G * (XW * b + r);
        }
        if (xw_on) {
          const int b = j / (XW - 1), r = j - b * (XW - 1);
          return g + G * (XW * b + r);
        }
        return g + G * j;
      };
      auto ticket = [&]() __attribute__((always_inline)) {
        int v = 0;
        if (lane == 0) v = atomicAdd(&sm->gu_next, 1);
        return v;
      };
      if constexpr (W8) {
        const size_t HB = (size_t)(H >> 7);
        int tk = ticket();
        for (;;) {
          const int t = task_of(__builtin_amdgcn_readfirstlane(tk));
          if (t >= T) break;
          const int rr = t / I2;
          const int jp = t - rr * I2;
          const size_t j0 = 2 * (size_t)jp;
          const uint8_t* base = static_cast<const uint8_t*>(p.lw[l].wgu) +
                                (size_t)sm->uexp[so + rr] * (2 * (size_t)I) * H;
          load_rows8<CPLH>(A, base + j0 * H, base + ((size_t)I + j0) * H, H, lane);
          load_rows8<CPLH>(B, base + (j0 + 1) * H, base + ((size_t)I + j0 + 1) * H, H, lane);
          const float* sb = p.lw[l].sgu + (size_t)sm->uexp[so + rr] * ((2 * (size_t)I) >> 7) * HB;
          load_scales8<CPLH>(SC, sb + (j0 >> 7) * HB, sb + (((size_t)I + j0) >> 7) * HB, H, lane);
          tk = ticket();
          emit_task(A, B, SC, jp, rr);
        }
      } else {
        int tk = ticket();
        for (;;) {
          const int t = task_of(__builtin_amdgcn_readfirstlane(tk));
          if (t >= T) break;
          const int rr = t / I2;
          const int jp = t - rr * I2;
          const size_t j0 = 2 * (size_t)jp;
          const uint16_t* base = static_cast<const uint16_t*>(p.lw[l].wgu) +
                                 (size_t)sm->uexp[so + rr] * (2 * (size_t)I) * H;
          load_rows<CPLH>(A, base + j0 * H, base + ((size_t)I + j0) * H, lane);
          load_rows<CPLH>(B, base + (j0 + 1) * H, base + ((size_t)I + j0 + 1) * H, lane);
          tk = ticket();
          emit_task(A, B, SC, jp, rr);
        }
      }
    }
    MOE_STAMP(5);

    // ---------------- P7: down projection
    // This workgroup's down tasks: the shared expert's blocks of its own output
    // rows, then its slice's blocks of the routed experts.  Their SwiGLU inputs
    // are staged in LDS in chunks, and each task waits only for its own
    // segment's chunks (see below).
    uint64_t* y_l = p.y_buf + (size_t)l * MK * H;
    int dn_order = 0;  // one token row: this wave's place among the waves leaving the down loop
    {
      // (the thread number made opaque again: the lane-dependent values of the
      // down projection are made here, not hoisted into the gate/up phase)
      int tid_p7 = tid;
      asm volatile("" : "+v"(tid_p7));
      const int tid = tid_p7;
      const int lane = tid & 63;
      const int BR = 8 * DB;
      const int nbs = (S && NR > 0) ? (NR + BR - 1) / BR : 0;
      // This workgroup's down slice of the (slot, output row) space: G equal
      // slices in slot order (at most two pieces), or, folded, half-slice g of
      // the first half of the space and half-slice 2G - 1 - g of the second
      // (at most four pieces): every workgroup then starts on rows of early
      // slots while the last slots' gate/up tasks, whose finish varies most
      // between workgroups, are still completing.  Thread 0 writes the table
      // of pieces and staging segments into LDS (kept out of registers, which
      // the streaming loops need); the barrier below publishes it.
      if (tid == 0) {
        const int SG = p.fold ? 2 * G : G;
        int ws = nbs ? M * I2 : 0, nc = (ws + 511) >> 9, nt = nbs;
        sm->dk_ws[0] = 0;
        sm->dk_nc[0] = 0;
        for (int k = 0; k < 4; ++k) {
          Piece pc;
          const int hb = k >> 1;  // half-slice: 0 the first (or the only), 1 the folded one
          const int h0 = hb ? (2 * G - 1 - g) * U : g * U;
          const bool has = (hb == 0 || p.fold) && range_piece(h0, h0 + U, SG, U, I, H, k & 1, pc);
          const int nb = has ? (pc.n1 - pc.n0 + BR - 1) / BR : 0;
          const int nrow = has ? __builtin_popcount(sm->umask[pc.r]) : 0;
          sm->dk_r[k] = has ? pc.r : 0;
          sm->dk_n0[k] = has ? pc.n0 : 0;
          sm->dk_n1[k] = has ? pc.n1 : 0;
          sm->dk_nb[k] = nb;
          sm->dk_nrow[k] = nrow;
          sm->dk_pb[k] = has ? sm->pbase[pc.r] : 0;
          sm->dk_ws[k + 1] = ws;
          sm->dk_nc[k + 1] = nc;
          const int w = nb ? nrow * I2 : 0;
          ws += w;
          nc += (w + 511) >> 9;
          nt += nb;
        }
        sm->dk_ws[5] = ws;
        sm->dk_nc[5] = nc;
        sm->dk_ntask = nt;
      }
      // (without the barrier the SwiGLU rows staged below would overwrite x,
      // which the routed gate/up rows read; the slot tables read below may
      // come from wave 0 alone with one token row)
      __syncthreads();
      const int ntask = sm->dk_ntask;
      // task f -> (expert, first row, end row, kind: 0 shared, 1 + k piece k)
      auto task = [&](int f, int& e, int& n, int& n_end, int& kind) __attribute__((always_inline)) {
        e = E; n = n0 + f * BR; n_end = n0 + NR; kind = 0;
        if (f < nbs) return;
        f -= nbs;
        for (int k = 0; k < 4; ++k) {
          const int nb = sm->dk_nb[k];
          if (f < nb) {
            e = sm->uexp[sm->dk_r[k]]; n = sm->dk_n0[k] + f * BR; n_end = sm->dk_n1[k]; kind = 1 + k;
            return;
          }
          f -= nb;
        }
      };
      using DR = std::conditional_t<W8, DownRegs8<C8I, DB8>, DownRegs<CPLI, DBLK>>;
      DR DA;
      int e, n, n_end, kind;
      const uint64_t* hsrc = p.hs_buf + ((size_t)l * kCopies + cp) * M * I2;
      // The SwiGLU inputs of the tasks are staged into LDS in segments (shared
      // | piece 0 .. piece 3, words of two bf16), in chunks of up to 512 words,
      // each within one segment, which the waves claim from an LDS counter; a
      // down task waits only for its own segment's chunks, so the shared blocks
      // and an earlier slot's blocks start while a later slot's rows are still
      // on their way.  Bit c of st_done: chunk c is in LDS (also after a missed
      // deadline, so that no wave waits on it).  At most 5 ceil(MOE_MAXM I /
      // 1024) chunks (60 for I = 768).
      static_assert(5 * ((MOE_MAXM * 32 * CPLI + 511) / 512) <= 64, "staging chunks fit the mask");
      {
        const int nct = sm->dk_nc[5];
        // a wave claims at most 65 times (at most 64 chunks)
        for (int claim = 0; claim <= 64; ++claim) {
          int c = 0;
          if (lane == 0) c = atomicAdd(&sm->st_next, 1);
          c = lane0_scalar(c);
          if (c >= nct) break;
          int sg = 0;
          while (sg < 4 && c >= sm->dk_nc[sg + 1]) ++sg;
          sg = lane0_scalar(sg);
          const int a = sm->dk_ws[sg] + (c - sm->dk_nc[sg]) * 512, b = sm->dk_ws[sg + 1];
          const uint64_t* src = (sg == 0 ? hsrc : hr_l + (size_t)sm->dk_pb[sg - 1] * I2) - sm->dk_ws[sg];
          if (!stage_tagged<8, 64>(min(512, b - a), hs32 + a, tag, wt, lane,
                                   [&](int i) { return src + (a + i); }))
            sm->abort_flag = 1;
          if (lane == 0)
            __hip_atomic_fetch_or(&sm->st_done, 1ull << c, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      MOE_STAMP(6);
      // the chunks of segment kd
      auto await_inputs = [&](int kd) __attribute__((always_inline)) {
        const int c0 = sm->dk_nc[kd], nc = sm->dk_nc[kd + 1] - c0;
        const uint64_t need = (nc >= 64 ? ~0ull : ((1ull << nc) - 1ull)) << c0;
        while ((__hip_atomic_load(&sm->st_done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) & need) != need) {
          if (wt.expired()) {
            record_status(p.hdr, -6 /* MOE_E_TIMEOUT */);
            sm->abort_flag = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      };
      auto down = [&](const DR& R, int nn, int ne, int nrows, const uint4* hv, auto emit)
                      __attribute__((always_inline)) {
        if constexpr (W8)
          compute_down8<C8I, DB8>(R, I8, nn, ne, nrows, hv, lane, emit);
        else
          compute_down<CPLI, DBLK>(R, I8, nn, ne, nrows, hv, lane, emit);
      };
      auto run = [&](int f, const DR& R) __attribute__((always_inline)) {
        int e2, nn, ne, kd;
        task(f, e2, nn, ne, kd);
        await_inputs(kd);
        if (kd == 0) {
          down(R, nn, ne, M, hs4, [&](int m, int row, float y) {
            ysh[m * p.nr_max + (row - n0)] = y;
          });
        } else {
          const int pb = sm->dk_pb[kd - 1], nr = sm->dk_nrow[kd - 1];
          const uint4* hv = hs4 + (size_t)sm->dk_ws[kd] / 4;
          down(R, nn, ne, nr, hv, [&](int t, int row, float y) {
            st_tag(y_l + (size_t)(pb + t) * H + row, __float_as_uint(y), tag);
          });
        }
      };
      // the down tasks, too, go to the waves in order from a ticket counter
      int tk = 0;
      if (lane == 0) tk = atomicAdd(&sm->dn_next, 1);
      for (;;) {
        const int f = lane0_scalar(tk);
        if (f >= ntask) break;
        task(f, e, n, n_end, kind);
        if constexpr (W8)
          load_down8<C8I, DB8>(DA, p, l, e, n, n_end, lane);
        else
          load_down<CPLI, DBLK>(DA, p, l, e, n, n_end, lane);
        if (lane == 0) tk = atomicAdd(&sm->dn_next, 1);
        run(f, DA);
      }
      if (M == 1) {
        int o = 0;
        if (lane == 0) o = atomicAdd(&sm->dn_done, 1);
        dn_order = lane0_scalar(o);
      }
      __syncthreads();
      if (sm->abort_flag == 1) break;
    }
    MOE_STAMP(7);

    // ---------------- P8: combine (+ residual) and hand off
    const bool last = (l == L - 1);
    if (last && (p.flags & F_ALIAS)) {
      if (tid == 0) {
        for (;;) {
          if (ld_u32(p.hdr + xread) >= (uint32_t)G) break;
          if (wt.expired()) { record_status(p.hdr, -6); sm->abort_flag = 1; break; }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
      if (sm->abort_flag == 1) break;
    }
    if (NR > 0) {
      // this workgroup's rows of every routed (expert, row) output -> LDS
      const int nP = sm->nP;
      auto yat = [&](int i) {
        const int pr = i / NR;
        return y_l + (size_t)pr * H + n0 + (i - pr * NR);
      };
      // One token row: the first two waves to leave the down loop poll (one
      // word per lane).  A wave's loads and stores retire in order, so the
      // waves whose own down-output stores are oldest see the words soonest.
      if (M == 1 && nP * NR <= 128) {
        if (dn_order < 2 &&
            !stage_tagged<1, 128>(nP * NR, reinterpret_cast<uint32_t*>(ysr), tag, wt,
                                  dn_order * 64 + lane, yat))
          sm->abort_flag = 1;
      } else if (!stage_tagged<4>(nP * NR, reinterpret_cast<uint32_t*>(ysr), tag, wt, tid, yat)) {
        sm->abort_flag = 1;
      }
    }
    __syncthreads();
    if (sm->abort_flag == 1) break;
    {
      for (int i = tid; i < (NR >> 1) * M; i += MOE_WG) {
        const int np = i / M, m = i - np * M;
        const int nl = 2 * np, n = n0 + nl;
        // routed sum in fp32, scaled once, then the shared expert
        float q0, q1;
        if (K <= 8)
          routed_sum<8>(sm, ysr, K, m, NR, nl, q0, q1);
        else
          routed_sum<MOE_MAX_TOPK>(sm, ysr, K, m, NR, nl, q0, q1);
        const float a0 = (S ? ysh[m * p.nr_max + nl] : 0.0f) + p.scale * q0;
        const float a1 = (S ? ysh[m * p.nr_max + nl + 1] : 0.0f) + p.scale * q1;
        if (p.flags & F_RESIDUAL) {
          const float h0 = bf_to_f(sm->hres[m * p.nr_max + nl]);
          const float h1 = bf_to_f(sm->hres[m * p.nr_max + nl + 1]);
          const uint32_t word = pk_bf(h0 + a0, h1 + a1);
          if (last) {
            reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = word;
          } else {
            uint64_t* r = p.res_buf + (size_t)(l + 1) * kCopies * M * H2 + ((m * H + n) >> 1);
#pragma unroll
            for (int c = 0; c < kCopies; ++c) st_tag(r + (size_t)c * M * H2, word, tag);
          }
          if (p.h_all)
            reinterpret_cast<uint32_t*>(p.h_all)[((size_t)(l + 1) * M * H + (size_t)m * H + n) >> 1] =
                word;
        } else if (p.flags & F_OUT_F32) {
          reinterpret_cast<float2*>(p.out)[(m * H + n) >> 1] = make_float2(a0, a1);
        } else {
          reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = pk_bf(a0, a1);
        }
      }
    }
    __syncthreads();
    MOE_STAMP(8);
    if (sm->abort_flag == 1) break;
  } while (NL > 1 && ++l < L);

  // ---------------- end of call
  __syncthreads();
  sbase = 0;
  MOE_STAMP(31);
#undef MOE_STAMP
}

}  // namespace moe
