// C-ABI boundary of libmoedecode (declared in include/moe_decode.h).
//
// Every argument check runs on the host before anything is enqueued and
// touches no device, so a rejected call has no side effect.  A specialised
// path states its coverage and fails early outside it, leaving the caller free
// to use a general path (SGLang Low-Latency Mode, Plugin System: guard;
// Ling-3.0-flash on 4 Blackwell GPUs, Two fusions and a retune: the pair-axis
// kernel's hard size gate with fallback).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/moe_decode.h"
#include "moe_layer.hpp"
#include "moe_lmhead.hpp"
#include "moe_prefetch.hpp"

using namespace moe;

static_assert(MOE_MAX_LAYERS == 64, "layer table size must match the header");
// kernel arguments of the chain kernel (one weight slot per layer) stay within 4 KiB
static_assert(sizeof(ParamsT<MOE_MAX_LAYERS>) <= 4096, "kernel argument block too large");

namespace {

constexpr size_t kHdrBytes = (size_t)HDR_BYTES;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct DevInfo {
  int num_cu = 0;
  int max_lds = 0;
  bool ok = false;
};

std::mutex g_mu;
DevInfo g_dev[64];

int device_info(DevInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_E_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  if (!d.ok) {
    if (hipDeviceGetAttribute(&d.num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_E_HIP;
    if (hipDeviceGetAttribute(&d.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
        hipSuccess)
      return MOE_E_HIP;
    d.ok = true;
  }
  *out = d;
  return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Per-workspace host state: the layer kernel's calls on a workspace are
// counted here, and the count is the step tag of the next call (a launch
// argument), so the kernel reads no control word before its first weight loads
// and needs no end-of-call counting to advance the step.  Tags only grow (zero
// is skipped), so no call can take a stale word of an earlier call on the same
// workspace for its own.  moe_workspace_init resets the state with the memory;
// moe_workspace_debug sets the flags and the deadline.
struct WsState {
  uint32_t epoch = 0;
  uint32_t flags = 0;
  uint32_t deadline = 0;  // 100 MHz ticks, 0 = default
};
std::mutex g_ws_mu;
std::unordered_map<const void*, WsState> g_ws;

struct CallTag {
  uint32_t tag, flags, deadline;
};

CallTag next_call(const void* ws) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsState& st = g_ws[ws];
  if (++st.epoch == 0) st.epoch = 1;
  return CallTag{st.epoch, st.flags, st.deadline ? st.deadline : kDefaultDeadlineTicks};
}

uint32_t ws_flags(const void* ws) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_ws.find(ws);
  return it == g_ws.end() ? 0u : it->second.flags;
}

// A launch that failed ran no kernel: its tag is given back, so that the tags
// of the calls that did run stay consecutive (each call clears the input-read
// counter of the other tag parity for the next one).
void undo_call(const void* ws, uint32_t tag) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsState& st = g_ws[ws];
  if (st.epoch == tag) st.epoch = tag - 1;
}

// Chunk plan of a row of `len` bf16 values split over `lpr` lanes, `cpl`
// 16-byte loads per lane.
struct RowPlan {
  int lpr, cpl;
};

bool plan_h_rows(int H, RowPlan* rp) {
  if (H % 256) return false;
  rp->lpr = 32;
  rp->cpl = H / 256;
  return true;
}

// Down-projection rows are split over 8 lanes each (I/64 loads per lane);
// several 8-row blocks go in flight together when rows are short.
bool plan_i_rows(int I, RowPlan* rp) {
  if (I % 64) return false;
  rp->lpr = 8;
  rp->cpl = I / 64;
  return true;
}

int down_blocks(int cpli) {
  const int b = 10 / cpli;
  return b < 1 ? 1 : (b > 4 ? 4 : b);
}

// Launch of the persistent layer kernel.  Its workgroups wait on each
// other's tagged words, so all of them must be resident at once.  The default
// is a plain launch behind an occupancy check (one workgroup fits a CU with
// its registers and LDS), which holds while no other kernel shares the device
// during the call; every wait also has a deadline, so a grid that is not
// wholly resident ends with MOE_E_TIMEOUT instead of hanging.  Built with
// MOE_COOP_LAUNCH=1 the kernel goes through hipLaunchCooperativeKernel, which
// guarantees co-residency or fails the launch, at a measured cost of about
// 18 us per launch on MI355X (a single Ling layer takes 30 us).
#ifndef MOE_COOP_LAUNCH
#define MOE_COOP_LAUNCH 0
#endif

// Compiled (CPLH, CPLI) variants of the layer kernel: hidden size 256 * CPLH,
// intermediate size 64 * CPLI; NL layer weight slots in the kernel arguments.
template <int NL>
using LayerKern = void (*)(ParamsT<NL>);

template <int NL>
LayerKern<NL> pick_layer_kernel(int cplh, int cpli, bool w8) {
#define MOE_K(a, b, f)                      \
  if (cplh == a && cpli == b && w8 == f)   \
    return moe_layer_kernel<a, b, (10 / b < 1 ? 1 : (10 / b > 4 ? 4 : 10 / b)), NL, f>;
  MOE_K(1, 1, false) MOE_K(10, 12, false) MOE_K(10, 3, false) MOE_K(10, 1, false)
  MOE_K(10, 4, false) MOE_K(8, 12, false) MOE_K(8, 3, false) MOE_K(4, 4, false)
  MOE_K(2, 2, false)
  // fp8 experts (I a multiple of 128)
  MOE_K(1, 2, true) MOE_K(10, 12, true) MOE_K(2, 2, true)
#undef MOE_K
  return nullptr;
}

// Per-process record of the kernels whose dynamic-LDS limit was raised and
// whose co-residency was checked, so repeated calls skip both runtime queries.
struct KernelReady {
  const void* fn;
  int lds;
  int device;
};
std::mutex g_ready_mu;
std::vector<KernelReady> g_ready;

// not_resident: the debug flag DBG_NOT_RESIDENT of the call's workspace; the
// occupancy answer is then taken as zero blocks (a test of the gate below)
int prepare_kernel(const void* fn, int lds, int block, bool not_resident = false) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
  if (!not_resident) {
    std::lock_guard<std::mutex> lk(g_ready_mu);
    for (const KernelReady& r : g_ready)
      if (r.fn == fn && r.lds >= lds && r.device == dev) return MOE_OK;
  }
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return MOE_E_HIP;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block, lds) != hipSuccess)
    return MOE_E_HIP;
  if (not_resident) nb = 0;
  if (nb < 1) return MOE_E_UNSUPPORTED;  // the persistent grid would not be co-resident
  std::lock_guard<std::mutex> lk(g_ready_mu);
  g_ready.push_back(KernelReady{fn, lds, dev});
  return MOE_OK;
}

typedef void (*LmKern)(LmParams);
template <int MM>
LmKern pick_lm_kernel_mm(int cplh) {
  switch (cplh) {
    case 1: return moe_lmhead_kernel<1, MM>;
    case 2: return moe_lmhead_kernel<2, MM>;
    case 4: return moe_lmhead_kernel<4, MM>;
    case 8: return moe_lmhead_kernel<8, MM>;
    case 10: return moe_lmhead_kernel<10, MM>;
    default: return nullptr;
  }
}
LmKern pick_lm_kernel(int cplh, int M) { return M <= 8 ? pick_lm_kernel_mm<8>(cplh) : nullptr; }
// The matrix-core lm_head from this many token rows on (H a multiple of 256).
// Its time hardly depends on the row count (V = 157184, H = 2560: 122-127 us
// from 2 to 8 rows, 134 us at 16), while the dot products grow with it
// (119 us at one row, 122 at two, 125 at three, 141 at six, 167 at eight).
#ifndef MOE_LM_MFMA_ROWS
#define MOE_LM_MFMA_ROWS 3
#endif
LmKern pick_lm_mfma_kernel(int H) {
  const int sc = H >> 6;  // 64-element super-chunks per row
  if (sc % 8 == 0) return moe_lmhead_mfma_kernel<8>;
  if (sc % 4 == 0) return moe_lmhead_mfma_kernel<4>;
  return nullptr;
}

int check_dims(const moe_dims* d) {
  if (!d) return MOE_E_ARG;
  if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->inter <= 0) return MOE_E_ARG;
  if (d->n_shared != 0 && d->n_shared != 1) return MOE_E_ARG;
  if (d->top_k > d->n_experts) return MOE_E_ARG;
  if (d->n_experts > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK) return MOE_E_UNSUPPORTED;
  RowPlan a, b;
  if (!plan_h_rows(d->hidden, &a) || !plan_i_rows(d->inter, &b)) return MOE_E_UNSUPPORTED;
  if (d->hidden > 16384 || d->inter > 16384) return MOE_E_UNSUPPORTED;
  if (!isfinite(d->routed_scale)) return MOE_E_ARG;
  if (d->expert_format != MOE_EXPERT_BF16 && d->expert_format != MOE_EXPERT_FP8_B128)
    return MOE_E_ARG;
  if (d->expert_format == MOE_EXPERT_FP8_B128 && (d->hidden % 128 || d->inter % 128))
    return MOE_E_UNSUPPORTED;  // block-128 quantisation
  return MOE_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// fp8 experts need both block-scale tensors; bf16 experts take none.
int check_expert_scales(const moe_dims& d, const moe_layer_weights& w) {
  if (d.expert_format != MOE_EXPERT_FP8_B128) return (!w.s_gate_up && !w.s_down) ? MOE_OK : MOE_E_ARG;
  if (!w.s_gate_up || !w.s_down) return MOE_E_ARG;
  if (!aligned4(w.s_gate_up) || !aligned4(w.s_down)) return MOE_E_ALIGN;
  return MOE_OK;
}

// Workspace regions after the header (all tagged 64-bit words):
//   lg  [L][kCopies][M][E]    router logits
//   hs  [L][kCopies][M][I/2]  shared expert SwiGLU output (bf16 pairs)
//   hr  [L][M*K][I/2]    routed (expert, row) SwiGLU outputs (bf16 pairs)
//   y   [L][M*K][H]      routed (expert, row) down-projection outputs (fp32)
//   res [L+1][kCopies][M][H/2] residual stream between chained layers (bf16 pairs)
// (the words every workgroup reads are kept in one copy per XCD)
struct WsLayout {
  size_t lg, hs, hr, y, res, total;
};

WsLayout ws_layout(const moe_dims& d, int M, int L) {
  WsLayout w;
  const size_t E = (size_t)d.n_experts, H = (size_t)d.hidden, I = (size_t)d.inter;
  const size_t MK = (size_t)M * d.top_k;
  w.lg = kHdrBytes;
  const size_t C = (size_t)kCopies;
  w.hs = align_up(w.lg + (size_t)L * C * M * E * 8, 256);
  w.hr = align_up(w.hs + (size_t)L * C * M * (I / 2) * 8, 256);
  w.y = align_up(w.hr + (size_t)L * MK * (I / 2) * 8, 256);
  w.res = align_up(w.y + (size_t)L * MK * H * 8, 256);
  w.total = align_up(w.res + (size_t)(L + 1) * C * M * (H / 2) * 8, 256);
  return w;
}

struct LdsPlan {
  int xs, lg, hs, ysh, ysr, small, gn, p1w, total, nr_max, fold;
};

// LDS of the layer kernel: x [M][H] bf16, aliased by the SwiGLU rows of the
// shared expert and of up to two (four, folded) routed slice pieces
// [3 or 5][M][I] bf16 once the routed gate/up rows are done; logits [M][E] fp32; the shared expert's
// outputs for the owned rows [M][nr_max] fp32; the routed (expert, row)
// outputs of the owned rows [M*K][nr_max] fp32; the small tables; the
// norm's gain [H] bf16; and, where they fit, the P1 rows of waves 0-2 (two
// token rows on).
int plan_lds(const moe_dims& d, int M, int G, int max_lds, LdsPlan* lp) {
  const int H = d.hidden, E = d.n_experts, I = d.inter;
  lp->nr_max = 2 * (((H / 2) + G - 1) / G);
  if (lp->nr_max > 64) return MOE_E_UNSUPPORTED;  // residual rows kept in LDS
  // x (read until the routed gate/up rows are done) and the SwiGLU rows of the
  // down tasks (shared | pieces, written after) share a region: three segments,
  // or five with the down slices folded (four pieces), which is chosen where
  // it fits
  size_t o = 0;
  lp->xs = (int)o;
  lp->hs = (int)o;
  auto rest = [&](int segs) {
    const size_t xh = std::max((size_t)M * H * 2, (size_t)segs * M * I * 2);
    size_t q = align_up(xh, 16);
    q = align_up(q + (size_t)M * E * 4, 16);
    q = align_up(q + (size_t)M * lp->nr_max * 4, 16);
    q = align_up(q + (size_t)M * d.top_k * lp->nr_max * 4, 16);
    q = align_up(q + sizeof(Small), 16);
    q = align_up(q + (size_t)H * 2, 16);
    return q;
  };
  lp->fold = rest(5) <= (size_t)max_lds ? 1 : 0;
  const size_t xh = std::max((size_t)M * H * 2, (size_t)(lp->fold ? 5 : 3) * M * I * 2);
  o = align_up(o + xh, 16);
  lp->lg = (int)o;
  o = align_up(o + (size_t)M * E * 4, 16);
  lp->ysh = (int)o;
  o = align_up(o + (size_t)M * lp->nr_max * 4, 16);
  lp->ysr = (int)o;
  o = align_up(o + (size_t)M * d.top_k * lp->nr_max * 4, 16);
  lp->small = (int)o;
  o = align_up(o + sizeof(Small), 16);
  lp->gn = (int)o;  // the norm's gain
  o = align_up(o + (size_t)H * 2, 16);
  // the router / shared-expert rows of waves 0-2 (two units of H bf16 per
  // half-wave row each), where they fit (-1: none): from two token rows on
  // for P1, and at one token row for the shared items of the layer loop
  lp->p1w = -1;
  {
    // 3 slots: two units of 2H bf16 (a bf16 row pair per half-wave); fp8
    // shared items use less plus their scales after the units
    const size_t w = (size_t)3 * (2 * H * 2 * 2 + 64 * 4 * ((H / 256 + 1) / 2));
    if (o + w <= (size_t)max_lds) {
      lp->p1w = (int)o;
      o += w;
    }
  }
  lp->total = (int)o;
  return o <= (size_t)max_lds ? MOE_OK : MOE_E_UNSUPPORTED;
}

template <int NL>
int launch_layer_nl(const moe_dims& d, int M, int L, uint32_t flags,
                    const moe_layer_weights* layers, const uint16_t* x, void* out,
                    const int32_t* tk_in, const float* tkg_in, int32_t* tk_out, float* tkg_out,
                    float* logits_out, uint16_t* h_all, void* ws, hipStream_t st) {
  DevInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  RowPlan ph, pi;
  plan_h_rows(d.hidden, &ph);
  plan_i_rows(d.inter, &pi);
  LayerKern<NL> kern =
      pick_layer_kernel<NL>(ph.cpl, pi.cpl, d.expert_format == MOE_EXPERT_FP8_B128);
  if (!kern) return MOE_E_UNSUPPORTED;
  const int G = di.num_cu;
  LdsPlan lp;
  rc = plan_lds(d, M, G, di.max_lds, &lp);
  if (rc) return rc;
  rc = prepare_kernel((const void*)kern, lp.total, MOE_WG,
                      (ws_flags(ws) & DBG_NOT_RESIDENT) != 0u);
  if (rc) return rc;

  const WsLayout wl = ws_layout(d, M, L);
  ParamsT<NL> p;
  memset(&p, 0, sizeof(p));
  p.H = d.hidden;
  p.E = d.n_experts;
  p.K = d.top_k;
  p.I = d.inter;
  p.S = d.n_shared;
  p.M = M;
  p.L = L;
  p.flags = flags;
  p.nr_max = lp.nr_max;
  p.scale = d.routed_scale == 0.0f ? 1.0f : d.routed_scale;
  const CallTag ct = next_call(ws);
  p.tag = ct.tag;
  p.dbg = ct.flags;
  p.budget = ct.deadline;
  p.lds_xs = lp.xs;
  p.lds_lg = lp.lg;
  p.lds_hs = lp.hs;
  p.lds_ysh = lp.ysh;
  p.lds_ysr = lp.ysr;
  p.lds_small = lp.small;
  p.lds_gn = lp.gn;
  p.fold = lp.fold;
  p.lds_p1w = lp.p1w;
  p.x_in = x;
  p.out = out;
  p.tk_idx_in = tk_in;
  p.tk_gate_in = tkg_in;
  p.tk_idx_out = tk_out;
  p.tk_gate_out = tkg_out;
  p.logits_out = logits_out;
  p.h_all = h_all;
  unsigned char* base = (unsigned char*)ws;
  p.hdr = (uint32_t*)base;
  p.lg_buf = (uint64_t*)(base + wl.lg);
  p.hs_buf = (uint64_t*)(base + wl.hs);
  p.hr_buf = (uint64_t*)(base + wl.hr);
  p.y_buf = (uint64_t*)(base + wl.y);
  p.res_buf = (uint64_t*)(base + wl.res);
  for (int l = 0; l < L; ++l) {
    p.lw[l].wr = layers[l].w_router;
    p.lw[l].wgu = layers[l].w_gate_up;
    p.lw[l].wd = layers[l].w_down;
    p.lw[l].bias = layers[l].router_bias;
    p.lw[l].gain = (flags & F_PRENORM) ? layers[l].norm_gain : nullptr;
    p.lw[l].sgu = layers[l].s_gate_up;
    p.lw[l].sd = layers[l].s_down;
  }
  // The workgroups wait on each other's tagged words, so all of them must be
  // resident at once: a cooperative launch guarantees that or fails (then
  // nothing runs and MOE_E_UNSUPPORTED is returned).
#if MOE_COOP_LAUNCH
  void* args[] = {&p};
  const hipError_t le = hipLaunchCooperativeKernel((const void*)kern, dim3(G), dim3(MOE_WG), args,
                                                   (unsigned)lp.total, st);
#else
  hipLaunchKernelGGL(kern, dim3(G), dim3(MOE_WG), lp.total, st, p);
  const hipError_t le = hipGetLastError();
#endif
  if (le != hipSuccess) {
    (void)hipGetLastError();  // clear the launch error
    undo_call(ws, p.tag);
    return le == hipErrorCooperativeLaunchTooLarge ? MOE_E_UNSUPPORTED : MOE_E_HIP;
  }
  return MOE_OK;
}

// Single-layer calls carry one weight slot in their (smaller, faster to
// launch) argument block; chains carry MOE_MAX_LAYERS.
int launch_layer(const moe_dims& d, int M, int L, uint32_t flags, const moe_layer_weights* layers,
                 const uint16_t* x, void* out, const int32_t* tk_in, const float* tkg_in,
                 int32_t* tk_out, float* tkg_out, float* logits_out, uint16_t* h_all, void* ws,
                 hipStream_t st) {
  if (L == 1)
    return launch_layer_nl<1>(d, M, L, flags, layers, x, out, tk_in, tkg_in, tk_out, tkg_out,
                              logits_out, h_all, ws, st);
  return launch_layer_nl<MOE_MAX_LAYERS>(d, M, L, flags, layers, x, out, tk_in, tkg_in, tk_out,
                                         tkg_out, logits_out, h_all, ws, st);
}

int check_ws(const moe_dims* d, int M, int L, void* ws, size_t ws_bytes) {
  if (!ws) return MOE_E_WORKSPACE;
  if (!aligned16(ws)) return MOE_E_ALIGN;
  const WsLayout wl = ws_layout(*d, M, L);
  return ws_bytes >= wl.total ? MOE_OK : MOE_E_WORKSPACE;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported shape or option";
    case MOE_E_ALIGN: return "pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_HIP: return "HIP runtime error";
    case MOE_E_TIMEOUT: return "device wait passed its deadline";
    case MOE_E_INDEX: return "expert index out of range";
    default: return "unknown status";
  }
}

int moe_workspace_size(const moe_dims* dims, int32_t max_rows, int32_t n_layers, size_t* bytes) {
  if (!bytes) return MOE_E_ARG;
  int rc = check_dims(dims);
  if (rc) return rc;
  if (max_rows < 1 || n_layers < 1) return MOE_E_ARG;
  if (max_rows > MOE_MAX_ROWS || n_layers > MOE_MAX_LAYERS) return MOE_E_UNSUPPORTED;
  *bytes = ws_layout(*dims, max_rows, n_layers).total;
  return MOE_OK;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_E_WORKSPACE;
  if (!aligned16(ws)) return MOE_E_ALIGN;
  if (ws_bytes < kHdrBytes) return MOE_E_WORKSPACE;
  if (hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream) != hipSuccess) return MOE_E_HIP;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  g_ws[ws] = WsState{};
  return MOE_OK;
}

int moe_router_topk(const moe_dims* dims, int32_t M, const uint16_t* x, const uint16_t* w_router,
                    const float* router_bias, int32_t* topk_idx, float* topk_gate, float* logits,
                    void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1) return MOE_E_ARG;
  if (M > MOE_MAX_ROWS) return MOE_E_UNSUPPORTED;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_E_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_E_ALIGN;
  if (!aligned4(router_bias) || !aligned4(topk_idx) || !aligned4(topk_gate) || !aligned4(logits))
    return MOE_E_ALIGN;
  rc = check_ws(dims, M, 1, ws, ws_bytes);
  if (rc) return rc;
  moe_layer_weights lw = {w_router, nullptr, nullptr, router_bias, nullptr, nullptr, nullptr};
  return launch_layer(*dims, M, 1, F_ROUTER_ONLY, &lw, x, nullptr, nullptr, nullptr, topk_idx,
                      topk_gate, logits, nullptr, ws, (hipStream_t)stream);
}

int moe_experts_fused(const moe_dims* dims, int32_t M, const uint16_t* x, const int32_t* topk_idx,
                      const float* topk_gate, const moe_layer_weights* w, void* out,
                      int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1) return MOE_E_ARG;
  if (M > MOE_MAX_ROWS) return MOE_E_UNSUPPORTED;
  if (!x || !topk_idx || !topk_gate || !w || !out || !w->w_gate_up || !w->w_down) return MOE_E_ARG;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_E_ARG;
  if (!aligned16(x) || !aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned16(out))
    return MOE_E_ALIGN;
  if (((uintptr_t)topk_idx & 3u) || ((uintptr_t)topk_gate & 3u)) return MOE_E_ALIGN;
  rc = check_expert_scales(*dims, *w);
  if (rc) return rc;
  rc = check_ws(dims, M, 1, ws, ws_bytes);
  if (rc) return rc;
  const size_t osz = (size_t)M * dims->hidden * (out_dtype == MOE_OUT_F32 ? 4 : 2);
  uint32_t flags = F_TOPK_IN | (out_dtype == MOE_OUT_F32 ? F_OUT_F32 : 0u);
  if (overlaps(out, osz, x, (size_t)M * dims->hidden * 2)) flags |= F_ALIAS;
  moe_layer_weights lw = {nullptr, w->w_gate_up, w->w_down, nullptr, nullptr, w->s_gate_up,
                          w->s_down};
  return launch_layer(*dims, M, 1, flags, &lw, x, out, topk_idx, topk_gate, nullptr, nullptr,
                      nullptr, nullptr, ws, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// moe_layer_chain's argument checks (all but the workspace): MOE_OK, or the
// error to return with nothing enqueued; *flags receives the kernel's mode flags.
int check_chain(const moe_dims* dims, int32_t M, int32_t n_layers,
                const moe_layer_weights* layers, const uint16_t* x_in, void* out,
                int32_t out_dtype, int32_t mode, int32_t* topk_idx_all, uint16_t* h_all,
                uint32_t* flags_out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1 || n_layers < 1) return MOE_E_ARG;
  if (M > MOE_MAX_ROWS || n_layers > MOE_MAX_LAYERS) return MOE_E_UNSUPPORTED;
  if (!layers || !x_in || !out) return MOE_E_ARG;
  if (mode != MOE_CHAIN_RESIDUAL && mode != MOE_CHAIN_LAYER_ONLY &&
      mode != MOE_CHAIN_PRENORM_RESIDUAL && mode != MOE_CHAIN_PRENORM_LAYER_ONLY)
    return MOE_E_ARG;
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return MOE_E_ARG;
  const bool layer_only = mode == MOE_CHAIN_LAYER_ONLY || mode == MOE_CHAIN_PRENORM_LAYER_ONLY;
  const bool prenorm = mode == MOE_CHAIN_PRENORM_RESIDUAL || mode == MOE_CHAIN_PRENORM_LAYER_ONLY;
  if (layer_only && n_layers != 1) return MOE_E_UNSUPPORTED;
  if (!layer_only && out_dtype != MOE_OUT_BF16) return MOE_E_UNSUPPORTED;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights& w = layers[l];
    if (!w.w_router || !w.w_gate_up || !w.w_down) return MOE_E_ARG;
    if (!aligned16(w.w_router) || !aligned16(w.w_gate_up) || !aligned16(w.w_down))
      return MOE_E_ALIGN;
    if (!aligned4(w.router_bias) || (prenorm && !aligned16(w.norm_gain))) return MOE_E_ALIGN;
    rc = check_expert_scales(*dims, w);
    if (rc) return rc;
  }
  if (!aligned16(x_in) || !aligned16(out)) return MOE_E_ALIGN;
  if (topk_idx_all && ((uintptr_t)topk_idx_all & 3u)) return MOE_E_ALIGN;
  if (h_all && layer_only) return MOE_E_ARG;
  if (h_all && !aligned16(h_all)) return MOE_E_ALIGN;
  if (h_all && (overlaps(h_all, (size_t)(n_layers + 1) * M * dims->hidden * 2, x_in,
                         (size_t)M * dims->hidden * 2)))
    return MOE_E_ARG;
  uint32_t flags = 0;
  if (mode == MOE_CHAIN_RESIDUAL) flags |= F_RESIDUAL;
  if (mode == MOE_CHAIN_PRENORM_RESIDUAL) flags |= F_RESIDUAL | F_PRENORM;
  if (mode == MOE_CHAIN_PRENORM_LAYER_ONLY) flags |= F_PRENORM;
  if (out_dtype == MOE_OUT_F32) flags |= F_OUT_F32;
  const size_t osz = (size_t)M * dims->hidden * (out_dtype == MOE_OUT_F32 ? 4 : 2);
  if (overlaps(out, osz, x_in, (size_t)M * dims->hidden * 2)) flags |= F_ALIAS;
  *flags_out = flags;
  return MOE_OK;
}

// ---- the library's own workspace, for moe_layer_chain_noalloc
//
// A static device array, one per GPU (each GPU that runs the call holds its
// own copy until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

struct ScratchDev {
  void* ptr = nullptr;
  bool ready = false;
};
ScratchDev g_scratch[64];

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address.  On the first call on a device it is
// looked up and the whole array is cleared once, by a fill kernel on `stream`
// (a kernel, not a memset: a caller may be capturing that stream), and the
// host's step count for it starts at zero; later calls only read the address.
int scratch_for_device(void** out, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_E_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  ScratchDev& sd = g_scratch[dev];
  if (!sd.ready) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_E_HIP;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, stream, (uint4*)ptr,
                       (size_t)MOE_NOALLOC_SCRATCH_BYTES / 16);
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    {
      std::lock_guard<std::mutex> lk2(g_ws_mu);
      g_ws[ptr] = WsState{};
    }
    sd.ptr = ptr;
    sd.ready = true;
  }
  *out = sd.ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_chain(const moe_dims* dims, int32_t M, int32_t n_layers,
                    const moe_layer_weights* layers, const uint16_t* x_in, void* out,
                    int32_t out_dtype, int32_t mode, int32_t* topk_idx_all, uint16_t* h_all,
                    void* ws, size_t ws_bytes, void* stream) {
  uint32_t flags = 0;
  int rc = check_chain(dims, M, n_layers, layers, x_in, out, out_dtype, mode, topk_idx_all, h_all,
                       &flags);
  if (rc) return rc;
  rc = check_ws(dims, M, n_layers, ws, ws_bytes);
  if (rc) return rc;
  return launch_layer(*dims, M, n_layers, flags, layers, x_in, out, nullptr, nullptr, topk_idx_all,
                      nullptr, nullptr, h_all, ws, (hipStream_t)stream);
}

int moe_layer_chain_noalloc(const moe_dims* dims, int32_t M, int32_t n_layers,
                            const moe_layer_weights* layers, const uint16_t* x_in, void* out,
                            int32_t out_dtype, int32_t mode, int32_t* topk_idx_all,
                            uint16_t* h_all, void* stream) {
  uint32_t flags = 0;
  int rc = check_chain(dims, M, n_layers, layers, x_in, out, out_dtype, mode, topk_idx_all, h_all,
                       &flags);
  if (rc) return rc;
  // the call's workspace must fit the static one (checked before any HIP call)
  if (ws_layout(*dims, M, n_layers).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_E_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_for_device(&ws, (hipStream_t)stream);
  if (rc) return rc;
  return launch_layer(*dims, M, n_layers, flags, layers, x_in, out, nullptr, nullptr, topk_idx_all,
                      nullptr, nullptr, h_all, ws, (hipStream_t)stream);
}

int lmhead_argmax(int32_t M, int32_t H, int32_t V, const uint16_t* h, const uint16_t* w_lm,
                  int32_t* token, float* max_logit, void* ws, size_t ws_bytes, void* stream) {
  if (M < 1 || H < 1 || V < 1) return MOE_E_ARG;
  if (M > MOE_MAX_ROWS) return MOE_E_UNSUPPORTED;
  if (!h || !w_lm || !token) return MOE_E_ARG;
  if (!ws) return MOE_E_WORKSPACE;
  if (ws_bytes < kHdrBytes) return MOE_E_WORKSPACE;
  if (!aligned16(h) || !aligned16(w_lm) || !aligned16(ws)) return MOE_E_ALIGN;
  if (((uintptr_t)token & 3u) || (max_logit && ((uintptr_t)max_logit & 3u))) return MOE_E_ALIGN;
  RowPlan ph;
  if (!plan_h_rows(H, &ph)) return MOE_E_UNSUPPORTED;
  const bool mfma = M >= MOE_LM_MFMA_ROWS;
  LmKern kern = mfma ? pick_lm_mfma_kernel(H) : pick_lm_kernel(ph.cpl, M);
  if (!kern) return MOE_E_UNSUPPORTED;
  DevInfo di;
  int rc = device_info(&di);
  if (rc) return rc;
  // x in LDS (the matrix-core kernel pads each row by 8 elements), then the
  // per-wave bests and the last-workgroup flag
  const size_t xrow = (size_t)H * 2 + (mfma ? 16 : 0);
  const int lds = (int)align_up((size_t)M * xrow, 16) + MOE_LM_WAVES * MOE_MAXM * 8 + 16;
  if (lds > di.max_lds) return MOE_E_UNSUPPORTED;
  rc = prepare_kernel((const void*)kern, lds, MOE_LM_WG);
  if (rc) return rc;
  LmParams p;
  p.M = M;
  p.H = H;
  p.V = V;
  p.h = h;
  p.w = w_lm;
  p.token = token;
  p.max_logit = max_logit;
  p.hdr = (uint32_t*)ws;
  // The dot-product kernel: two workgroups per CU (they run in two rounds, one
  // fits a CU at a time), fewer for a small vocabulary: at least one row pair
  // per wave.  No workgroup waits on another until the last one collects the
  // slots, so they need not be co-resident.
  int G;
  if (mfma) {
    // one workgroup per CU (its waves hold two batches of 16 rows in flight),
    // at least one 16-row tile per wave
    const long long tiles = ((long long)V + 15) / 16;
    G = di.num_cu < MOE_LM_MAX_GRID ? di.num_cu : MOE_LM_MAX_GRID;
    if ((long long)G * MOE_LM_WAVES > tiles) G = (int)((tiles + MOE_LM_WAVES - 1) / MOE_LM_WAVES);
  } else {
    const long long pairs = ((long long)V + 1) / 2;
    G = 2 * di.num_cu < MOE_LM_MAX_GRID ? 2 * di.num_cu : MOE_LM_MAX_GRID;
    if ((long long)G * MOE_LM_WAVES > pairs) G = (int)((pairs + MOE_LM_WAVES - 1) / MOE_LM_WAVES);
  }
  if (G < 1) G = 1;
  hipLaunchKernelGGL(kern, dim3(G), dim3(MOE_LM_WG), lds, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_expert_prefetch(const moe_dims* dims, const moe_layer_weights* w,
                        const int32_t* expert_ids, int32_t n, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!w || !w->w_gate_up || !w->w_down || n < 0) return MOE_E_ARG;
  if (n > MOE_MAX_PREFETCH_IDS) return MOE_E_UNSUPPORTED;
  if (n > 0 && !expert_ids) return MOE_E_ARG;
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned4(expert_ids))
    return MOE_E_ALIGN;
  rc = check_expert_scales(*dims, *w);
  if (rc) return rc;
  if (n == 0) return MOE_OK;
  const moe_dims& d = *dims;
  const bool fp8 = d.expert_format == MOE_EXPERT_FP8_B128;
  const uint64_t H = (uint64_t)d.hidden, I = (uint64_t)d.inter, wb = fp8 ? 1 : 2;
  PrefetchParams p;
  p.wgu = (const uint8_t*)w->w_gate_up;
  p.wd = (const uint8_t*)w->w_down;
  p.sgu = (const uint8_t*)w->s_gate_up;
  p.sd = (const uint8_t*)w->s_down;
  p.gu_bytes = 2 * I * H * wb;
  p.d_bytes = H * I * wb;
  p.sgu_bytes = fp8 ? (2 * I / 128) * (H / 128) * 4 : 0;
  p.sd_bytes = fp8 ? (H / 128) * (I / 128) * 4 : 0;
  // H is a multiple of 256 (check_dims), so every row block is whole 16-byte chunks
  const uint64_t units = p.gu_bytes / 16 + p.d_bytes / 16 + p.sgu_bytes / 4 + p.sd_bytes / 4;
  if (units >= (1ull << 31)) return MOE_E_UNSUPPORTED;
  p.u_gu = (uint32_t)(p.gu_bytes / 16);
  p.u_d = (uint32_t)(p.d_bytes / 16);
  p.u_sgu = (uint32_t)(p.sgu_bytes / 4);
  p.u_sd = (uint32_t)(p.sd_bytes / 4);
  p.ids = expert_ids;
  p.n_valid = d.n_experts + d.n_shared;
  const uint64_t per_block = (uint64_t)kPrefetchWG * kPrefetchBatch;
  uint64_t gx = (p.u_gu + p.u_d + per_block - 1) / per_block;
  if (gx > 4096) gx = 4096;
  hipLaunchKernelGGL(moe_prefetch_kernel, dim3((unsigned)gx, (unsigned)n), dim3(kPrefetchWG), 0,
                     (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_last_device_status(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_E_WORKSPACE;
  if (ws_bytes < kHdrBytes) return MOE_E_WORKSPACE;
  if (!aligned16(ws)) return MOE_E_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_E_HIP;
  uint32_t v = 0;
  uint32_t* sp = (uint32_t*)ws + HDR_STATUS;
  if (hipMemcpy(&v, sp, 4, hipMemcpyDeviceToHost) != hipSuccess) return MOE_E_HIP;
  const uint32_t zero = 0;
  if (hipMemcpy(sp, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return MOE_E_HIP;
  return (int)(int32_t)v;
}

int moe_workspace_debug(void* ws, size_t ws_bytes, uint32_t flags, uint32_t deadline_us,
                        void* stream) {
  if (!ws) return MOE_E_WORKSPACE;
  if (ws_bytes < kHdrBytes) return MOE_E_WORKSPACE;
  if (!aligned16(ws)) return MOE_E_ALIGN;
  if (deadline_us > 40000000u) return MOE_E_ARG;  // 100 MHz ticks must fit 32 bits
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_E_HIP;
  const uint32_t vals[2] = {flags, deadline_us * 100u};
  // the lm_head reads its deadline from the workspace; the layer kernel takes
  // both with its launch
  if (hipMemcpy((uint32_t*)ws + HDR_FLAGS, vals, 8, hipMemcpyHostToDevice) != hipSuccess)
    return MOE_E_HIP;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsState& state = g_ws[ws];
  state.flags = flags;
  state.deadline = deadline_us * 100u;
  return MOE_OK;
}

}  // extern "C"
