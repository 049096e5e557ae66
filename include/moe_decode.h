/* libmoedecode: the small-M mixture-of-experts decoder step on one AMD Instinct
 * MI355X (gfx950).
 *
 * The step, for M = 1..16 token rows (batch-1 decode, speculative verify of up
 * to 8 draft tokens, and a 16-token tree verify):
 * a bf16 router GEMV, softmax top-k with renormalised gates, a gather of the
 * selected experts' weights, fused gate/up GEMV with SwiGLU, the down GEMV,
 * a gate-weighted combine plus the always-on shared expert, and optionally a
 * bf16 lm_head GEMV with greedy argmax.
 *
 * Sources (page titles and sections):
 *  [LING]  "Ling-3.0-flash on 4 Blackwell GPUs" (LMSYS blog), sections
 *          "The model", "PDL: stacking the latency floors of small kernels",
 *          "Two fusions and a retune", "bf16 router gate and lm_head".
 *  [LLM]   "SGLang Low-Latency Mode: Kernels and Runtime", sections
 *          "Low-Latency-Specific Optimizations" (item 3: at most eight rows,
 *          bitmap placement) and "AMD Low-Latency Kernels" (step-tagged values,
 *          a deadline on every wait, routing-independent weights loaded early).
 *  [MUSE]  "Muse Spark Open Ultrafast: Pushing beyond 1,000 Tokens per second",
 *          sections "Speculative decoding" (the target verifies 16 tokens per step)
 *          and "Megakernel internals" (prefetching weights into the caches;
 *          speculative expert prefetching).
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous; bf16 travels as uint16_t bit patterns.  Weight and activation
 *    pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on it: they never synchronise, never allocate
 *    device memory and never print.
 *  - All argument checks run on the host before anything is enqueued and need
 *    no device; a call that returns an error has enqueued nothing.
 *  - The workspace `ws` is caller-allocated device memory of at least
 *    moe_workspace_size() bytes, zeroed once by moe_workspace_init().  It holds
 *    step tags, counters and the values passed between workgroups; one
 *    workspace serves one stream at a time.  Calls on one workspace that
 *    overlap in time race.
 *  - Device-side failures (an out-of-range expert index in caller-provided
 *    top-k input, a wait that missed its deadline) are recorded as a sticky
 *    status in the workspace; read it with moe_last_device_status().
 *  - The layer calls (moe_router_topk, moe_experts_fused, moe_layer_chain,
 *    moe_layer_chain_noalloc) launch one workgroup per compute unit, and those
 *    workgroups wait on each other, so the whole grid must be resident at
 *    once.  No other kernel may run on the device while a layer call runs
 *    (work on other streams must be ordered before or after it, e.g. by
 *    events).  A grid that cannot become wholly resident does not hang: every
 *    wait has a deadline, and the call then records MOE_E_TIMEOUT.  A call
 *    whose grid cannot fit at all (occupancy check) returns MOE_E_UNSUPPORTED.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape: H hidden size, E routed experts, K experts per row, I expert
 * intermediate size (of this call: a tensor-parallel shard passes its share),
 * S shared experts (0 or 1).  [LING] "The model": H=2560, E=512, K=8, I=768, S=1.
 * routed_scale: the routed scaling factor s of the combine,
 *   acc = y_shared + s * sum_k g_k y_k  (the routed part summed in fp32, scaled once:
 *   [LING] "PDL: stacking ...", small-M combine as an fp32 sum times a scale);
 *   must be finite; 0 (a zero-initialised struct) means 1.
 * expert_format: how every expert weight of the call is stored (MOE_EXPERT_BF16,
 *   or MOE_EXPERT_FP8_B128: fp8 e4m3 codes with one fp32 scale per 128 x 128
 *   block, the block quantisation of [LING] "Where the time goes now"; it needs
 *   H and I to be multiples of 128, so a TP4 shard of I = 768 is not
 *   representable, as that section notes).  The router is bf16 either way. */
typedef struct {
  int32_t hidden;
  int32_t n_experts;
  int32_t top_k;
  int32_t inter;
  int32_t n_shared;
  float routed_scale;
  int32_t expert_format;
} moe_dims;

enum { MOE_EXPERT_BF16 = 0, MOE_EXPERT_FP8_B128 = 1 };

/* One layer's weights (device pointers, bf16 bits unless stated):
 *   w_router    [E][H]
 *   w_gate_up   [E+S][2I][H]  rows [0, I) are the gate projection, rows [I, 2I) the up projection
 *   w_down      [E+S][H][I]
 *               (MOE_EXPERT_FP8_B128: one byte per weight, an OCP fp8 e4m3 code;
 *               the weight is its value times the scale of its 128 x 128 block)
 *   s_gate_up   MOE_EXPERT_FP8_B128 only: [E+S][2I/128][H/128] fp32 block scales of
 *               w_gate_up, 4-byte aligned (NULL for bf16)
 *   s_down      MOE_EXPERT_FP8_B128 only: [E+S][H/128][I/128] fp32 block scales of w_down
 *   router_bias [E] fp32, optional (NULL: none): a per-expert selection bias.  Experts
 *               are chosen by fp32(logit + bias); the gates still come from the
 *               unbiased logits.  [LING] "PDL: stacking ...", figure on the router
 *               path: the top-k kernel loads its bias before the logits are ready.
 *               4-byte aligned.  Ignored by moe_experts_fused (routing is given).
 *   norm_gain   [H] bf16, optional (NULL: unit gain): the gain of the RMSNorm in
 *               front of the router and the experts (the norm that opens the router
 *               chain in [LING] "PDL: stacking ...").  16-byte aligned.  Used by the
 *               PRENORM modes of moe_layer_chain only, ignored elsewhere.
 * The shared expert, if any, is stored at expert index E. */
typedef struct {
  const uint16_t* w_router;
  const void* w_gate_up;
  const void* w_down;
  const float* router_bias;
  const uint16_t* norm_gain;
  const float* s_gate_up;
  const float* s_down;
} moe_layer_weights;

enum moe_status {
  MOE_OK = 0,
  MOE_E_ARG = -1,          /* null pointer, bad size, bad mode */
  MOE_E_UNSUPPORTED = -2,  /* shape or option outside what the kernels cover; use a general path */
  MOE_E_ALIGN = -3,        /* a tensor pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = -4,    /* workspace missing or smaller than moe_workspace_size() */
  MOE_E_HIP = -5,          /* the HIP runtime reported an error (device query or launch) */
  MOE_E_TIMEOUT = -6,      /* device: a wait passed its deadline (sticky, in the workspace) */
  MOE_E_INDEX = -7         /* device: caller-provided expert index out of range (sticky) */
};

enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 };
enum {
  MOE_CHAIN_RESIDUAL = 0,
  MOE_CHAIN_LAYER_ONLY = 1,
  MOE_CHAIN_PRENORM_RESIDUAL = 2,
  MOE_CHAIN_PRENORM_LAYER_ONLY = 3
};

#define MOE_MAX_ROWS 16     /* [LLM] item 3 keeps at most eight rows per tile; the kernels take
                               up to sixteen, for a 16-token verify ([MUSE] "Speculative
                               decoding": one pass of the target over 16 tokens) */
#define MOE_MAX_LAYERS 64
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_PREFETCH_IDS 4096
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20) /* the static workspace of moe_layer_chain_noalloc */

/* Bytes of workspace needed for calls with up to `max_rows` rows and up to
 * `n_layers` chained layers (use n_layers = 1 for the single-layer calls).
 * Pure host computation.  Returns MOE_OK or MOE_E_ARG / MOE_E_UNSUPPORTED. */
int moe_workspace_size(const moe_dims* dims, int32_t max_rows, int32_t n_layers, size_t* bytes);

/* Zero the workspace (tags, counters, sticky status) on `stream`.  Call once
 * after allocation, before the first call that uses it. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Router: logits[m][e] = sum_h x[m][h] * w_router[e][h] (fp32 accumulation of
 * bf16 products), then per row the K largest selection scores
 * s[m][e] = fp32(logits[m][e] + router_bias[e]) (s = logits without a bias) in
 * descending order (equal scores: lower expert index first) and gates
 * g_k = p_k / sum_k' p_k' with p = softmax(logits[m]) -- the renormalised top-k
 * softmax of the unbiased logits.
 * [LING] "PDL: stacking the latency floors of small kernels" (router chain:
 * gate matvec then top-k; the top-k's bias) and "bf16 router gate and lm_head".
 *   x [M][H] bf16; router_bias [E] fp32 (optional, NULL: none; 4-byte aligned);
 *   topk_idx [M][K] int32 (out); topk_gate [M][K] fp32 (out);
 *   logits [M][E] fp32 (out, optional: NULL to skip; unbiased). */
int moe_router_topk(const moe_dims* dims, int32_t M, const uint16_t* x, const uint16_t* w_router,
                    const float* router_bias, int32_t* topk_idx, float* topk_gate, float* logits,
                    void* ws, size_t ws_bytes, void* stream);

/* Experts for given routing: for each row m and selected expert e = topk_idx[m][k]
 * (and the shared expert), a = W_gate[e] x_m, b = W_up[e] x_m (fp32; fp8 weights are
 * decoded and scaled per block, activations stay bf16),
 * h = bf16(silu(a) * b), y = W_down[e] h (fp32); then
 *   acc[m] = y_shared + sum_k topk_gate[m][k] * y_{topk_idx[m][k]}   (fp32)
 * (times dims->routed_scale on the routed sum, see moe_dims)
 * and out[m] = bf16(acc[m]) (MOE_OUT_BF16) or acc[m] unrounded (MOE_OUT_F32, the
 * partial sum of a tensor-parallel shard).  Every selected expert is streamed
 * from HBM once per call, whatever the number of rows that chose it.
 * [LING] "PDL: stacking ..." (MoE chain; fp32 combine, one final cast),
 * "Two fusions and a retune" (SwiGLU in the up-projection epilogue, silu in
 * float, one rounding), "The model" (top-8 plus one shared expert).
 *   x [M][H] bf16; topk_idx [M][K] int32; topk_gate [M][K] fp32 (device);
 *   w: host struct of device pointers; out [M][H] bf16 or fp32.
 * An index outside [0, E) is skipped and sets the sticky MOE_E_INDEX. */
int moe_experts_fused(const moe_dims* dims, int32_t M, const uint16_t* x, const int32_t* topk_idx,
                      const float* topk_gate, const moe_layer_weights* w, void* out,
                      int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* n_layers MoE layers in ONE persistent launch: per layer the router, top-k,
 * experts and combine above, with the layer-to-layer handoff done on the device
 * by step-tagged values instead of kernel launches ([LLM] "AMD Low-Latency
 * Kernels": tagged stage outputs, deadlines on waits).
 *   MOE_CHAIN_RESIDUAL:   h_0 = x_in, h_{l+1} = bf16(h_l + acc_l); out = h_L.
 *   MOE_CHAIN_LAYER_ONLY: n_layers must be 1; out = MoE(x_in) exactly as
 *                         moe_experts_fused would return it (bf16 or fp32).
 *   MOE_CHAIN_PRENORM_RESIDUAL: h_{l+1} = bf16(h_l + MoE_l(u_l)) with
 *                         u_l = bf16((h_l * r) * norm_gain_l) (fp32 products; unit gain
 *                         when layers[l].norm_gain is NULL),
 *                         r = fp32(1 / sqrt(mean(h_l^2) + 1e-6)), the mean of squares
 *                         summed in double (the RMSNorm that opens the router chain
 *                         in [LING] "PDL: stacking ..."); keeps every layer's input
 *                         at unit scale.  out = h_L.
 *   MOE_CHAIN_PRENORM_LAYER_ONLY: n_layers must be 1; out = MoE(u) with u the
 *                         normed input as above (router front, router and experts
 *                         in one launch), bf16 or fp32.
 *   layers: host array [n_layers] of device weight pointers;
 *   x_in [M][H] bf16; out [M][H] (bf16, or fp32 in the LAYER_ONLY modes); out may alias x_in;
 *   topk_idx_all [n_layers][M][K] int32 (out, optional: NULL to skip);
 *   h_all [n_layers+1][M][H] bf16 (out, optional, residual modes only): h_all[0] = x_in,
 *         h_all[l+1] = the residual stream after layer l; must not overlap x_in. */
int moe_layer_chain(const moe_dims* dims, int32_t M, int32_t n_layers,
                    const moe_layer_weights* layers, const uint16_t* x_in, void* out,
                    int32_t out_dtype, int32_t mode, int32_t* topk_idx_all, uint16_t* h_all,
                    void* ws, size_t ws_bytes, void* stream);

/* moe_layer_chain for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments and results, with no workspace argument.
 * The library's own static device buffer of MOE_NOALLOC_SCRATCH_BYTES (32 MiB)
 * per GPU, held until the process ends, serves as the workspace.
 *   Limit: the call's workspace, moe_workspace_size(dims, M, n_layers), must
 *   fit in it (e.g. the Ling-shaped layer up to 16 rows, or 16 chained layers
 *   at 6 rows): MOE_E_WORKSPACE otherwise, with nothing enqueued.
 *   The call allocates nothing.  The first call on a device looks up the
 *   buffer's address and clears it once with a fill kernel on `stream`.
 *   Every call on one GPU shares the buffer: calls that overlap in time on one
 *   GPU (other streams, other host threads) race and must not be issued.
 *   Device-side status (MOE_E_TIMEOUT, MOE_E_INDEX) stays in that buffer and
 *   is not reported. */
int moe_layer_chain_noalloc(const moe_dims* dims, int32_t M, int32_t n_layers,
                            const moe_layer_weights* layers, const uint16_t* x_in, void* out,
                            int32_t out_dtype, int32_t mode, int32_t* topk_idx_all,
                            uint16_t* h_all, void* stream);

/* bf16 lm_head GEMV and greedy argmax: z[m][v] = sum_h h[m][h] * w_lm[v][h]
 * (fp32 accumulation), token[m] = the smallest v with the largest z[m][v].
 * [LING] "bf16 router gate and lm_head"; greedy decoding.
 *   h [M][H] bf16; w_lm [V][H] bf16; token [M] int32 (out);
 *   max_logit [M] fp32 (out, optional; the z[m][token[m]] found).
 *   1 <= M <= MOE_MAX_ROWS, V >= 1, H a multiple of 256; for 1 or 2 rows H / 256
 *   must be 1, 2, 4, 8 or 10 (MOE_E_UNSUPPORTED otherwise).  token and
 *   max_logit 4-byte aligned.
 *   ws: any workspace from moe_workspace_size() (the lm_head uses only its
 *   header: step tags, counters and one slot per workgroup), ws_bytes its size.
 *   For 1 or 2 rows the sums are formed by vector dot products, from 3 rows on
 *   by the matrix cores (16-row vocabulary tiles); both accumulate in fp32 but in
 *   different orders, so max_logit can differ in its last bits between them. */
int lmhead_argmax(int32_t M, int32_t H, int32_t V, const uint16_t* h, const uint16_t* w_lm,
                  int32_t* token, float* max_logit, void* ws, size_t ws_bytes, void* stream);

/* Speculative expert prefetch: read the gate/up and down weights (and, for fp8
 * experts, their block scales) of the experts listed in expert_ids into the
 * device caches, so that a later call on the same weights finds them there.
 * Consecutive decode steps tend to route alike, so the experts a layer chose on
 * the previous step are the natural guess, issued while other work (attention)
 * runs.  [MUSE] "Megakernel internals": speculative expert prefetching.  On
 * MI355X the level that holds a layer's experts is the 256 MB Infinity Cache
 * shared by all XCDs (an XCD's L2 is 4 MB).  The call computes and writes
 * nothing: every result of a later call is the same with or without it.
 *   dims, w: the layer's shape and weights (as for moe_experts_fused; the router
 *       fields are ignored);
 *   expert_ids [n] int32 device pointer, 4-byte aligned: ids in [0, E) name routed
 *       experts, E the shared expert (when S = 1); an id outside [0, E+S) is
 *       skipped without error (a guess is a hint);
 *   0 <= n <= MOE_MAX_PREFETCH_IDS; n = 0 enqueues nothing.
 * Needs no workspace.  Returns MOE_OK, or MOE_E_ARG / MOE_E_ALIGN /
 * MOE_E_UNSUPPORTED / MOE_E_HIP with nothing enqueued (MOE_E_HIP: launch). */
int moe_expert_prefetch(const moe_dims* dims, const moe_layer_weights* w,
                        const int32_t* expert_ids, int32_t n, void* stream);

/* Synchronise `stream`, return the sticky device status recorded in the
 * workspace (MOE_OK, MOE_E_TIMEOUT or MOE_E_INDEX) and clear it. */
int moe_last_device_status(void* ws, size_t ws_bytes, void* stream);

/* Test and measurement hook: set the wait deadline (microseconds, 0 = default
 * 200 ms) and debug flags for later calls on this workspace.
 *   bit 0: the router never publishes its logits, so every wait on them ends at
 *          the deadline (exercises the timeout path);
 *   bit 1: phase stamps.  The fused kernel records the 100 MHz global clock at
 *          its phase boundaries into the workspace at byte offset 4096, as
 *          uint64 [256 workgroups][32 slots]: slots 10*s + e for layer slot
 *          s (0: first layer, 1: second, 2: last) and event e (0 layer start,
 *          1 input staged, 2 router and shared gate/up rows done, 3 logits
 *          received, 9 top-k done, 4 expert union built, 5 routed gate/up
 *          done, 6 down inputs staged, 7 down projection done, 8 combine
 *          done); slot 31 is
 *          the end of the call;
 *   bit 2: the occupancy check of the fused layer kernel reports that its grid
 *          would not be resident, so layer calls on this workspace return
 *          MOE_E_UNSUPPORTED with nothing enqueued (exercises that gate). */
int moe_workspace_debug(void* ws, size_t ws_bytes, uint32_t flags, uint32_t deadline_us,
                        void* stream);

/* Static description of a status code. */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
