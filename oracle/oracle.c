/* CPU oracle of the small-M MoE decoder step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file:
 * it is used by the tests, by the smoke check and by the benchmark's CPU
 * baseline leg.  It shares no code with the HIP kernels.
 *
 * It is the plain definition of the layer, written for a reader to check by
 * eye: every dot product is an fp32 sum of exact bf16 x bf16 products taken
 * left to right in index order, with the rounding points stated below.  It is
 * built with -ffp-contract=off and without fast-math; OpenMP only splits work
 * over independent outputs, so results do not depend on the thread count.
 *
 * Sources (page titles and sections; formulas restated, not quoted):
 *  - "Ling-3.0-flash on 4 Blackwell GPUs" (LMSYS blog), section "The model":
 *    512 routed experts plus one shared expert, top-8 (+1), expert
 *    intermediate size 768, hidden size 2560, about 157k vocabulary.
 *  - same page, "PDL: stacking the latency floors of small kernels": the
 *    router chain is gate matvec then top-k; the MoE chain is up-GEMM,
 *    activation, down-GEMM, combine; the small-M combine sums in fp32 and
 *    casts once.
 *  - same page, "Two fusions and a retune": SwiGLU folded into the up-GEMM
 *    epilogue, silu evaluated in float and the product rounded once.
 *  - same page, "bf16 router gate and lm_head": bf16 router and lm_head
 *    weights; greedy decoding takes the argmax token.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  gates are a full softmax over all experts' logits renormalised over the
 *  selected K; ties in selection and argmax go to the lower index; the shared
 *  expert is added with weight 1; a residual chain rounds h + acc once; the
 *  chain workload feeds each layer bf16(RMSNorm(h)) (without it the residual
 *  stream of random layers diverges within a dozen layers); a selection bias
 *  is added to the logits in fp32 for choosing experts only; the routed
 *  scaling factor multiplies the fp32 routed sum before the shared expert is
 *  added; the norm's gain multiplies h * r in fp32 before the one rounding.
 *
 * Parity pins: every exported function is pinned by the CPU tests
 * (exact rational arithmetic on dyadic inputs, float64 bounds, brute-force
 * selection, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ---- bf16 <-> fp32 ------------------------------------------------------ */

/* bf16 bits -> fp32: exact (bf16 is the top half of an fp32). */
static float bf2f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16 bits, IEEE round to nearest, ties to even; NaN stays NaN. */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float oracle_bf16_to_f32(uint16_t b) { return bf2f(b); }

void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---- router: bf16 gate matvec -------------------------------------------
 * logits[m][e] = sum_h x[m][h] * W_r[e][h], fp32, h ascending.
 * ("bf16 router gate and lm_head"; router chain in "PDL: stacking ...") */
void oracle_router_logits(int H, int E, int M, const uint16_t* x, const uint16_t* w_router,
                          float* logits) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int m = 0; m < M; ++m)
    for (int e = 0; e < E; ++e) {
      const uint16_t* xr = x + (size_t)m * H;
      const uint16_t* wr = w_router + (size_t)e * H;
      float s = 0.0f;
      for (int h = 0; h < H; ++h) s = s + bf2f(xr[h]) * bf2f(wr[h]);
      logits[(size_t)m * E + e] = s;
    }
}

/* ---- softmax top-k with renormalised gates ------------------------------
 * Selection: the K experts with the largest selection scores
 * s_e = fp32(l_e + b_e), in descending order, equal scores ordered by lower
 * expert index; b is an optional per-expert selection bias (NULL: s_e = l_e).
 * The bias only chooses experts: the gates use the unbiased logits.
 * (Reading of "PDL: stacking ...", figure on the router path, where the top-k
 * kernel loads a bias of its own before its producer's output is ready.)
 * Gates: p_e = exp(l_e - max_l) (exp in double, rounded once to fp32),
 * Z = sum_e p_e (index order), q_e = p_e / Z, G = sum_k q_{S[k]} (rank order),
 * g_k = q_{S[k]} / G. */
void oracle_select_gates(int E, int K, int M, const float* logits, const float* bias,
                         int32_t* idx, float* gate) {
  float* p = (float*)malloc(sizeof(float) * (size_t)E);
  float* sc = (float*)malloc(sizeof(float) * (size_t)E);
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int m = 0; m < M; ++m) {
    const float* l = logits + (size_t)m * E;
    for (int e = 0; e < E; ++e) sc[e] = bias ? l[e] + bias[e] : l[e];
    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || sc[e] > sc[best]) best = e; /* strict: first (lowest) index wins ties */
      }
      taken[best] = 1;
      idx[(size_t)m * K + k] = best;
    }
    float mu = l[0];
    for (int e = 1; e < E; ++e)
      if (l[e] > mu) mu = l[e];
    float Z = 0.0f;
    for (int e = 0; e < E; ++e) {
      p[e] = (float)exp((double)l[e] - (double)mu);
      Z = Z + p[e];
    }
    float G = 0.0f;
    for (int k = 0; k < K; ++k) G = G + p[idx[(size_t)m * K + k]] / Z;
    for (int k = 0; k < K; ++k) gate[(size_t)m * K + k] = (p[idx[(size_t)m * K + k]] / Z) / G;
  }
  free(p);
  free(sc);
  free(taken);
}

/* ---- SwiGLU epilogue -----------------------------------------------------
 * h = bf16(silu(a) * b): silu(a) = a / (1 + exp(-a)) evaluated in double and
 * rounded once to fp32, the product formed in fp32, then one rounding to bf16.
 * ("Two fusions and a retune": silu stays in float, single final rounding.) */
uint16_t oracle_swiglu(float a, float b) {
  float s = (float)((double)a / (1.0 + exp(-(double)a)));
  return oracle_f32_to_bf16(s * b);
}

/* ---- one expert on one token row -----------------------------------------
 * w_gu: [2I][H], rows [0, I) gate, rows [I, 2I) up;  w_d: [H][I].
 * a_j = sum_h x_h Wg[j][h],  b_j = sum_h x_h Wu[j][h]   (fp32, h ascending)
 * hb_j = bf16(silu(a_j) * b_j)
 * y_n = sum_j hb_j Wd[n][j]                              (fp32, j ascending) */
void oracle_expert(int H, int I, const uint16_t* x_row, const uint16_t* w_gu, const uint16_t* w_d,
                   uint16_t* h_out, float* y) {
  uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
#pragma omp parallel for schedule(static)
  for (int j = 0; j < I; ++j) {
    const uint16_t* wg = w_gu + (size_t)j * H;
    const uint16_t* wu = w_gu + (size_t)(I + j) * H;
    float a = 0.0f, b = 0.0f;
    for (int h = 0; h < H; ++h) a = a + bf2f(x_row[h]) * bf2f(wg[h]);
    for (int h = 0; h < H; ++h) b = b + bf2f(x_row[h]) * bf2f(wu[h]);
    hb[j] = oracle_swiglu(a, b);
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; ++n) {
    const uint16_t* wd = w_d + (size_t)n * I;
    float s = 0.0f;
    for (int j = 0; j < I; ++j) s = s + bf2f(hb[j]) * bf2f(wd[j]);
    y[n] = s;
  }
  if (h_out) memcpy(h_out, hb, sizeof(uint16_t) * (size_t)I);
  free(hb);
}

/* ---- fp8 block-128 expert weights ---------------------------------------
 * ("Ling-3.0-flash on 4 Blackwell GPUs", "Where the time goes now": fp8 weights with
 * 128-wide quantisation blocks halve the bytes of the bandwidth-bound work.)
 * Codes are OCP FP8 E4M3 ("e4m3fn"): sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the code with
 * every exponent and mantissa bit set is NaN; there are no infinities.
 * A weight is code value times the fp32 scale of its 128 x 128 block:
 *   W[r][c] = dec(q[r][c]) * s[r / 128][c / 128],
 * formed exactly in double and rounded once to fp32; activations stay bf16. */
float oracle_fp8_e4m3_to_f32(uint8_t c) {
  int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return (float)(sign ? -v : v);
}

void oracle_dequant_fp8(int rows, int cols, const uint8_t* q, const float* s, float* w) {
  const int cb = cols / 128;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      double v = (double)oracle_fp8_e4m3_to_f32(q[(size_t)r * cols + c]) *
                 (double)s[(size_t)(r / 128) * cb + c / 128];
      w[(size_t)r * cols + c] = (float)v;
    }
}

/* One expert on one token row with fp32 weights (the dequantised fp8 ones):
 * a_j = sum_h x_h Wg[j][h], b_j = sum_h x_h Wu[j][h] (fp32, h ascending),
 * hb_j = bf16(silu(a_j) * b_j), y_n = sum_j hb_j Wd[n][j] (fp32, j ascending). */
static void expert_f32w(int H, int I, const uint16_t* x_row, const float* w_gu, const float* w_d,
                        uint16_t* h_out, float* y) {
  uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
#pragma omp parallel for schedule(static)
  for (int j = 0; j < I; ++j) {
    const float* wg = w_gu + (size_t)j * H;
    const float* wu = w_gu + (size_t)(I + j) * H;
    float a = 0.0f, b = 0.0f;
    for (int h = 0; h < H; ++h) a = a + bf2f(x_row[h]) * wg[h];
    for (int h = 0; h < H; ++h) b = b + bf2f(x_row[h]) * wu[h];
    hb[j] = oracle_swiglu(a, b);
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; ++n) {
    const float* wd = w_d + (size_t)n * I;
    float t = 0.0f;
    for (int j = 0; j < I; ++j) t = t + bf2f(hb[j]) * wd[j];
    y[n] = t;
  }
  if (h_out) memcpy(h_out, hb, sizeof(uint16_t) * (size_t)I);
  free(hb);
}

/* One fp8 expert: q_gu [2I][H] codes with s_gu [2I/128][H/128], q_d [H][I] codes
 * with s_d [H/128][I/128]; dequantise, then the fp32-weight expert above. */
void oracle_expert_fp8(int H, int I, const uint16_t* x_row, const uint8_t* q_gu,
                       const float* s_gu, const uint8_t* q_d, const float* s_d, uint16_t* h_out,
                       float* y) {
  float* wgu = (float*)malloc(sizeof(float) * (size_t)2 * I * H);
  float* wd = (float*)malloc(sizeof(float) * (size_t)H * I);
  oracle_dequant_fp8(2 * I, H, q_gu, s_gu, wgu);
  oracle_dequant_fp8(H, I, q_d, s_d, wd);
  expert_f32w(H, I, x_row, wgu, wd, h_out, y);
  free(wgu);
  free(wd);
}

/* ---- experts + gate-weighted combine + shared expert -----------------------
 * Per row m and output n (fp32, one rounding per operation, no contraction):
 *   R = 0, then for k = 0..K-1 in rank order: R = R + g[m][k] * y_{idx[m][k]}[m][n]
 *   acc[m][n] = y_shared[m][n] + scale * R          (y_shared = 0 without one)
 * The routed part is summed in fp32 and scaled once ("PDL: stacking ...": the
 * small-M combine is an fp32 sum times a scale with a single final cast; the
 * scale is the routed scaling factor, 1 unless the model sets one).  The
 * caller casts acc once.  `expert(ctx, e, row, y)` computes expert e on one
 * token row, returning -1 if its weights are missing. */
typedef int (*expert_fn)(void* ctx, int e, const uint16_t* x_row, float* y);

static int combine_core(int H, int E, int K, int S, int M, const uint16_t* x, const int32_t* idx,
                        const float* gate, float scale, expert_fn expert, void* ctx, float* acc) {
  float* y = (float*)malloc(sizeof(float) * (size_t)H);
  float* R = (float*)malloc(sizeof(float) * (size_t)H);
  int rc = 0;
  for (int m = 0; m < M && rc == 0; ++m) {
    const uint16_t* xr = x + (size_t)m * H;
    float* a = acc + (size_t)m * H;
    for (int n = 0; n < H; ++n) R[n] = 0.0f;
    for (int k = 0; k < K; ++k) {
      int e = idx[(size_t)m * K + k];
      if (e < 0 || e >= E || expert(ctx, e, xr, y) != 0) { rc = -1; break; }
      float g = gate[(size_t)m * K + k];
      for (int n = 0; n < H; ++n) {
        float t = g * y[n];
        R[n] = R[n] + t;
      }
    }
    if (rc) break;
    if (S) {
      if (expert(ctx, E, xr, y) != 0) { rc = -1; break; }
    } else {
      for (int n = 0; n < H; ++n) y[n] = 0.0f;
    }
    for (int n = 0; n < H; ++n) {
      float t = scale * R[n];
      a[n] = y[n] + t;
    }
  }
  free(R);
  free(y);
  return rc;
}

/* bf16 experts: w_gu_tab / w_d_tab are tables of per-expert weight pointers
 * indexed by expert id (shared expert at index E); only the experts used need
 * to be present.  Returns 0, or -1 if an index is out of range or a needed
 * weight is missing. */
struct bf16_tabs {
  int H, I;
  const uint16_t* const* gu;
  const uint16_t* const* d;
};

static int bf16_expert(void* ctx, int e, const uint16_t* x_row, float* y) {
  const struct bf16_tabs* t = (const struct bf16_tabs*)ctx;
  if (!t->gu[e] || !t->d[e]) return -1;
  oracle_expert(t->H, t->I, x_row, t->gu[e], t->d[e], NULL, y);
  return 0;
}

int oracle_experts_combine(int H, int E, int K, int I, int S, int M, const uint16_t* x,
                           const int32_t* idx, const float* gate,
                           const uint16_t* const* w_gu_tab, const uint16_t* const* w_d_tab,
                           float scale, float* acc) {
  struct bf16_tabs t = {H, I, w_gu_tab, w_d_tab};
  return combine_core(H, E, K, S, M, x, idx, gate, scale, bf16_expert, &t, acc);
}

/* fp8 experts: code and scale tables per expert id, as above. */
struct fp8_tabs {
  int H, I;
  const uint8_t* const* qgu;
  const float* const* sgu;
  const uint8_t* const* qd;
  const float* const* sd;
};

static int fp8_expert(void* ctx, int e, const uint16_t* x_row, float* y) {
  const struct fp8_tabs* t = (const struct fp8_tabs*)ctx;
  if (!t->qgu[e] || !t->sgu[e] || !t->qd[e] || !t->sd[e]) return -1;
  oracle_expert_fp8(t->H, t->I, x_row, t->qgu[e], t->sgu[e], t->qd[e], t->sd[e], NULL, y);
  return 0;
}

int oracle_experts_combine_fp8(int H, int E, int K, int I, int S, int M, const uint16_t* x,
                               const int32_t* idx, const float* gate,
                               const uint8_t* const* q_gu_tab, const float* const* s_gu_tab,
                               const uint8_t* const* q_d_tab, const float* const* s_d_tab,
                               float scale, float* acc) {
  struct fp8_tabs t = {H, I, q_gu_tab, s_gu_tab, q_d_tab, s_d_tab};
  return combine_core(H, E, K, S, M, x, idx, gate, scale, fp8_expert, &t, acc);
}

/* out = bf16(acc): the single final cast of the combine. */
void oracle_cast_bf16(int64_t n, const float* acc, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(acc[i]);
}

/* Residual chain step: h_next = bf16(h + acc), one rounding. */
void oracle_residual(int64_t n, const uint16_t* h, const float* acc, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    float t = bf2f(h[i]) + acc[i];
    out[i] = oracle_f32_to_bf16(t);
  }
}

/* RMSNorm in front of the router and the experts (the router chain of
 * "PDL: stacking ..." opens with a norm; the chain workload also relies on it
 * to keep every layer's input at unit scale):
 *   ss = sum_n h_n^2 accumulated in double (each square of a bf16 value is exact,
 *        and for the chain's value range so is every partial sum, so ss is the
 *        exact sum whatever the order),
 *   r = 1 / sqrt(ss / H + eps) in double, rounded once to fp32,
 *   u_n = bf16((h_n * r) * w_n), both products in fp32 and one rounding to bf16,
 * with w the norm's bf16 gain vector [H] (NULL: unit gain, u_n = bf16(h_n * r)). */
void oracle_rmsnorm(int M, int H, const uint16_t* h, float eps, const uint16_t* gain,
                    uint16_t* u) {
  for (int m = 0; m < M; ++m) {
    const uint16_t* hr = h + (size_t)m * H;
    double ss = 0.0;
    for (int n = 0; n < H; ++n) {
      double v = (double)bf2f(hr[n]);
      ss = ss + v * v;
    }
    float r = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
    for (int n = 0; n < H; ++n) {
      float t = bf2f(hr[n]) * r;
      if (gain) t = t * bf2f(gain[n]);
      u[(size_t)m * H + n] = oracle_f32_to_bf16(t);
    }
  }
}

/* ---- bf16 lm_head GEMV and greedy argmax ------------------------------------
 * z[m][v] = sum_h h[m][h] W[v][h] (fp32, h ascending); token[m] = the smallest
 * v with the largest z.  ("bf16 router gate and lm_head"; greedy decoding.) */
void oracle_lmhead_argmax(int M, int H, int V, const uint16_t* hrows, const uint16_t* w,
                          int32_t* token, float* max_logit) {
  for (int m = 0; m < M; ++m) {
    const uint16_t* hr = hrows + (size_t)m * H;
    int nt = omp_get_max_threads();
    float* bv = (float*)malloc(sizeof(float) * (size_t)nt);
    int* bi = (int*)malloc(sizeof(int) * (size_t)nt);
    for (int t = 0; t < nt; ++t) bi[t] = -1;
#pragma omp parallel num_threads(nt)
    {
      int t = omp_get_thread_num(), T = omp_get_num_threads();
      int64_t lo = (int64_t)V * t / T, hi = (int64_t)V * (t + 1) / T;
      float best = 0.0f;
      int besti = -1;
      for (int64_t v = lo; v < hi; ++v) {
        const uint16_t* wr = w + (size_t)v * H;
        float s = 0.0f;
        for (int h = 0; h < H; ++h) s = s + bf2f(hr[h]) * bf2f(wr[h]);
        if (besti < 0 || s > best) { best = s; besti = (int)v; }
      }
      bv[t] = best;
      bi[t] = besti;
    }
    /* ranges are in ascending v order: a strict > keeps the smallest v on ties */
    float best = 0.0f;
    int besti = -1;
    for (int t = 0; t < nt; ++t) {
      if (bi[t] < 0) continue;
      if (besti < 0 || bv[t] > best) { best = bv[t]; besti = bi[t]; }
    }
    token[m] = besti;
    if (max_logit) max_logit[m] = best;
    free(bv);
    free(bi);
  }
}

/* ---- algorithmic bytes of one layer call -----------------------------------
 * Unique weight bytes streamed: the router, plus every expert in the union of
 * the rows' selections and the shared expert, each read once (3 * H * I bf16
 * values per expert).  Returns the union size through *U. */
int64_t oracle_unique_weight_bytes(int H, int E, int K, int I, int S, int M, const int32_t* idx,
                                   int include_router, int* U) {
  unsigned char* seen = (unsigned char*)calloc((size_t)E, 1);
  int u = 0;
  for (int i = 0; i < M * K; ++i) {
    int e = idx[i];
    if (e >= 0 && e < E && !seen[e]) { seen[e] = 1; ++u; }
  }
  free(seen);
  if (U) *U = u;
  int64_t bytes = (int64_t)(u + S) * 3 * (int64_t)H * I * 2;
  if (include_router) bytes += (int64_t)E * H * 2;
  return bytes;
}
