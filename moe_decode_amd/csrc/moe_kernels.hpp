// gfx950 kernels of libmoedecode.
//
// moe_layer_kernel: one persistent launch runs one or several MoE layers.  One
// 512-thread workgroup per CU; every workgroup is resident for the whole call.
// Per layer:
//   P0  stage the layer input x [M][H] in LDS (layer 0 from the caller's
//       buffer, later layers from the step-tagged residual words); under the
//       pre-norm chain, keep this workgroup's rows of h_l for the residual and
//       replace x by bf16(RMSNorm(h_l))
//   P1  router GEMV rows and the shared expert's gate/up rows.  The shared
//       expert does not depend on routing, so its weights stream while the
//       router's logits travel ("weights that do not depend on routing load
//       before their inputs arrive", SGLang Low-Latency Mode, AMD Low-Latency
//       Kernels).
//   P4  every workgroup reads all logits (tagged) and computes the softmax
//       top-k itself, so no second device-wide hop is needed.
//   P5  union of the rows' expert choices: a bitmap over experts plus
//       population counts gives each selected expert its slot, with no scan
//       or sort (SGLang Low-Latency Mode, item 3, at most eight rows).
//   P6  gate/up GEMV + SwiGLU for the routed experts; each (expert, row-pair
//       of the intermediate dimension) is one wave task; results are written
//       as tagged bf16 pairs.  Every selected expert's rows stream once, for
//       all the token rows that chose it.
//   P7  down GEMV: workgroup g owns output rows [n0, n1) of every expert, so
//       the combine needs no atomics and rounds once.
//   P8  combine y_shared + sum_k g_k y_k in fp32 (rank order), then one cast
//       (or the residual h + acc with one rounding, or the fp32 partial).
//
// moe_lmhead_kernel: bf16 lm_head GEMV with the greedy argmax folded in; the
// per-row best (logit, index) pairs meet in a 64-bit atomic max.
#pragma once

#include "moe_device.hpp"

namespace moe {

#ifndef MOE_MAX_LAYERS
#define MOE_MAX_LAYERS 64
#endif

struct LayerW {
  const uint16_t* wr;   // [E][H]
  const uint16_t* wgu;  // [E+S][2I][H]
  const uint16_t* wd;   // [E+S][H][I]
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

struct Params {
  int H, E, K, I, S, M, L;
  uint32_t flags;
  int lpr_i;          // lanes per down-projection row (8, 16 or 32)
  int hb_pairs;       // (expert, row) pairs of h staged in LDS at a time
  int nr_max;         // output rows owned by one workgroup, at most
  int pmax;           // h slots per layer = M * (K + S)
  // LDS byte offsets
  int lds_xs, lds_r, lds_ys, lds_small;
  const uint16_t* x_in;
  void* out;
  const int32_t* tk_idx_in;
  const float* tk_gate_in;
  int32_t* tk_idx_out;   // [L][M][K] (or [M][K])
  uint16_t* h_all;       // [L+1][M][H] residual stream per layer (optional)
  float* tk_gate_out;    // [M][K]
  float* logits_out;     // [M][E]
  uint32_t* hdr;
  uint64_t* lg_buf;      // [L][M][E]      tagged fp32 logits
  uint64_t* h_buf;       // [L][pmax][I/2] tagged bf16 pairs
  uint64_t* res_buf;     // [L+1][M][H/2]  tagged bf16 pairs
  LayerW lw[MOE_MAX_LAYERS];
};

// Small LDS tables (after the big regions).
struct Small {
  int nU, nP, nG, abort_flag;
  int tk_idx[MOE_MAXM * 16];
  float tk_gate[MOE_MAXM * 16];
  float tk_val[MOE_MAXM * 16];
  int upos[MOE_MAXM * 16];
  int uexp[MOE_MAXM * 16 + 1];
  uint32_t umask[MOE_MAXM * 16 + 1];
  int pbase[MOE_MAXM * 16 + 2];
  int gstart[MOE_MAXM * 16 + 2];   // union-entry boundaries of the h staging groups
  uint32_t bm[32];                 // expert bitmap (E <= 1024)
  int bpre[32];                    // population-count prefix per bitmap word
  float rn[MOE_MAXM];              // RMSNorm scale per token row
  uint16_t hres[MOE_MAXM * 64];    // residual input h_l of this workgroup's output rows
};

__device__ __forceinline__ float swiglu(float a, float b) {
  const float s = a / (1.0f + expf(-a));
  return s * b;
}

__device__ __forceinline__ float select8(const float (&acc)[MOE_MAXM], int i) {
  float v = acc[0];
#pragma unroll
  for (int m = 1; m < MOE_MAXM; ++m) v = (i == m) ? acc[m] : v;
  return v;
}

// Router task: rows e0 = 2*it (lanes 0-31) and e0 + 1 (lanes 32-63), all M token rows.
template <int CPLH>
__device__ __forceinline__ void router_task(const Params& p, int l, int it, const uint4* xs4,
                                            uint32_t tag, int lane, uint32_t dbg) {
  const int grp = lane >> 5, li = lane & 31;
  const int e = 2 * it + grp;
  const bool valid = e < p.E;
  const int H8 = p.H >> 3;
  const uint4* row = reinterpret_cast<const uint4*>(p.lw[l].wr + (size_t)(valid ? e : 0) * p.H);
  uint4 w[CPLH];
#pragma unroll
  for (int q = 0; q < CPLH; ++q) w[q] = row[li + 32 * q];
  float acc[MOE_MAXM];
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) {
    acc[m] = 0.0f;
    if (m < p.M) {
#pragma unroll
      for (int q = 0; q < CPLH; ++q) acc[m] = dot8(w[q], xs4[m * H8 + li + 32 * q], acc[m]);
      acc[m] = group_sum(acc[m], 32);
    }
  }
  if (valid && li < p.M && !(dbg & DBG_NO_ROUTER_PUBLISH)) {
    const float v = select8(acc, li);
    st_tag(p.lg_buf + ((size_t)l * p.M + li) * p.E + e, __float_as_uint(v), tag);
  }
}

// Gate/up task of expert e at intermediate pair jp (rows 2jp, 2jp+1): gate row
// on lanes 0-31, up row on lanes 32-63, for the token rows in `mask`; writes
// bf16(silu(a) * b) for both rows as one tagged word per token row.
template <int CPLH>
__device__ __forceinline__ void gateup_task(const Params& p, int l, int e, int jp, uint32_t mask,
                                            int pair_base, const uint4* xs4, uint32_t tag,
                                            int lane) {
  const int grp = lane >> 5, li = lane & 31;
  const int H8 = p.H >> 3;
  const size_t I = (size_t)p.I;
  const uint16_t* base = p.lw[l].wgu + (size_t)e * (2 * I) * p.H;
  const int j0 = 2 * jp;
  const uint4* r0 = reinterpret_cast<const uint4*>(base + ((size_t)grp * I + j0) * p.H);
  const uint4* r1 = reinterpret_cast<const uint4*>(base + ((size_t)grp * I + j0 + 1) * p.H);
  uint4 w0[CPLH], w1[CPLH];
#pragma unroll
  for (int q = 0; q < CPLH; ++q) w0[q] = r0[li + 32 * q];
#pragma unroll
  for (int q = 0; q < CPLH; ++q) w1[q] = r1[li + 32 * q];
  uint32_t word = 0u;
#pragma unroll
  for (int m = 0; m < MOE_MAXM; ++m) {
    if (m < p.M && ((mask >> m) & 1u)) {
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int q = 0; q < CPLH; ++q) {
        const uint4 xv = xs4[m * H8 + li + 32 * q];
        a0 = dot8(w0[q], xv, a0);
        a1 = dot8(w1[q], xv, a1);
      }
      a0 = group_sum(a0, 32);
      a1 = group_sum(a1, 32);
      const float g0 = readlane_f(a0, 0), u0 = readlane_f(a0, 32);
      const float g1 = readlane_f(a1, 0), u1 = readlane_f(a1, 32);
      const uint32_t wm = f_to_bf(swiglu(g0, u0)) | (f_to_bf(swiglu(g1, u1)) << 16);
      if (lane == m) word = wm;
    }
  }
  if (lane < p.M && ((mask >> lane) & 1u)) {
    const int pair = pair_base + __builtin_popcount(mask & ((1u << lane) - 1u));
    st_tag(p.h_buf + ((size_t)l * p.pmax + pair) * (p.I >> 1) + jp, word, tag);
  }
}

// Softmax top-k of one token row (one wave).  Experts are held in contiguous
// blocks per lane, so the lowest lane among equal keys holds the lowest index.
__device__ __forceinline__ void topk_row(const Params& p, const float* lgs, int m, Small* sm,
                                         int lane) {
  const int E = p.E, K = p.K;
  const int per = (E + 63) >> 6;  // <= 16
  uint32_t keys[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane * per + i;
    keys[i] = (i < per && e < E) ? f_key(lgs[m * E + e]) : 0u;
  }
  uint32_t taken = 0u;
  for (int k = 0; k < K; ++k) {
    uint32_t lb = 0u;
    int li = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!((taken >> i) & 1u) && keys[i] > lb) { lb = keys[i]; li = i; }
    const uint32_t wmax = wave_max_u32(lb);
    const uint64_t ball = __ballot(li >= 0 && lb == wmax);
    const int wl = __builtin_ctzll(ball);
    const int wi = __builtin_amdgcn_readlane(li, wl);
    if (lane == wl) taken |= 1u << wi;
    const int e = wl * per + wi;
    if (lane == 0) {
      sm->tk_idx[m * K + k] = e;
      sm->tk_val[m * K + k] = lgs[m * E + e];
    }
  }
  // gates: p_k = exp(l_k - max), renormalised over the K selected (the full
  // softmax denominator cancels in the renormalisation)
  if (lane == 0) {
    const float mu = sm->tk_val[m * K];
    float s = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float pk = expf(sm->tk_val[m * K + k] - mu);
      sm->tk_gate[m * K + k] = pk;
      s = s + pk;
    }
    for (int k = 0; k < K; ++k) sm->tk_gate[m * K + k] = sm->tk_gate[m * K + k] / s;
  }
}

// Union of the selected experts (+ shared at slot 0), per-slot row masks, the
// (slot, row) pair numbering and the h staging groups.  Whole workgroup.
__device__ __forceinline__ void build_union(const Params& p, Small* sm, int tid) {
  const int MK = p.M * p.K, S = p.S;
  if (tid < 32) sm->bm[tid] = 0u;
  __syncthreads();
  if (tid < MK) {
    const int e = sm->tk_idx[tid];
    if (e >= 0) atomicOr(&sm->bm[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (tid < 32) {
    int pre = 0;
    for (int w = 0; w < tid; ++w) pre += __builtin_popcount(sm->bm[w]);
    sm->bpre[tid] = pre;
    uint32_t bits = sm->bm[tid];
    int pos = S + pre;
    while (bits) {
      const int b = __builtin_ctz(bits);
      bits &= bits - 1u;
      sm->uexp[pos] = tid * 32 + b;
      sm->umask[pos] = 0u;
      ++pos;
    }
    if (tid == 31) sm->nU = S + pre + __builtin_popcount(sm->bm[31]);
  }
  if (tid == 0 && S) {
    sm->uexp[0] = p.E;
    sm->umask[0] = (1u << p.M) - 1u;
  }
  __syncthreads();
  if (tid < MK) {
    const int e = sm->tk_idx[tid];
    int u = -1;
    if (e >= 0) {
      u = S + sm->bpre[e >> 5] + __builtin_popcount(sm->bm[e >> 5] & ((1u << (e & 31)) - 1u));
      atomicOr(&sm->umask[u], 1u << (tid / p.K));
    }
    sm->upos[tid] = u;
  }
  __syncthreads();
  if (tid == 0) {
    int np = 0, ng = 0, gp = 0;
    sm->gstart[0] = 0;
    for (int u = 0; u < sm->nU; ++u) {
      const int c = __builtin_popcount(sm->umask[u]);
      if (gp + c > p.hb_pairs) {   // start a new staging group at u
        sm->gstart[++ng] = u;
        gp = 0;
      }
      sm->pbase[u] = np;
      np += c;
      gp += c;
    }
    sm->pbase[sm->nU] = np;
    sm->gstart[++ng] = sm->nU;
    sm->nP = np;
    sm->nG = ng;
  }
  __syncthreads();
}

template <int CPLH, int CPLI>
__global__ __launch_bounds__(MOE_WG, 1) void moe_layer_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + p.lds_xs);
  const uint4* xs4 = reinterpret_cast<const uint4*>(xs);
  float* lgs = reinterpret_cast<float*>(lds + p.lds_r);
  uint32_t* hs32 = reinterpret_cast<uint32_t*>(lds + p.lds_r);
  const uint4* hs4 = reinterpret_cast<const uint4*>(lds + p.lds_r);
  float* ys = reinterpret_cast<float*>(lds + p.lds_ys);
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
  const int I2 = I >> 1, H2 = H >> 1;
  const bool router_only = (p.flags & F_ROUTER_ONLY) != 0u;
  const bool topk_in = (p.flags & F_TOPK_IN) != 0u;

  if (tid == 0) sm->abort_flag = 0;

  // output rows owned by this workgroup (whole row pairs)
  const int r0 = (int)(((long long)g * H2) / G), r1 = (int)(((long long)(g + 1) * H2) / G);
  const int n0 = 2 * r0, NR = 2 * (r1 - r0);

  for (int l = 0; l < p.L; ++l) {
    // ---------------- P0: layer input -> LDS
    if (l == 0) {
      const uint4* src = reinterpret_cast<const uint4*>(p.x_in);
      uint4* dst = reinterpret_cast<uint4*>(xs);
      for (int i = tid; i < (M * H) >> 3; i += MOE_WG) dst[i] = src[i];
    } else {
      const uint64_t* src = p.res_buf + (size_t)l * M * H2;
      uint32_t* dst = reinterpret_cast<uint32_t*>(xs);
      for (int i = tid; i < M * H2; i += MOE_WG) {
        uint64_t v;
        if (!wait_tag(src + i, tag, wt, v)) sm->abort_flag = 1;
        dst[i] = (uint32_t)v;
      }
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

    // ---------------- P1: router rows + shared expert gate/up rows
    const int NRI = topk_in ? 0 : (E + 1) >> 1;
    const int NSI = (router_only || !S) ? 0 : I2;
    for (int it = gw; it < NRI + NSI; it += NW) {
      if (it < NRI)
        router_task<CPLH>(p, l, it, xs4, tag, lane, dbg);
      else
        gateup_task<CPLH>(p, l, E, it - NRI, (1u << M) - 1u, 0, xs4, tag, lane);
    }

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
      for (int i = tid; i < M * K; i += MOE_WG) {
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
      bool ok = true;
      for (int i = tid; i < M * E; i += MOE_WG) {
        uint64_t v;
        if (!wait_tag(src + i, tag, wt, v)) ok = false;
        lgs[i] = __uint_as_float((uint32_t)v);
      }
      if (!ok) sm->abort_flag = 1;
      __syncthreads();
      if (sm->abort_flag == 1) break;
      for (int m = wv; m < M; m += MOE_WAVES) topk_row(p, lgs, m, sm, lane);
      __syncthreads();
      if (g == 0 || router_only) {
        int32_t* oi = p.tk_idx_out ? p.tk_idx_out + (size_t)l * M * K : nullptr;
        for (int i = tid; i < M * K; i += MOE_WG) {
          if (oi) oi[i] = sm->tk_idx[i];
          if (p.tk_gate_out && l == 0) p.tk_gate_out[i] = sm->tk_gate[i];
        }
        if (p.logits_out && l == 0)
          for (int i = tid; i < M * E; i += MOE_WG) p.logits_out[i] = lgs[i];
      }
      if (router_only) break;
    }

    // ---------------- P5: union of the selected experts
    build_union(p, sm, tid);
    const int nU = sm->nU;

    // ---------------- P6: routed experts, gate/up + SwiGLU
    {
      const int NI = (nU - S) * I2;
      for (int it = gw; it < NI; it += NW) {
        const int u = S + it / I2, jp = it - (it / I2) * I2;
        gateup_task<CPLH>(p, l, sm->uexp[u], jp, sm->umask[u], sm->pbase[u], xs4, tag, lane);
      }
    }

    // ---------------- P7: down projection of this workgroup's rows, all experts
    const int lpr = p.lpr_i, rpi = 64 / lpr;
    const int NB = (NR + rpi - 1) / rpi;
    const int I8 = I >> 3;
    const int gl = lane / lpr, li = lane % lpr;
    const uint64_t* hsrc = p.h_buf + (size_t)l * p.pmax * I2;
    for (int gi = 0; gi < sm->nG; ++gi) {
      const int u0 = sm->gstart[gi], u1 = sm->gstart[gi + 1];
      const int pb0 = sm->pbase[u0], pb1 = sm->pbase[u1];
      {
        bool ok = true;
        for (int i = tid; i < (pb1 - pb0) * I2; i += MOE_WG) {
          uint64_t v;
          if (!wait_tag(hsrc + (size_t)pb0 * I2 + i, tag, wt, v)) ok = false;
          hs32[i] = (uint32_t)v;
        }
        if (!ok) sm->abort_flag = 1;
      }
      __syncthreads();
      if (sm->abort_flag == 1) break;
      if (NR > 0) {
        for (int it = wv; it < (u1 - u0) * NB; it += MOE_WAVES) {
          const int u = u0 + it / NB, blk = it - (it / NB) * NB;
          const int n = n0 + blk * rpi + gl;
          const bool active = n < n0 + NR;
          const uint32_t mask = sm->umask[u];
          const int e = sm->uexp[u];
          const uint4* row = reinterpret_cast<const uint4*>(
              p.lw[l].wd + ((size_t)e * H + (active ? n : n0)) * I);
          uint4 w[CPLI];
#pragma unroll
          for (int q = 0; q < CPLI; ++q) w[q] = row[li + lpr * q];
          float acc[MOE_MAXM];
          const int pb = sm->pbase[u] - pb0;
#pragma unroll
          for (int m = 0; m < MOE_MAXM; ++m) {
            acc[m] = 0.0f;
            if (m < M && ((mask >> m) & 1u)) {
              const int pr = pb + __builtin_popcount(mask & ((1u << m) - 1u));
#pragma unroll
              for (int q = 0; q < CPLI; ++q) acc[m] = dot8(w[q], hs4[pr * I8 + li + lpr * q], acc[m]);
              acc[m] = group_sum(acc[m], lpr);
            }
          }
          if (active && li < M && ((mask >> li) & 1u))
            ys[((size_t)u * p.nr_max + (n - n0)) * M + li] = select8(acc, li);
        }
      }
      __syncthreads();
    }
    if (sm->abort_flag == 1) break;

    // ---------------- P8: combine (+ residual) and hand off
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
    for (int i = tid; i < (NR >> 1) * M; i += MOE_WG) {
      const int np = i / M, m = i - np * M;
      const int nl = 2 * np;
      float acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float a = S ? ys[((size_t)0 * p.nr_max + nl + t) * M + m] : 0.0f;
        for (int k = 0; k < K; ++k) {
          const int u = sm->upos[m * K + k];
          if (u >= 0) {
            const float tmul = sm->tk_gate[m * K + k] * ys[((size_t)u * p.nr_max + nl + t) * M + m];
            a = a + tmul;
          }
        }
        acc[t] = a;
      }
      const int n = n0 + nl;
      if (p.flags & F_RESIDUAL) {
        const float h0 = bf_to_f(sm->hres[m * p.nr_max + nl]);
        const float h1 = bf_to_f(sm->hres[m * p.nr_max + nl + 1]);
        const uint32_t word = f_to_bf(h0 + acc[0]) | (f_to_bf(h1 + acc[1]) << 16);
        if (last)
          reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = word;
        else
          st_tag(p.res_buf + (size_t)(l + 1) * M * H2 + ((m * H + n) >> 1), word, tag);
        if (p.h_all)
          reinterpret_cast<uint32_t*>(p.h_all)[((size_t)(l + 1) * M * H + (size_t)m * H + n) >> 1] =
              word;
      } else if (p.flags & F_OUT_F32) {
        reinterpret_cast<float2*>(p.out)[(m * H + n) >> 1] = make_float2(acc[0], acc[1]);
      } else {
        reinterpret_cast<uint32_t*>(p.out)[(m * H + n) >> 1] = f_to_bf(acc[0]) | (f_to_bf(acc[1]) << 16);
      }
    }
    __syncthreads();
  }

  // ---------------- end of call: the last workgroup advances the step
  __syncthreads();
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

// ------------------------------------------------------------------ lm_head

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
