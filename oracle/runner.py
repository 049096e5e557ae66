"""Run the oracle on a synthetic workload (TEST INFRASTRUCTURE ONLY).

Generates, through the shared seeded generator, exactly the weights the
oracle's own routing selects, so a layer never needs the full expert tensor
on the host.
"""
import numpy as np

from datagen import workloads as W

from . import (cast_bf16, experts_combine, experts_combine_fp8, lmhead_argmax, residual, rmsnorm,
               router_topk)


class ExpertCache:
    """Host copies of generated expert weights, keyed by (layer, expert)."""

    def __init__(self, wl):
        self.wl = wl
        self.gu = {}
        self.d = {}

    def get(self, layer, e):
        """bf16 weights, or (codes, scales) pairs for an fp8 workload."""
        k = (layer, e)
        if k not in self.gu:
            if self.wl.fp8:
                self.gu[k] = W.expert_gate_up_fp8(self.wl, layer, e)
                self.d[k] = W.expert_down_fp8(self.wl, layer, e)
            else:
                self.gu[k] = W.expert_gate_up(self.wl, layer, e)
                self.d[k] = W.expert_down(self.wl, layer, e)
        return self.gu[k], self.d[k]

    def drop_layer(self, layer):
        for k in [k for k in self.gu if k[0] == layer]:
            del self.gu[k]
            del self.d[k]


def layer(wl, x, layer_idx=0, cache=None, w_router=None):
    """One MoE layer on its (already normed) input x: returns dict(idx, gate, logits,
    acc fp32 [M, H]), with the workload's selection bias and routed scaling factor."""
    if w_router is None:
        w_router = W.router(wl, layer_idx)
    idx, gate, logits = router_topk(x, w_router, wl.K, W.router_bias(wl, layer_idx))
    cache = cache or ExpertCache(wl)
    used = sorted(set(int(e) for e in idx.ravel()))
    if wl.S:
        used.append(wl.E)
    gu, d = {}, {}
    for e in used:
        gu[e], d[e] = cache.get(layer_idx, e)
    combine = experts_combine_fp8 if wl.fp8 else experts_combine
    acc = combine(x, idx, gate, gu, d, wl.E, wl.S, wl.routed_scale)
    return dict(idx=idx, gate=gate, logits=logits, acc=acc)


def front_layer(wl, x, layer_idx=0, cache=None):
    """One layer with the router front: u = bf16(RMSNorm(x) * gain) feeds the router and the
    experts when wl.prenorm; returns layer()'s dict plus u_in."""
    u = rmsnorm(x, gain=W.norm_gain(wl, layer_idx)) if wl.prenorm else x
    r = layer(wl, u, layer_idx, cache)
    r["u_in"] = u
    return r


def layer_output(wl, res):
    """The layer's output as the call returns it (fp32 partial or one bf16 cast)."""
    return res["acc"] if wl.out_f32 else cast_bf16(res["acc"])


def chain(wl, x, n_layers=None, keep_cache=False, prenorm=None, routers=None):
    """Residual chain h_{l+1} = bf16(h_l + MoE_l(u_l)) with u_l = bf16(RMSNorm(h_l) * gain_l)
    when prenorm (the chain workload), else u_l = h_l; returns (h_L, per-layer results)."""
    n_layers = wl.n_layers if n_layers is None else n_layers
    prenorm = wl.prenorm if prenorm is None else prenorm
    h = np.ascontiguousarray(x, dtype=np.uint16)
    per = []
    cache = ExpertCache(wl)
    for l in range(n_layers):
        u = rmsnorm(h, gain=W.norm_gain(wl, l)) if prenorm else h
        r = layer(wl, u, l, cache, w_router=None if routers is None else routers[l])
        r["h_in"] = h
        r["u_in"] = u
        h = residual(h, r["acc"])
        per.append(r)
        if not keep_cache:
            cache.drop_layer(l)
    return h, per


def router_margin(logits, K, bias=None):
    """Per row: K-th largest selection score minus the (K+1)-th largest (how far from a tie
    the selection is); the score is the logit plus the selection bias, if any."""
    sc = logits.astype(np.float32) + (np.float32(0) if bias is None else bias.astype(np.float32))
    s = -np.sort(-sc.astype(np.float64), axis=1)
    if s.shape[1] <= K:
        return np.full(s.shape[0], np.inf)
    return s[:, K - 1] - s[:, K]


def lmhead_margin(h, w):
    """Per row: gap between the two largest float64 lm_head logits."""
    hf = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = np.empty((h.shape[0], w.shape[0]))
    step = 16384
    for v0 in range(0, w.shape[0], step):
        wf = (w[v0:v0 + step].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        z[:, v0:v0 + step] = hf @ wf.T
    s = -np.sort(-z, axis=1)
    return s[:, 0] - s[:, 1]


def lm_head(wl, h, w=None):
    if w is None:
        w = W.lmhead(wl)
    return lmhead_argmax(h, w)
