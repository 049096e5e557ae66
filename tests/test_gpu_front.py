"""GPU parity of the router front: RMSNorm with a gain vector in front of the
router and the experts, a per-expert selection bias, and the routed scaling
factor of the combine ("Ling-3.0-flash on 4 Blackwell GPUs", "PDL: stacking
the latency floors of small kernels": the router chain opens with a norm, the
top-k loads a bias of its own, and the small-M combine scales an fp32 sum).

Same bars as the plain layer: expert sets bit-exact on inputs whose K-th and
(K+1)-th selection scores (logit + bias) are at least 1e-3 apart, bf16 outputs
within a norm-wise relative error of 1e-2, fp32 outputs within 1e-3.
"""
from dataclasses import replace

import numpy as np
import pytest

import moe_decode_amd as md
import oracle
from oracle import runner
from datagen import workloads as W
from datagen import device as D

from gpu_support import f32, frac_beyond_one_ulp, order_agrees, rel_err_normwise, same_sets, say
from gpu_support import x_tiefree

pytestmark = pytest.mark.gpu


def _dims(wl, **kw):
    a = dict(hidden=wl.H, n_experts=wl.E, top_k=wl.K, inter=wl.I, n_shared=wl.S,
             routed_scale=wl.routed_scale)
    a.update(kw)
    return md.dims(**a)


def _empty(shape, dtype, dev):
    import torch
    return torch.empty(shape, dtype=dtype, device=dev)


class _Front:
    """Device weights of one layer with its front vectors (kept alive with the struct)."""

    def __init__(self, wl, dw, l=0, bias=True, gain=True):
        L = dw.layer(wl, l)
        b = W.router_bias(wl, l) if bias else None
        g = W.norm_gain(wl, l) if gain else None
        self.bias = None if b is None else D.to_device(b)
        self.gain = None if g is None else D.to_device(g)
        self.lw = md.layer_weights(L.w_router, L.w_gate_up, L.w_down, self.bias, self.gain)
        self.L = L


def _front_gpu(wl, dw, gpu, x, out_f32=False, inplace=False, mode=None, fr=None):
    """One layer through moe_layer_chain(PRENORM_LAYER_ONLY): returns (idx, out)."""
    import torch
    M = x.shape[0]
    d = _dims(wl)
    fr = _Front(wl, dw) if fr is None else fr
    mode = md.MOE_CHAIN_PRENORM_LAYER_ONLY if mode is None else mode
    ws = md.new_workspace(d, M, 1)
    xin = D.to_device(x)
    if inplace:
        assert not out_f32
        out = xin
    else:
        out = _empty((M, wl.H), torch.float32 if out_f32 else torch.int16, gpu)
    idx = _empty((M, wl.K), torch.int32, gpu)
    say("layer_chain mode=%d %s M=%d f32=%s inplace=%s" % (mode, wl.name, M, out_f32, inplace))
    md.check(md.moe_layer_chain(d, M, [fr.lw], xin, out,
                                md.MOE_OUT_F32 if out_f32 else md.MOE_OUT_BF16, mode, idx, ws))
    md.check(md.moe_last_device_status(ws))
    o = out.cpu().numpy()
    return idx.cpu().numpy(), (o if out_f32 else o.view(np.uint16))


def _scores(wl, logits, l=0):
    b = W.router_bias(wl, l)
    return logits if b is None else logits.astype(np.float32) + b


def _check_front(wl, x, idx_g, out_g, out_f32):
    ref = runner.front_layer(wl, x)
    assert same_sets(idx_g, ref["idx"]), (idx_g, ref["idx"])
    assert order_agrees(idx_g, ref["idx"], _scores(wl, ref["logits"]))
    if out_f32:
        err = rel_err_normwise(out_g, ref["acc"])
        assert err <= 1e-3, err
    else:
        ref_out = oracle.cast_bf16(ref["acc"])
        err = rel_err_normwise(f32(out_g), f32(ref_out))
        assert err <= 1e-2, err
        assert frac_beyond_one_ulp(out_g, ref_out) <= 0.01
    return ref


# ------------------------------------------------------------------ selection bias

def _planted(rng, M, E):
    """Dyadic logits and biases whose sums tie often (every value exact in fp32)."""
    lg = rng.integers(-8, 9, (M, E)) / 8.0
    b = rng.integers(-4, 5, E) / 8.0
    b[:E // 8] = 4.0                     # a block of experts lifted above every row's logits
    return lg, b.astype(np.float32)


@pytest.mark.parametrize("E,K,M", [(16, 2, 3), (512, 8, 1), (512, 8, 6), (1024, 8, 4),
                                   (256, 16, 8)])
def test_router_bias_planted_ties_exact(gpu, E, K, M):
    """Selection on fp32(logit + bias), lower index among equal scores, in the
    fast and the plain selection paths; gates from the unbiased logits."""
    import torch
    rng = np.random.default_rng(1000 + E + M)
    H = 256
    lgt, b = _planted(rng, M, E)
    x = np.zeros((M, H))
    w = np.zeros((E, H))
    for m in range(M):
        x[m, m] = 1.0
        w[:, m] = lgt[m]
    xb = oracle.f32_to_bf16(x.astype(np.float32)).reshape(M, H)
    wb = oracle.f32_to_bf16(w.astype(np.float32)).reshape(E, H)
    d = md.dims(H, E, K, 64, 0)
    ws = md.new_workspace(d, M, 1)
    idx = _empty((M, K), torch.int32, gpu)
    gate = _empty((M, K), torch.float32, gpu)
    lg = _empty((M, E), torch.float32, gpu)
    say("router_topk bias planted E=%d K=%d M=%d" % (E, K, M))
    md.check(md.moe_router_topk(d, M, D.to_device(xb), D.to_device(wb), D.to_device(b), idx,
                                gate, lg, ws))
    md.check(md.moe_last_device_status(ws))
    ri, rg, rl = oracle.router_topk(xb, wb, K, b)
    assert np.array_equal(lg.cpu().numpy(), rl)            # logits come out unbiased
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.allclose(gate.cpu().numpy(), rg, rtol=1e-5, atol=0)
    # the bias really moved the selection
    r0, _, _ = oracle.router_topk(xb, wb, K)
    assert not np.array_equal(np.sort(ri, 1), np.sort(r0, 1))


@pytest.mark.parametrize("E,K", [(16, 2), (200, 5), (512, 8)])
def test_layer_one_row_planted_ties_exact(gpu, E, K):
    """One token row through the fused layer, where every wave selects the row
    on its own: with planted ties and a bias the selection (and its order) is
    exactly the oracle's; zero experts make the layer's output exactly zero."""
    import torch
    rng = np.random.default_rng(3000 + E)
    H, I = 256, 64
    lgt, b = _planted(rng, 1, E)
    x = np.zeros((1, H))
    w = np.zeros((E, H))
    x[0, 0] = 1.0
    w[:, 0] = lgt[0]
    xb = oracle.f32_to_bf16(x.astype(np.float32)).reshape(1, H)
    wb = oracle.f32_to_bf16(w.astype(np.float32)).reshape(E, H)
    d = md.dims(H, E, K, I, 1)
    ws = md.new_workspace(d, 1, 1)
    # every expert weight tensor holds E routed + S shared experts ([E+S][2I][H], [E+S][H][I])
    gu = torch.zeros((E + 1, 2 * I, H), dtype=torch.int16, device=gpu)
    dn = torch.zeros((E + 1, H, I), dtype=torch.int16, device=gpu)
    assert gu.shape[0] == E + d.n_shared and dn.shape[0] == E + d.n_shared
    # (layer_weights holds the tensors too; named here so the dependency is plain)
    wr, bias = D.to_device(wb), D.to_device(b)
    lw = md.layer_weights(wr, gu, dn, bias)
    out = _empty((1, H), torch.int16, gpu)
    idx = _empty((1, K), torch.int32, gpu)
    say("layer_chain one row, bias planted E=%d K=%d" % (E, K))
    md.check(md.moe_layer_chain(d, 1, [lw], D.to_device(xb), out, md.MOE_OUT_BF16,
                                md.MOE_CHAIN_LAYER_ONLY, idx, ws))
    md.check(md.moe_last_device_status(ws))
    ri, _, _ = oracle.router_topk(xb, wb, K, b)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert not out.cpu().numpy().any()


@pytest.mark.parametrize("wl,M", [(W.C7, 6), (W.C7, 1), (W.C6, 3)])
def test_router_bias_on_normed_rows(gpu, dw, wl, M):
    """The router alone on the normed input u (tie-free on the biased scores)."""
    import torch
    x = x_tiefree(wl, M)
    u = oracle.rmsnorm(x, gain=W.norm_gain(wl, 0))
    fr = _Front(wl, dw)
    d = _dims(wl)
    ws = md.new_workspace(d, M, 1)
    idx = _empty((M, wl.K), torch.int32, gpu)
    gate = _empty((M, wl.K), torch.float32, gpu)
    say("router_topk bias %s M=%d" % (wl.name, M))
    md.check(md.moe_router_topk(d, M, D.to_device(u), fr.L.w_router, fr.bias, idx, gate, None,
                                ws))
    md.check(md.moe_last_device_status(ws))
    ri, rg, rl = oracle.router_topk(u, W.router(wl, 0), wl.K, W.router_bias(wl, 0))
    gi, gg = idx.cpu().numpy(), gate.cpu().numpy()
    assert same_sets(gi, ri) and order_agrees(gi, ri, _scores(wl, rl))
    for m in range(M):
        ref = dict(zip(ri[m], rg[m]))
        for k in range(wl.K):
            assert abs(gg[m, k] - ref[gi[m, k]]) <= 1e-5 * ref[gi[m, k]]


# ------------------------------------------------------------------ fused front layer

@pytest.mark.parametrize("M", [1, 2, 3])
@pytest.mark.parametrize("out_f32", [False, True])
def test_front_layer_tiny(gpu, dw, M, out_f32):
    wl = W.C6
    x = x_tiefree(wl, M)
    idx, out = _front_gpu(wl, dw, gpu, x, out_f32=out_f32)
    _check_front(wl, x, idx, out, out_f32)


@pytest.mark.parametrize("M", [1, 6, 8])
def test_front_layer_ling(gpu, dw, M):
    wl = replace(W.C7, M=M)
    x = x_tiefree(W.C7, M)
    idx, out = _front_gpu(wl, dw, gpu, x)
    _check_front(wl, x, idx, out, False)


def test_front_layer_ling_fp32_partial(gpu, dw):
    wl = W.C7
    x = x_tiefree(wl, 6)
    idx, out = _front_gpu(wl, dw, gpu, x, out_f32=True)
    _check_front(wl, x, idx, out, True)


def test_fused_norm_equals_oracle_norm_bit_for_bit(gpu, dw):
    """The fused norm (with gain) feeds the rest of the layer exactly the bf16
    input the oracle's norm computes: the norm-fused call and the plain call on
    the oracle's normed rows return identical bits."""
    wl = W.C7
    x = x_tiefree(wl, 6)
    fr = _Front(wl, dw)
    idx_a, out_a = _front_gpu(wl, dw, gpu, x, fr=fr)
    u = oracle.rmsnorm(x, gain=W.norm_gain(wl, 0))
    idx_b, out_b = _front_gpu(wl, dw, gpu, u, fr=fr, mode=md.MOE_CHAIN_LAYER_ONLY)
    assert np.array_equal(idx_a, idx_b)
    assert np.array_equal(out_a, out_b)


def test_front_layer_inplace(gpu, dw):
    wl = W.C6
    x = x_tiefree(wl, 3)
    idx_a, out_a = _front_gpu(wl, dw, gpu, x)
    idx_b, out_b = _front_gpu(wl, dw, gpu, x, inplace=True)
    assert np.array_equal(idx_a, idx_b) and np.array_equal(out_a, out_b)


def test_front_without_bias_or_gain_is_the_plain_prenorm_layer(gpu, dw):
    """NULL bias and NULL gain: the unit-gain norm and plain selection."""
    wl = replace(W.C6, bias_sigma=0.0, gain_sigma=0.0)
    x = x_tiefree(W.C1, 3)
    fr = _Front(wl, dw, bias=False, gain=False)
    idx, out = _front_gpu(wl, dw, gpu, x, fr=fr)
    ref = runner.front_layer(wl, x)
    clear = runner.router_margin(ref["logits"], wl.K) >= 1e-3   # rows tie-free on u
    assert clear.sum() >= 2
    assert same_sets(idx[clear], ref["idx"][clear])
    rows = np.nonzero(clear)[0]
    assert rel_err_normwise(f32(out[rows]), f32(oracle.cast_bf16(ref["acc"])[rows])) <= 1e-2


# ------------------------------------------------------------------ routed scale

@pytest.mark.parametrize("out_f32", [False, True])
def test_experts_fused_routed_scale(gpu, dw, out_f32):
    """moe_experts_fused with a routed scaling factor (bias and gain are ignored there)."""
    import torch
    wl = replace(W.C3, routed_scale=2.5)
    x = x_tiefree(W.C3, 6)
    ref = runner.layer(wl, x)
    fr = _Front(W.C7, dw)                     # bias and gain set: must be ignored
    d = _dims(wl)
    ws = md.new_workspace(d, 6, 1)
    out = _empty((6, wl.H), torch.float32 if out_f32 else torch.int16, gpu)
    say("experts_fused routed_scale=2.5 f32=%s" % out_f32)
    md.check(md.moe_experts_fused(d, 6, D.to_device(x), D.to_device(ref["idx"]),
                                  D.to_device(ref["gate"]), fr.lw, out,
                                  md.MOE_OUT_F32 if out_f32 else md.MOE_OUT_BF16, ws))
    md.check(md.moe_last_device_status(ws))
    o = out.cpu().numpy()
    if out_f32:
        assert rel_err_normwise(o, ref["acc"]) <= 1e-3
    else:
        assert rel_err_normwise(f32(o.view(np.uint16)), f32(oracle.cast_bf16(ref["acc"]))) <= 1e-2
    # and the scale matters: the unscaled combine is far from it
    plain = runner.layer(W.C3, x)["acc"]
    assert rel_err_normwise(plain, ref["acc"]) > 0.05


# ------------------------------------------------------------------ chain with the front

def _valid_selection(sel, scores, K, tol=1e-3):
    srt = -np.sort(-scores.astype(np.float64))
    kth = srt[K - 1]
    must = set(np.nonzero(scores > kth + tol)[0].tolist())
    may = set(np.nonzero(scores >= kth - tol)[0].tolist())
    s = set(int(e) for e in sel)
    return len(s) == K and must <= s <= may


def test_chain_front_tiny_teacher_forced(gpu, dw):
    """Four pre-norm residual layers, each with its own gain, bias and the routed
    scale; every layer is checked against the oracle on the GPU's own input to it."""
    import torch
    wl = replace(W.C6, n_layers=4, residual=True, M=8)
    M, NL = 8, 4
    x = x_tiefree(W.C1, M)
    fronts = [_Front(wl, dw, l) for l in range(NL)]
    d = _dims(wl)
    ws = md.new_workspace(d, M, NL)
    out = _empty((M, wl.H), torch.int16, gpu)
    idx = _empty((NL, M, wl.K), torch.int32, gpu)
    h_all = _empty((NL + 1, M, wl.H), torch.int16, gpu)
    say("layer_chain front PRENORM_RESIDUAL L=%d M=%d" % (NL, M))
    md.check(md.moe_layer_chain(d, M, [f.lw for f in fronts], D.to_device(x), out,
                                md.MOE_OUT_BF16, md.MOE_CHAIN_PRENORM_RESIDUAL, idx, ws,
                                h_all=h_all))
    md.check(md.moe_last_device_status(ws))
    hs = h_all.cpu().numpy().view(np.uint16)
    ids = idx.cpu().numpy()
    assert np.array_equal(hs[0], x) and np.array_equal(hs[NL], out.cpu().numpy().view(np.uint16))
    cache = runner.ExpertCache(wl)
    exact = 0
    for l in range(NL):
        u = oracle.rmsnorm(hs[l], gain=W.norm_gain(wl, l))
        r = runner.layer(wl, u, l, cache)
        sc = _scores(wl, r["logits"], l)
        clear = runner.router_margin(r["logits"], wl.K, W.router_bias(wl, l)) >= 1e-3
        for m in range(M):
            if clear[m]:
                assert set(ids[l, m]) == set(r["idx"][m]), (l, m)
                exact += 1
            else:
                assert _valid_selection(ids[l, m], sc[m], wl.K), (l, m)
        ref_next = oracle.residual(hs[l], r["acc"])
        rows = np.nonzero(clear)[0]
        assert rel_err_normwise(f32(hs[l + 1][rows]), f32(ref_next[rows])) <= 1e-2
    assert exact >= 0.8 * NL * M
