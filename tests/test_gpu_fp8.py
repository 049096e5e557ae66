"""GPU parity of the fp8 expert path: e4m3 codes with one fp32 scale per
128 x 128 block ("Ling-3.0-flash on 4 Blackwell GPUs", "Where the time goes
now": fp8 weights with block-128 quantisation), bf16 router and activations.

Same bars as the bf16 layer: expert indices bit-exact on tie-free inputs, bf16
outputs within a norm-wise relative error of 1e-2 of the oracle (which
dequantises every weight exactly and rounds it once to fp32), fp32 outputs
within 1e-3.
"""
from dataclasses import replace

import numpy as np
import pytest

import moe_decode_amd as md
import oracle
from oracle import runner
from datagen import workloads as W
from datagen import device as D

from gpu_support import (f32, free_running_report, frac_beyond_one_ulp, order_agrees,
                         rel_err_normwise, same_sets, say, x_tiefree)

pytestmark = pytest.mark.gpu


def _dims(wl, **kw):
    a = dict(hidden=wl.H, n_experts=wl.E, top_k=wl.K, inter=wl.I, n_shared=wl.S,
             routed_scale=wl.routed_scale, expert_format=md.MOE_EXPERT_FP8_B128)
    a.update(kw)
    return md.dims(**a)


def _lw(L, bias=None, gain=None):
    return md.layer_weights(L.w_router, L.w_gate_up, L.w_down, bias, gain, L.s_gate_up, L.s_down)


def _empty(shape, dtype, dev):
    import torch
    return torch.empty(shape, dtype=dtype, device=dev)


def _layer_gpu(wl, dw, gpu, x, out_f32=False, mode=None, lw=None):
    import torch
    M = x.shape[0]
    d = _dims(wl)
    lw = _lw(dw.layer_fp8(wl, 0)) if lw is None else lw
    ws = md.new_workspace(d, M, 1)
    out = _empty((M, wl.H), torch.float32 if out_f32 else torch.int16, gpu)
    idx = _empty((M, wl.K), torch.int32, gpu)
    mode = md.MOE_CHAIN_LAYER_ONLY if mode is None else mode
    say("layer_chain fp8 mode=%d %s M=%d f32=%s" % (mode, wl.name, M, out_f32))
    md.check(md.moe_layer_chain(d, M, [lw], D.to_device(x), out,
                                md.MOE_OUT_F32 if out_f32 else md.MOE_OUT_BF16, mode, idx, ws))
    md.check(md.moe_last_device_status(ws))
    o = out.cpu().numpy()
    return idx.cpu().numpy(), (o if out_f32 else o.view(np.uint16))


def _check(wl, ref, idx, out, out_f32):
    assert same_sets(idx, ref["idx"]), (idx, ref["idx"])
    assert order_agrees(idx, ref["idx"], ref["logits"])
    if out_f32:
        err = rel_err_normwise(out, ref["acc"])
        assert err <= 1e-3, err
    else:
        ref_out = oracle.cast_bf16(ref["acc"])
        err = rel_err_normwise(f32(out), f32(ref_out))
        assert err <= 1e-2, err
        assert frac_beyond_one_ulp(out, ref_out) <= 0.01


def test_fp8_device_generator_matches_host(gpu, dw):
    say("datagen fp8 device vs host")
    for wl in (W.C8, W.C10):
        L = dw.layer_fp8(wl, 0)
        for e in (0, 5, wl.E):
            q, s = W.expert_gate_up_fp8(wl, 0, e)
            assert np.array_equal(L.w_gate_up[e].cpu().numpy(), q)
            assert np.array_equal(L.s_gate_up[e].cpu().numpy(), s)
            q, s = W.expert_down_fp8(wl, 0, e)
            assert np.array_equal(L.w_down[e].cpu().numpy(), q)
            assert np.array_equal(L.s_down[e].cpu().numpy(), s)


@pytest.mark.parametrize("M", [1, 2, 3])
@pytest.mark.parametrize("out_f32", [False, True])
def test_fp8_layer_tiny(gpu, dw, M, out_f32):
    wl = W.C8
    x = x_tiefree(wl, M)
    idx, out = _layer_gpu(wl, dw, gpu, x, out_f32)
    _check(wl, runner.layer(wl, x), idx, out, out_f32)


@pytest.mark.parametrize("wl,M", [(W.C9, 1), (W.C10, 6), (W.C10, 8)])
def test_fp8_layer_ling(gpu, dw, wl, M):
    x = x_tiefree(wl, M)
    wlm = replace(wl, M=M)
    idx, out = _layer_gpu(wlm, dw, gpu, x)
    _check(wlm, runner.layer(wlm, x), idx, out, False)


def test_fp8_layer_ling_fp32_partial(gpu, dw):
    wl = W.C10
    x = x_tiefree(wl, 6)
    idx, out = _layer_gpu(wl, dw, gpu, x, out_f32=True)
    _check(wl, runner.layer(wl, x), idx, out, True)


def test_fp8_experts_fused_duplicate_indices(gpu, dw):
    import torch
    wl = W.C8
    x = x_tiefree(wl, 3)
    idx = np.array([[3, 3], [5, 9], [0, 15]], np.int32)
    gate = np.array([[0.25, 0.75], [0.6, 0.4], [0.5, 0.5]], np.float32)
    gu = {e: W.expert_gate_up_fp8(wl, 0, e) for e in range(wl.E + 1)}
    dn = {e: W.expert_down_fp8(wl, 0, e) for e in range(wl.E + 1)}
    ref = oracle.experts_combine_fp8(x, idx, gate, gu, dn, wl.E, 1)
    d = _dims(wl)
    ws = md.new_workspace(d, 3, 1)
    out = _empty((3, wl.H), torch.float32, gpu)
    L = dw.layer_fp8(wl, 0)
    say("experts_fused fp8 tiny duplicates")
    md.check(md.moe_experts_fused(d, 3, D.to_device(x), D.to_device(idx), D.to_device(gate),
                                  md.layer_weights(None, L.w_gate_up, L.w_down, None, None,
                                                   L.s_gate_up, L.s_down),
                                  out, md.MOE_OUT_F32, ws))
    assert md.moe_last_device_status(ws) == md.MOE_OK
    assert rel_err_normwise(out.cpu().numpy(), ref) <= 1e-3


def test_fp8_experts_fused_ling_with_oracle_routing(gpu, dw):
    import torch
    wl = W.C10
    x = x_tiefree(wl, 6)
    ref = runner.layer(wl, x)
    d = _dims(wl)
    ws = md.new_workspace(d, 6, 1)
    out = _empty((6, wl.H), torch.int16, gpu)
    L = dw.layer_fp8(wl, 0)
    say("experts_fused fp8 ling M=6")
    md.check(md.moe_experts_fused(d, 6, D.to_device(x), D.to_device(ref["idx"]),
                                  D.to_device(ref["gate"]), _lw(L), out, md.MOE_OUT_BF16, ws))
    assert md.moe_last_device_status(ws) == md.MOE_OK
    o = out.cpu().numpy().view(np.uint16)
    assert rel_err_normwise(f32(o), f32(oracle.cast_bf16(ref["acc"]))) <= 1e-2


def test_fp8_with_router_front(gpu, dw):
    """fp8 experts behind the fused router front (norm gain, selection bias, routed scale)."""
    wl = replace(W.C8, prenorm=True, bias_sigma=0.25, gain_sigma=0.1, routed_scale=2.5)
    x = x_tiefree(W.C8, 3)
    L = dw.layer_fp8(wl, 0)
    bias = D.to_device(W.router_bias(wl, 0))
    gain = D.to_device(W.norm_gain(wl, 0))
    idx, out = _layer_gpu(wl, dw, gpu, x, mode=md.MOE_CHAIN_PRENORM_LAYER_ONLY,
                          lw=_lw(L, bias, gain))
    ref = runner.front_layer(wl, x)
    sc = ref["logits"].astype(np.float32) + W.router_bias(wl, 0)
    clear = runner.router_margin(ref["logits"], wl.K, W.router_bias(wl, 0)) >= 1e-3
    assert clear.sum() >= 2
    assert same_sets(idx[clear], ref["idx"][clear])
    assert order_agrees(idx[clear], ref["idx"][clear], sc[clear])
    rows = np.nonzero(clear)[0]
    assert rel_err_normwise(f32(out[rows]), f32(oracle.cast_bf16(ref["acc"])[rows])) <= 1e-2


def test_fp8_chain_tiny_teacher_forced(gpu, dw):
    import torch
    wl = replace(W.C8, n_layers=3, residual=True)
    M, NL = 4, 3
    x = x_tiefree(W.C8, M)
    layers = [_lw(dw.layer_fp8(wl, l)) for l in range(NL)]
    d = _dims(wl)
    ws = md.new_workspace(d, M, NL)
    out = _empty((M, wl.H), torch.int16, gpu)
    idx = _empty((NL, M, wl.K), torch.int32, gpu)
    h_all = _empty((NL + 1, M, wl.H), torch.int16, gpu)
    say("layer_chain fp8 RESIDUAL L=%d M=%d" % (NL, M))
    md.check(md.moe_layer_chain(d, M, layers, D.to_device(x), out, md.MOE_OUT_BF16,
                                md.MOE_CHAIN_RESIDUAL, idx, ws, h_all=h_all))
    md.check(md.moe_last_device_status(ws))
    hs = h_all.cpu().numpy().view(np.uint16)
    ids = idx.cpu().numpy()
    cache = runner.ExpertCache(wl)
    exact = 0
    for l in range(NL):
        r = runner.layer(wl, hs[l], l, cache)
        clear = runner.router_margin(r["logits"], wl.K) >= 1e-3
        for m in range(M):
            if clear[m]:
                assert set(ids[l, m]) == set(r["idx"][m]), (l, m)
                exact += 1
        rows = np.nonzero(clear)[0]
        ref_next = oracle.residual(hs[l], r["acc"])
        assert rel_err_normwise(f32(hs[l + 1][rows]), f32(ref_next[rows])) <= 1e-2
    assert exact >= 0.75 * NL * M


def test_fp8_chain16_lmhead_full_size(gpu, dw):
    """The 16-layer Ling chain with fp8 experts at M=6 (pre-norm residual, one launch),
    then the lm_head argmax: every layer checked against the oracle on the GPU's own
    input to it, and the tokens equal to the oracle's argmax of the final hidden state."""
    import torch
    wl = W.C11
    M, NL = 6, wl.n_layers
    x = x_tiefree(wl, M)
    layers = [_lw(dw.layer_fp8(wl, l)) for l in range(NL)]
    d = _dims(wl)
    ws = md.new_workspace(d, M, NL)
    out = _empty((M, wl.H), torch.int16, gpu)
    idx = _empty((NL, M, wl.K), torch.int32, gpu)
    h_all = _empty((NL + 1, M, wl.H), torch.int16, gpu)
    say("layer_chain fp8 PRENORM_RESIDUAL L=%d M=%d" % (NL, M))
    md.check(md.moe_layer_chain(d, M, layers, D.to_device(x), out, md.MOE_OUT_BF16,
                                md.MOE_CHAIN_PRENORM_RESIDUAL, idx, ws, h_all=h_all))
    md.check(md.moe_last_device_status(ws))
    hs = h_all.cpu().numpy().view(np.uint16)
    h = out.cpu().numpy().view(np.uint16)
    ids = idx.cpu().numpy()
    assert np.array_equal(hs[0], x) and np.array_equal(hs[NL], h)
    cache = runner.ExpertCache(wl)
    exact = 0
    for l in range(NL):
        u = oracle.rmsnorm(hs[l])
        r = runner.layer(wl, u, l, cache)
        clear = runner.router_margin(r["logits"], wl.K) >= 1e-3
        for m in range(M):
            if clear[m]:
                assert set(ids[l, m]) == set(r["idx"][m]), (l, m)
                exact += 1
        rows = np.nonzero(clear)[0]
        ref_next = oracle.residual(hs[l], r["acc"])
        assert rel_err_normwise(f32(hs[l + 1][rows]), f32(ref_next[rows])) <= 1e-2, l
        cache.drop_layer(l)
    assert exact >= 0.9 * NL * M
    lm = dw.lmhead(wl)
    tok = _empty((M,), torch.int32, gpu)
    say("lmhead_argmax V=%d M=%d on the fp8 chain output" % (wl.V, M))
    md.check(md.lmhead_argmax(M, wl.H, wl.V, D.to_device(h), lm, tok, None, ws))
    w_host = D.from_device_bf16(lm)
    t_ref, _ = oracle.lmhead_argmax(h, w_host)
    marg = runner.lmhead_margin(h, w_host)
    got = tok.cpu().numpy()
    for m in range(M):
        if marg[m] >= 1e-4:
            assert got[m] == t_ref[m], (m, got[m], t_ref[m])
    # the free-running comparison with the oracle's own 16-layer chain: reported only
    rep = free_running_report(wl, x, ids, h, got, w_host)
    assert len(rep["rows"]) == M
