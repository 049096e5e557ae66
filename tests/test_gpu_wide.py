"""GPU parity at verify widths above eight rows, up to the 16-token verify
("Muse Spark Open Ultrafast", "Speculative decoding": the target checks 16
tokens in one pass).  Rows above eight take the plain top-k path (K rounds of
a wave-wide maximum per row); everything else is the same kernel as at M <= 8.
Same bars as the other parity tests.
"""
from dataclasses import replace

import numpy as np
import pytest

import moe_decode_amd as md
import oracle
from oracle import runner
from datagen import workloads as W
from datagen import device as D

from gpu_support import f32, rel_err_normwise, same_sets, say, x_tiefree
from test_gpu_parity import _check_layer, _dims, _empty, _layer_gpu, _planted_logits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [9, 12, 16])
def test_layer_tiny_wide(gpu, dw, M):
    wl = replace(W.C1, M=M)
    x = x_tiefree(W.C1, M)
    idx, out = _layer_gpu(wl, dw, gpu, x)
    _check_layer(wl, x, idx, out)


def test_layer_ling_m16(gpu, dw):
    wl = W.C12
    x = x_tiefree(wl, 16)
    idx, out = _layer_gpu(wl, dw, gpu, x)
    _check_layer(wl, x, idx, out)


def test_layer_ling_m16_fp32_partial(gpu, dw):
    wl = replace(W.C12, out_f32=True)
    x = x_tiefree(W.C12, 16)
    idx, out = _layer_gpu(wl, dw, gpu, x)
    _check_layer(wl, x, idx, out)


def test_layer_ling_fp8_m16(gpu, dw):
    import torch
    wl = W.C13
    x = x_tiefree(wl, 16)
    L = dw.layer_fp8(wl, 0)
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, 0.0, md.MOE_EXPERT_FP8_B128)
    ws = md.new_workspace(d, 16, 1)
    out = _empty((16, wl.H), torch.int16, gpu)
    idx = _empty((16, wl.K), torch.int32, gpu)
    say("layer_chain fp8 M=16")
    md.check(md.moe_layer_chain(d, 16, [md.layer_weights(L.w_router, L.w_gate_up, L.w_down,
                                                          None, None, L.s_gate_up, L.s_down)],
                                D.to_device(x), out, md.MOE_OUT_BF16, md.MOE_CHAIN_LAYER_ONLY,
                                idx, ws))
    md.check(md.moe_last_device_status(ws))
    _check_layer(wl, x, idx.cpu().numpy(), out.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("E,K", [(512, 8), (256, 16)])
def test_router_topk_planted_ties_m16(gpu, E, K):
    """Sixteen rows of exact dyadic logits with planted ties, with and without a
    selection bias: indices bit for bit."""
    import torch
    M, H = 16, 256
    rng = np.random.default_rng(2000 + E + K)
    lgt = _planted_logits(rng, M, E)
    x = np.zeros((M, H))
    w = np.zeros((E, H))
    for m in range(M):
        x[m, m] = 1.0
        w[:, m] = lgt[m]
    xb = oracle.f32_to_bf16(x.astype(np.float32)).reshape(M, H)
    wb = oracle.f32_to_bf16(w.astype(np.float32)).reshape(E, H)
    bias = (rng.integers(-4, 5, E) / 8.0).astype(np.float32)
    d = md.dims(H, E, K, 64, 0)
    ws = md.new_workspace(d, M, 1)
    for b in (None, bias):
        idx = _empty((M, K), torch.int32, gpu)
        gate = _empty((M, K), torch.float32, gpu)
        lg = _empty((M, E), torch.float32, gpu)
        say("router_topk planted ties M=16 E=%d K=%d bias=%s" % (E, K, b is not None))
        md.check(md.moe_router_topk(d, M, D.to_device(xb), D.to_device(wb),
                                    None if b is None else D.to_device(b), idx, gate, lg, ws))
        md.check(md.moe_last_device_status(ws))
        ri, rg, rl = oracle.router_topk(xb, wb, K, b)
        assert np.array_equal(lg.cpu().numpy(), rl)
        assert np.array_equal(idx.cpu().numpy(), ri)
        assert np.allclose(gate.cpu().numpy(), rg, rtol=1e-5, atol=0)


def test_experts_fused_m16_shared_experts_across_rows(gpu, dw):
    """Sixteen rows whose routing concentrates on a few experts (every slot chosen
    by several rows): the union, the row masks and the pair numbering at their widest."""
    import torch
    wl = replace(W.C1, M=16)
    x = x_tiefree(W.C1, 16)
    rng = np.random.default_rng(7)
    idx = np.stack([rng.choice(5, wl.K, replace=False) for _ in range(16)]).astype(np.int32)
    gate = rng.random((16, wl.K)).astype(np.float32)
    gu = {e: W.expert_gate_up(wl, 0, e) for e in range(wl.E + 1)}
    dn = {e: W.expert_down(wl, 0, e) for e in range(wl.E + 1)}
    ref = oracle.experts_combine(x, idx, gate, gu, dn, wl.E, 1)
    L = dw.layer(wl, 0)
    d = _dims(wl)
    ws = md.new_workspace(d, 16, 1)
    out = _empty((16, wl.H), torch.float32, gpu)
    say("experts_fused M=16 concentrated routing")
    md.check(md.moe_experts_fused(d, 16, D.to_device(x), D.to_device(idx), D.to_device(gate),
                                  md.layer_weights(None, L.w_gate_up, L.w_down), out,
                                  md.MOE_OUT_F32, ws))
    assert md.moe_last_device_status(ws) == md.MOE_OK
    assert rel_err_normwise(out.cpu().numpy(), ref) <= 1e-3


def test_chain_prenorm_tiny_m16(gpu, dw):
    import torch
    wl = replace(W.C1, M=16)
    M, NL = 16, 3
    x = x_tiefree(W.C1, M)
    layers = [md.layer_weights(dw.layer(wl, l).w_router, dw.layer(wl, l).w_gate_up,
                               dw.layer(wl, l).w_down) for l in range(NL)]
    d = _dims(wl)
    ws = md.new_workspace(d, M, NL)
    out = _empty((M, wl.H), torch.int16, gpu)
    idx = _empty((NL, M, wl.K), torch.int32, gpu)
    h_all = _empty((NL + 1, M, wl.H), torch.int16, gpu)
    say("layer_chain PRENORM_RESIDUAL L=%d M=%d" % (NL, M))
    md.check(md.moe_layer_chain(d, M, layers, D.to_device(x), out, md.MOE_OUT_BF16,
                                md.MOE_CHAIN_PRENORM_RESIDUAL, idx, ws, h_all=h_all))
    md.check(md.moe_last_device_status(ws))
    hs = h_all.cpu().numpy().view(np.uint16)
    ids = idx.cpu().numpy()
    cache = runner.ExpertCache(wl)
    exact = 0
    for l in range(NL):
        r = runner.layer(wl, oracle.rmsnorm(hs[l]), l, cache)
        clear = runner.router_margin(r["logits"], wl.K) >= 1e-3
        for m in range(M):
            if clear[m]:
                assert set(ids[l, m]) == set(r["idx"][m]), (l, m)
                exact += 1
        rows = np.nonzero(clear)[0]
        assert rel_err_normwise(f32(hs[l + 1][rows]),
                                f32(oracle.residual(hs[l], r["acc"])[rows])) <= 1e-2
    assert exact >= 0.8 * NL * M


@pytest.mark.parametrize("V", [1, 20001])
def test_lmhead_m16(gpu, V):
    import torch
    M, wl = 16, W.C5
    rng = np.random.default_rng(V)
    h = W.x_rows(wl, list(range(M)))
    w = W.lmhead_rows(wl, 0, V).copy()
    if V > 100:
        w[V - 3] = w[17]          # planted tie: index 17 must win if it is the maximum
    ws = md.new_workspace(_dims(wl), M, 1)
    tok = _empty((M,), torch.int32, gpu)
    mx = _empty((M,), torch.float32, gpu)
    say("lmhead_argmax M=16 V=%d" % V)
    md.check(md.lmhead_argmax(M, wl.H, V, D.to_device(h), D.to_device(w), tok, mx, ws))
    md.check(md.moe_last_device_status(ws))
    t_ref, m_ref = oracle.lmhead_argmax(h, w)
    marg = runner.lmhead_margin(h, w) if V > 1 else np.full(M, np.inf)
    got = tok.cpu().numpy()
    for m in range(M):
        if marg[m] >= 1e-4 or V == 1:
            assert got[m] == t_ref[m], (m, got[m], t_ref[m])
    assert np.all(np.abs(mx.cpu().numpy() - m_ref) <= 1e-4 * np.abs(m_ref) + 1e-5)


@pytest.mark.parametrize("wl,M,V", [(W.C5, 3, 4097), (W.C5, 6, 20001), (W.C5, 9, 4097),
                                    (W.C5, 12, 157), (W.C1, 4, 33), (W.C1, 12, 1000),
                                    (W.C1, 16, 17)])
def test_lmhead_matrix_cores_ragged(gpu, wl, M, V):
    """From 3 token rows the lm_head runs on the matrix cores (16-row tiles):
    ragged vocabularies (a partial last tile), hidden sizes of 40 and 4
    super-chunks, and a planted exact tie that the lower index must win."""
    import torch
    h = W.x_rows(wl, list(range(M)))
    w = W.lmhead_rows(wl, 0, V).copy()
    z = f32(h[0]).astype(np.float64) @ f32(w).astype(np.float64).T
    best = int(np.argmax(z))
    w[V - 1] = w[best]          # exact duplicate of row 0's winner at the highest index
    ws = md.new_workspace(_dims(wl), M, 1)
    tok = _empty((M,), torch.int32, gpu)
    mx = _empty((M,), torch.float32, gpu)
    say("lmhead_argmax matrix cores %s M=%d V=%d" % (wl.name, M, V))
    md.check(md.lmhead_argmax(M, wl.H, V, D.to_device(h), D.to_device(w), tok, mx, ws))
    md.check(md.moe_last_device_status(ws))
    t_ref, m_ref = oracle.lmhead_argmax(h, w)
    marg = runner.lmhead_margin(h, w)
    got = tok.cpu().numpy()
    assert got[0] == t_ref[0] == min(best, V - 1)
    for m in range(M):
        if marg[m] >= 1e-4:
            assert got[m] == t_ref[m], (m, got[m], t_ref[m])
    assert np.all(np.abs(mx.cpu().numpy() - m_ref) <= 1e-4 * np.abs(m_ref) + 1e-5)
