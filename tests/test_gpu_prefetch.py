"""GPU checks of the speculative expert prefetch ("Muse Spark Open Ultrafast:
Pushing beyond 1,000 Tokens per second", Megakernel internals: speculative
expert prefetching).

The prefetch only reads.  A layer call gives bit-identical results with and
without a prefetch in front of it, whatever the list holds: the experts the
layer then picks, wrong guesses, duplicates, the shared expert, and ids outside
[0, E+S), which are skipped.  The weights it read stay as they were, and the
prefetched call still agrees with the oracle to the layer's own bars.
"""
import numpy as np
import pytest

import moe_decode_amd as md
from oracle import runner
from datagen import workloads as W

from gpu_support import f32, rel_err_normwise, same_sets, say, x_tiefree

pytestmark = pytest.mark.gpu


def _setup(wl, dw):
    fp8 = wl.fp8
    L = dw.layer_fp8(wl, 0) if fp8 else dw.layer(wl, 0)
    d = md.dims(hidden=wl.H, n_experts=wl.E, top_k=wl.K, inter=wl.I, n_shared=wl.S,
                expert_format=md.MOE_EXPERT_FP8_B128 if fp8 else md.MOE_EXPERT_BF16)
    lw = md.layer_weights(L.w_router, L.w_gate_up, L.w_down, None, None, L.s_gate_up, L.s_down)
    return L, d, lw


def _layer(d, lw, x, out, idx, ws, M):
    md.check(md.moe_layer_chain(d, M, [lw], x, out, md.MOE_OUT_BF16, md.MOE_CHAIN_LAYER_ONLY,
                                idx, ws))


def _ids(gpu, vals):
    import torch
    return torch.tensor(np.asarray(vals, dtype=np.int32), device=gpu)


@pytest.mark.parametrize("wl", [W.C1, W.C2, W.C9, W.C3], ids=lambda w: w.name)
def test_prefetch_leaves_layer_results_bit_identical(gpu, dw, wl):
    import torch
    from datagen import device as D
    M = wl.M
    L, d, lw = _setup(wl, dw)
    x_host = x_tiefree(wl, M)
    x = D.to_device(x_host)
    ws = md.new_workspace(d, M, 1)
    out0 = torch.empty((M, wl.H), dtype=torch.int16, device=gpu)
    out1 = torch.empty_like(out0)
    idx0 = torch.empty((M, wl.K), dtype=torch.int32, device=gpu)
    idx1 = torch.empty_like(idx0)
    say("prefetch: layer without prefetch %s M=%d" % (wl.name, M))
    _layer(d, lw, x, out0, idx0, ws, M)
    md.check(md.moe_last_device_status(ws))
    chosen = np.unique(idx0.cpu().numpy())
    # right guesses, a wrong one, a duplicate, the shared expert, and ids to skip
    wrong = int(np.setdiff1d(np.arange(wl.E), chosen)[0])
    vals = list(chosen) + [wrong, int(chosen[0]), wl.E, -1, wl.E + wl.S, 1 << 30, -(1 << 31)]
    valid = sorted(set(v for v in vals if 0 <= v < wl.E + wl.S))
    snap = [(e, L.w_gate_up[e].clone(), L.w_down[e].clone()) for e in valid]
    ids = _ids(gpu, vals)
    say("prefetch: %d ids then the same layer %s" % (len(vals), wl.name))
    md.check(md.moe_expert_prefetch(d, lw, ids, len(vals)))
    _layer(d, lw, x, out1, idx1, ws, M)
    md.check(md.moe_last_device_status(ws))
    assert torch.equal(idx0, idx1)
    assert torch.equal(out0, out1)
    for e, g, dn in snap:
        assert torch.equal(L.w_gate_up[e], g), e
        assert torch.equal(L.w_down[e], dn), e
    if not wl.fp8:
        # the prefetched call against the oracle, to the layer's own bars
        ref = runner.layer(wl, x_host)
        assert same_sets(idx1.cpu().numpy(), ref["idx"])
        got = out1.cpu().numpy().view(np.uint16)
        assert rel_err_normwise(f32(got), f32(runner.layer_output(wl, ref))) <= 1e-2


def test_prefetch_longest_list(gpu, dw):
    """MOE_MAX_PREFETCH_IDS ids, most of them out of range: every expert of the
    tiny layer is read many times over and nothing changes."""
    import torch
    from datagen import device as D
    wl = W.C1
    M = 3
    L, d, lw = _setup(wl, dw)
    x = D.to_device(x_tiefree(wl, M))
    ws = md.new_workspace(d, M, 1)
    out0 = torch.empty((M, wl.H), dtype=torch.int16, device=gpu)
    out1 = torch.empty_like(out0)
    idx = torch.empty((M, wl.K), dtype=torch.int32, device=gpu)
    say("prefetch: tiny layer M=3 without prefetch")
    _layer(d, lw, x, out0, idx, ws, M)
    n = md.MOE_MAX_PREFETCH_IDS
    vals = (np.arange(n, dtype=np.int64) % (3 * (wl.E + wl.S))) - (wl.E + wl.S)
    gu, dn = L.w_gate_up.clone(), L.w_down.clone()
    say("prefetch: %d ids, then the layer" % n)
    md.check(md.moe_expert_prefetch(d, lw, _ids(gpu, vals), n))
    _layer(d, lw, x, out1, idx, ws, M)
    md.check(md.moe_last_device_status(ws))
    assert torch.equal(out0, out1)
    assert torch.equal(L.w_gate_up, gu) and torch.equal(L.w_down, dn)


def test_prefetch_whole_ling_layer_on_a_side_stream(gpu, dw):
    """Every expert of a Ling layer listed once, on a stream of its own (the way a
    caller overlaps it with other work), then the layer on the current stream
    after an event: same result as without."""
    import torch
    from datagen import device as D
    wl = W.C2
    L, d, lw = _setup(wl, dw)
    x = D.to_device(x_tiefree(wl, 1))
    ws = md.new_workspace(d, 1, 1)
    out0 = torch.empty((1, wl.H), dtype=torch.int16, device=gpu)
    out1 = torch.empty_like(out0)
    idx = torch.empty((1, wl.K), dtype=torch.int32, device=gpu)
    say("prefetch: Ling layer without prefetch")
    _layer(d, lw, x, out0, idx, ws, 1)
    ids = _ids(gpu, np.arange(wl.E + wl.S))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("prefetch: all %d experts on a side stream" % (wl.E + wl.S))
    md.check(md.moe_expert_prefetch(d, lw, ids, wl.E + wl.S, stream=side.cuda_stream))
    ev = torch.cuda.Event()
    ev.record(side)
    torch.cuda.current_stream().wait_event(ev)
    _layer(d, lw, x, out1, idx, ws, 1)
    md.check(md.moe_last_device_status(ws))
    assert torch.equal(out0, out1)


def test_prefetch_without_a_shared_expert(gpu, dw):
    """S = 0: id E names no expert and is skipped; the layer without a shared
    expert gives the same result with and without the prefetch."""
    import torch
    from datagen import device as D
    wl = W.C1
    M = 2
    L = dw.layer(wl, 0)
    d = md.dims(hidden=wl.H, n_experts=wl.E, top_k=wl.K, inter=wl.I, n_shared=0)
    lw = md.layer_weights(L.w_router, L.w_gate_up, L.w_down)
    x = D.to_device(x_tiefree(wl, M))
    ws = md.new_workspace(d, M, 1)
    out0 = torch.empty((M, wl.H), dtype=torch.int16, device=gpu)
    out1 = torch.empty_like(out0)
    idx = torch.empty((M, wl.K), dtype=torch.int32, device=gpu)
    say("prefetch: tiny layer without a shared expert, M=2")
    _layer(d, lw, x, out0, idx, ws, M)
    vals = [wl.E, 0, wl.E - 1, wl.E + 1]
    md.check(md.moe_expert_prefetch(d, lw, _ids(gpu, vals), len(vals)))
    _layer(d, lw, x, out1, idx, ws, M)
    md.check(md.moe_last_device_status(ws))
    assert torch.equal(out0, out1)
