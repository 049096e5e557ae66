"""moe_layer_chain_noalloc (the library's static workspace) against moe_layer_chain on a
caller workspace: the same kernels on the same inputs, so indices and outputs must be
identical bit for bit.  Two calls in a row, the second with a smaller input, then a
three-layer chain; every call through the C ABI."""
import numpy as np
import pytest

import moe_decode_amd as md
from datagen import workloads as W
from datagen import device as D

from gpu_support import say, x_tiefree

pytestmark = pytest.mark.gpu


def _dims(wl):
    return md.dims(wl.H, wl.E, wl.K, wl.I, wl.S)


def _lw(L):
    return md.layer_weights(L.w_router, L.w_gate_up, L.w_down)


def _both(wl, layers, x, mode, n_idx_layers):
    """(idx, out) from the workspace call and from the static-workspace call."""
    import torch
    M = x.shape[0]
    d = _dims(wl)
    xin = D.to_device(x)
    res = []
    for noalloc in (False, True):
        out = torch.empty((M, wl.H), dtype=torch.int16, device="cuda")
        idx = torch.full((n_idx_layers, M, wl.K), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            say("layer_chain_noalloc mode=%d %s L=%d M=%d" % (mode, wl.name, len(layers), M))
            md.check(md.moe_layer_chain_noalloc(d, M, layers, xin, out, md.MOE_OUT_BF16, mode,
                                                idx))
        else:
            ws = md.new_workspace(d, M, len(layers))
            say("layer_chain mode=%d %s L=%d M=%d" % (mode, wl.name, len(layers), M))
            md.check(md.moe_layer_chain(d, M, layers, xin, out, md.MOE_OUT_BF16, mode, idx, ws))
            md.check(md.moe_last_device_status(ws))
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), out.cpu().numpy().view(np.uint16)))
    return res


def test_noalloc_matches_workspace_call_then_smaller_then_chain(gpu, dw):
    # first call: the Ling-shaped layer at six rows
    wl = W.C3
    (i0, o0), (i1, o1) = _both(wl, [_lw(dw.layer(wl, 0))], x_tiefree(wl, 6),
                               md.MOE_CHAIN_LAYER_ONLY, 1)
    assert np.all(i0 >= 0) and np.array_equal(i0, i1) and np.array_equal(o0, o1)
    # second call, smaller: one row of another layer (the static workspace keeps the
    # first call's contents; the step tags keep them from being taken as this call's)
    wl = W.C2
    (i0, o0), (i1, o1) = _both(wl, [_lw(dw.layer(wl, 1))], x_tiefree(wl, 1),
                               md.MOE_CHAIN_LAYER_ONLY, 1)
    assert np.all(i0 >= 0) and np.array_equal(i0, i1) and np.array_equal(o0, o1)
    # a three-layer pre-norm residual chain of the tiny shape at two rows
    wl = W.C1
    layers = [_lw(dw.layer(wl, l)) for l in range(3)]
    (i0, o0), (i1, o1) = _both(wl, layers, W.x_rows(wl, [0, 1]), md.MOE_CHAIN_PRENORM_RESIDUAL, 3)
    assert np.all(i0 >= 0) and np.array_equal(i0, i1) and np.array_equal(o0, o1)


def test_noalloc_rejects_a_workspace_beyond_its_buffer(gpu):
    d = _dims(W.C3)
    lw = md.layer_weights(16, 16, 16)
    rc = md.moe_layer_chain_noalloc(d, 16, [lw] * 64, 16, 16, md.MOE_OUT_BF16,
                                    md.MOE_CHAIN_RESIDUAL, None)
    assert rc == md.MOE_E_WORKSPACE
