"""Generate the synthetic workloads directly in device memory (torch tensors).

Same keys and the same integer-exact generator as the host slices in
workloads.py, so every device tensor equals its host counterpart bit for bit.
"""
import numpy as np

from . import (SIGMA_W, TENSOR_DOWN, TENSOR_DOWN_FP8, TENSOR_GATE_UP, TENSOR_GATE_UP_FP8,
               TENSOR_LMHEAD, TENSOR_ROUTER, fill_device, fill_device_fp8, key)
from .workloads import WEIGHT_SEED


class DeviceLayer:
    def __init__(self, w_router, w_gate_up, w_down, s_gate_up=None, s_down=None):
        self.w_router = w_router      # int16 [E][H]
        self.w_gate_up = w_gate_up    # int16 [E+S][2I][H] (uint8 codes for fp8)
        self.w_down = w_down          # int16 [E+S][H][I] (uint8 codes for fp8)
        self.s_gate_up = s_gate_up    # fp8 only: float32 [E+S][2I/128][H/128]
        self.s_down = s_down          # fp8 only: float32 [E+S][H/128][I/128]


def _keys(keys, dev):
    import torch
    return torch.tensor(np.array(keys, dtype=np.uint64).view(np.int64), device=dev)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_layer(wl, layer, dev="cuda"):
    import torch
    H, E, I, S = wl.H, wl.E, wl.I, wl.S
    st = _stream()
    wr = torch.empty((E, H), dtype=torch.int16, device=dev)
    kr = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_ROUTER)], dev)
    fill_device(wr.data_ptr(), kr.data_ptr(), 1, 0, E, H, SIGMA_W, stream=st)
    gu = torch.empty((E + S, 2 * I, H), dtype=torch.int16, device=dev)
    kg = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_GATE_UP, e) for e in range(E + S)], dev)
    stride = 2 * I * H
    if wl.n_shards == 1:
        fill_device(gu.data_ptr(), kg.data_ptr(), E + S, stride, 2 * I, H, SIGMA_W, stream=st)
    else:
        fill_device(gu.data_ptr(), kg.data_ptr(), E + S, stride, I, H, SIGMA_W,
                    row0=wl.shard * I, ld_full=H, stream=st)
        fill_device(gu.data_ptr() + I * H * 2, kg.data_ptr(), E + S, stride, I, H, SIGMA_W,
                    row0=wl.I_full + wl.shard * I, ld_full=H, stream=st)
    dn = torch.empty((E + S, H, I), dtype=torch.int16, device=dev)
    kd = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_DOWN, e) for e in range(E + S)], dev)
    fill_device(dn.data_ptr(), kd.data_ptr(), E + S, H * I, H, I, SIGMA_W, col0=wl.shard * I,
                ld_full=wl.I_full, stream=st)
    torch.cuda.synchronize()
    del kr, kg, kd
    return DeviceLayer(wr, gu, dn)


def make_layer_fp8(wl, layer, dev="cuda"):
    """fp8 expert codes generated on the device; block scales generated on the host."""
    import torch
    from . import workloads as W
    H, E, I, S = wl.H, wl.E, wl.I, wl.S
    st = _stream()
    wr = torch.empty((E, H), dtype=torch.int16, device=dev)
    kr = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_ROUTER)], dev)
    fill_device(wr.data_ptr(), kr.data_ptr(), 1, 0, E, H, SIGMA_W, stream=st)
    gu = torch.empty((E + S, 2 * I, H), dtype=torch.uint8, device=dev)
    kg = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_GATE_UP_FP8, e) for e in range(E + S)],
               dev)
    fill_device_fp8(gu.data_ptr(), kg.data_ptr(), E + S, 2 * I * H, 2 * I, H, stream=st)
    dn = torch.empty((E + S, H, I), dtype=torch.uint8, device=dev)
    kd = _keys([key(WEIGHT_SEED, wl.family, layer, TENSOR_DOWN_FP8, e) for e in range(E + S)], dev)
    fill_device_fp8(dn.data_ptr(), kd.data_ptr(), E + S, H * I, H, I, stream=st)
    sg = np.stack([W.expert_gate_up_scales(wl, layer, e) for e in range(E + S)])
    sd = np.stack([W.expert_down_scales(wl, layer, e) for e in range(E + S)])
    torch.cuda.synchronize()
    del kr, kg, kd
    return DeviceLayer(wr, gu, dn, to_device(sg), to_device(sd))


def make_lmhead(wl, dev="cuda"):
    import torch
    w = torch.empty((wl.V, wl.H), dtype=torch.int16, device=dev)
    k = _keys([key(WEIGHT_SEED, wl.family, 0, TENSOR_LMHEAD)], dev)
    fill_device(w.data_ptr(), k.data_ptr(), 1, 0, wl.V, wl.H, SIGMA_W, stream=_stream())
    torch.cuda.synchronize()
    return w


def to_device(a, dev="cuda"):
    """Host uint16 (bf16 bits) or other numpy array -> device tensor (bf16 bits as int16)."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def from_device_bf16(t):
    return t.cpu().numpy().view(np.uint16)
