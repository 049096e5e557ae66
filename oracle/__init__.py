"""Python face of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: used by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py.  The product path never imports it.

All tensors are numpy arrays; bf16 values travel as uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from .build import SO

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise RuntimeError("liboracle.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(SO)
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_set_threads.argtypes = [_I]
        L.oracle_router_logits.argtypes = [_I, _I, _I, _P, _P, _P]
        L.oracle_select_gates.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        L.oracle_swiglu.restype = ctypes.c_uint16
        L.oracle_swiglu.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_expert.argtypes = [_I, _I, _P, _P, _P, _P, _P]
        L.oracle_experts_combine.restype = _I
        L.oracle_experts_combine.argtypes = [_I] * 6 + [_P] * 5 + [ctypes.c_float, _P]
        L.oracle_cast_bf16.argtypes = [_I64, _P, _P]
        L.oracle_residual.argtypes = [_I64, _P, _P, _P]
        L.oracle_lmhead_argmax.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        L.oracle_rmsnorm.argtypes = [_I, _I, _P, ctypes.c_float, _P, _P]
        L.oracle_fp8_e4m3_to_f32.restype = ctypes.c_float
        L.oracle_fp8_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_dequant_fp8.argtypes = [_I, _I, _P, _P, _P]
        L.oracle_expert_fp8.argtypes = [_I, _I] + [_P] * 7
        L.oracle_experts_combine_fp8.restype = _I
        L.oracle_experts_combine_fp8.argtypes = [_I] * 6 + [_P] * 7 + [ctypes.c_float, _P]
        L.oracle_unique_weight_bytes.restype = _I64
        L.oracle_unique_weight_bytes.argtypes = [_I] * 6 + [_P, _I, _P]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def set_threads(n):
    lib().oracle_set_threads(int(n))


def f32_to_bf16(a):
    a = _c(a, np.float32).ravel()
    return np.array([lib().oracle_f32_to_bf16(float(v)) for v in a], dtype=np.uint16)


def bf16_to_f32(b):
    """Exact widening of bf16 bits (a bit shift; no rounding involved)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def cast_bf16(acc):
    acc = _c(acc, np.float32)
    out = np.empty(acc.shape, dtype=np.uint16)
    lib().oracle_cast_bf16(acc.size, acc.ctypes.data, out.ctypes.data)
    return out


def swiglu(a, b):
    return int(lib().oracle_swiglu(float(a), float(b)))


def router_logits(x, w_router):
    x = _c(x, np.uint16)
    w = _c(w_router, np.uint16)
    M, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    out = np.empty((M, E), dtype=np.float32)
    lib().oracle_router_logits(H, E, M, x.ctypes.data, w.ctypes.data, out.ctypes.data)
    return out


def select_gates(logits, K, bias=None):
    """bias: optional fp32 [E] selection bias (chooses experts; gates stay unbiased)."""
    logits = _c(logits, np.float32)
    M, E = logits.shape
    if bias is not None:
        bias = _c(bias, np.float32)
        assert bias.shape == (E,)
    idx = np.empty((M, K), dtype=np.int32)
    gate = np.empty((M, K), dtype=np.float32)
    lib().oracle_select_gates(E, K, M, logits.ctypes.data,
                              None if bias is None else bias.ctypes.data, idx.ctypes.data,
                              gate.ctypes.data)
    return idx, gate


def router_topk(x, w_router, K, bias=None):
    logits = router_logits(x, w_router)
    idx, gate = select_gates(logits, K, bias)
    return idx, gate, logits


def expert(x_row, w_gu, w_d):
    """One expert on one row: returns (y fp32 [H], h bf16 bits [I])."""
    x_row = _c(x_row, np.uint16)
    w_gu = _c(w_gu, np.uint16)
    w_d = _c(w_d, np.uint16)
    H = x_row.shape[0]
    I = w_gu.shape[0] // 2
    assert w_gu.shape == (2 * I, H) and w_d.shape == (H, I)
    y = np.empty(H, dtype=np.float32)
    h = np.empty(I, dtype=np.uint16)
    lib().oracle_expert(H, I, x_row.ctypes.data, w_gu.ctypes.data, w_d.ctypes.data,
                        h.ctypes.data, y.ctypes.data)
    return y, h


def experts_combine(x, idx, gate, w_gu_tab, w_d_tab, E, S, scale=1.0):
    """acc fp32 [M, H] = y_shared + scale * sum_k gate_k y_k.
    w_gu_tab / w_d_tab: dict expert id -> array (shared at E)."""
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    M, H = x.shape
    K = idx.shape[1]
    keep = []
    gu_ptrs = (ctypes.c_void_p * (E + 1))()
    d_ptrs = (ctypes.c_void_p * (E + 1))()
    I = None
    for e, a in w_gu_tab.items():
        a = _c(a, np.uint16)
        keep.append(a)
        gu_ptrs[e] = a.ctypes.data
        I = a.shape[0] // 2
    for e, a in w_d_tab.items():
        a = _c(a, np.uint16)
        keep.append(a)
        d_ptrs[e] = a.ctypes.data
    acc = np.empty((M, H), dtype=np.float32)
    rc = lib().oracle_experts_combine(H, E, K, I, int(S), M, x.ctypes.data, idx.ctypes.data,
                                      gate.ctypes.data, ctypes.cast(gu_ptrs, _P),
                                      ctypes.cast(d_ptrs, _P), float(scale), acc.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_experts_combine: bad index or missing expert weights")
    return acc


def fp8_decode(codes):
    """float32 values of fp8 e4m3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().oracle_fp8_e4m3_to_f32(int(v)) for v in c.ravel()],
                    dtype=np.float32).reshape(c.shape)


def dequant_fp8(q, s):
    """fp32 weights [rows, cols] of codes q with 128x128 block scales s."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    rows, cols = q.shape
    assert s.shape == ((rows + 127) // 128, (cols + 127) // 128)
    w = np.empty((rows, cols), dtype=np.float32)
    lib().oracle_dequant_fp8(rows, cols, q.ctypes.data, s.ctypes.data, w.ctypes.data)
    return w


def expert_fp8(x_row, q_gu, s_gu, q_d, s_d):
    """One fp8 expert on one row: returns (y fp32 [H], h bf16 bits [I])."""
    x_row = _c(x_row, np.uint16)
    q_gu, s_gu = _c(q_gu, np.uint8), _c(s_gu, np.float32)
    q_d, s_d = _c(q_d, np.uint8), _c(s_d, np.float32)
    H = x_row.shape[0]
    I = q_gu.shape[0] // 2
    assert q_gu.shape == (2 * I, H) and q_d.shape == (H, I)
    y = np.empty(H, dtype=np.float32)
    h = np.empty(I, dtype=np.uint16)
    lib().oracle_expert_fp8(H, I, x_row.ctypes.data, q_gu.ctypes.data, s_gu.ctypes.data,
                            q_d.ctypes.data, s_d.ctypes.data, h.ctypes.data, y.ctypes.data)
    return y, h


def experts_combine_fp8(x, idx, gate, gu_tab, d_tab, E, S, scale=1.0):
    """acc fp32 [M, H] with fp8 experts.  gu_tab / d_tab: dict expert id -> (codes, scales)."""
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    M, H = x.shape
    K = idx.shape[1]
    keep = []
    tabs = [(ctypes.c_void_p * (E + 1))() for _ in range(4)]
    I = None
    for e, (q, s) in gu_tab.items():
        q, s = _c(q, np.uint8), _c(s, np.float32)
        keep += [q, s]
        I = q.shape[0] // 2
        tabs[0][e], tabs[1][e] = q.ctypes.data, s.ctypes.data
    for e, (q, s) in d_tab.items():
        q, s = _c(q, np.uint8), _c(s, np.float32)
        keep += [q, s]
        tabs[2][e], tabs[3][e] = q.ctypes.data, s.ctypes.data
    acc = np.empty((M, H), dtype=np.float32)
    rc = lib().oracle_experts_combine_fp8(H, E, K, I, int(S), M, x.ctypes.data, idx.ctypes.data,
                                          gate.ctypes.data, *[ctypes.cast(t, _P) for t in tabs],
                                          float(scale), acc.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_experts_combine_fp8: bad index or missing expert weights")
    return acc


def residual(h, acc):
    h = _c(h, np.uint16)
    acc = _c(acc, np.float32)
    assert h.shape == acc.shape
    out = np.empty(h.shape, dtype=np.uint16)
    lib().oracle_residual(h.size, h.ctypes.data, acc.ctypes.data, out.ctypes.data)
    return out


RMS_EPS = 1e-6


def rmsnorm(h, eps=RMS_EPS, gain=None):
    """u = bf16((h * r) * gain) per row; gain: optional bf16 bits [H] (None: unit gain)."""
    h = _c(h, np.uint16)
    M, H = h.shape
    if gain is not None:
        gain = _c(gain, np.uint16)
        assert gain.shape == (H,)
    u = np.empty_like(h)
    lib().oracle_rmsnorm(M, H, h.ctypes.data, eps, None if gain is None else gain.ctypes.data,
                         u.ctypes.data)
    return u


def lmhead_argmax(h, w):
    h = _c(h, np.uint16)
    w = _c(w, np.uint16)
    M, H = h.shape
    V = w.shape[0]
    tok = np.empty(M, dtype=np.int32)
    mx = np.empty(M, dtype=np.float32)
    lib().oracle_lmhead_argmax(M, H, V, h.ctypes.data, w.ctypes.data, tok.ctypes.data,
                               mx.ctypes.data)
    return tok, mx


def unique_weight_bytes(H, E, K, I, S, idx, include_router=True):
    idx = _c(idx, np.int32)
    M = idx.shape[0]
    U = ctypes.c_int(0)
    b = lib().oracle_unique_weight_bytes(H, E, K, I, int(S), M, idx.ctypes.data,
                                         1 if include_router else 0, ctypes.byref(U))
    return int(b), int(U.value)
