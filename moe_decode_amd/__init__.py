"""Python binding of libmoedecode (the small-M MoE decoder step on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmoedecode.so, reached through its C ABI (include/moe_decode.h).
PyTorch is used for device memory and streams.  There is no fallback: if the
library is missing, importing this package raises.

Pointer arguments accept a torch tensor (its data_ptr() is passed), a plain
integer address, or None (NULL).
"""
import ctypes
import os

# The library must bind to the HIP runtime that owns the caller's device
# memory and streams.  torch ships its own libamdhip64 with the same soname;
# loading torch first makes the dynamic linker reuse that one instead of
# pulling a second runtime from the system path.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoedecode.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoedecode.so is not built (run __graft_entry__.build()); "
                      "there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
MOE_E_ARG = -1
MOE_E_UNSUPPORTED = -2
MOE_E_ALIGN = -3
MOE_E_WORKSPACE = -4
MOE_E_HIP = -5
MOE_E_TIMEOUT = -6
MOE_E_INDEX = -7

MOE_OUT_BF16 = 0
MOE_OUT_F32 = 1
MOE_CHAIN_RESIDUAL = 0
MOE_CHAIN_LAYER_ONLY = 1
MOE_CHAIN_PRENORM_RESIDUAL = 2
MOE_CHAIN_PRENORM_LAYER_ONLY = 3
MOE_EXPERT_BF16 = 0
MOE_EXPERT_FP8_B128 = 1

MOE_MAX_ROWS = 16
MOE_MAX_LAYERS = 64
MOE_MAX_PREFETCH_IDS = 4096

DBG_NO_ROUTER_PUBLISH = 1
DBG_STAMPS = 2
DBG_NOT_RESIDENT = 4

EXPORTED = ("moe_workspace_size", "moe_workspace_init", "moe_router_topk", "moe_experts_fused",
            "moe_layer_chain", "moe_layer_chain_noalloc", "lmhead_argmax", "moe_expert_prefetch",
            "moe_last_device_status", "moe_workspace_debug", "moe_status_str")
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class moe_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("expert_format", ctypes.c_int32)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("norm_gain", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_lib.moe_workspace_size.restype = ctypes.c_int
_lib.moe_workspace_size.argtypes = [ctypes.POINTER(moe_dims), _I32, _I32, ctypes.POINTER(_SZ)]
_lib.moe_workspace_init.restype = ctypes.c_int
_lib.moe_workspace_init.argtypes = [_P, _SZ, _P]
_lib.moe_router_topk.restype = ctypes.c_int
_lib.moe_router_topk.argtypes = [ctypes.POINTER(moe_dims), _I32, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                 _P]
_lib.moe_experts_fused.restype = ctypes.c_int
_lib.moe_experts_fused.argtypes = [ctypes.POINTER(moe_dims), _I32, _P, _P, _P,
                                   ctypes.POINTER(moe_layer_weights), _P, _I32, _P, _SZ, _P]
_lib.moe_layer_chain.restype = ctypes.c_int
_lib.moe_layer_chain.argtypes = [ctypes.POINTER(moe_dims), _I32, _I32,
                                 ctypes.POINTER(moe_layer_weights), _P, _P, _I32, _I32, _P, _P,
                                 _P, _SZ, _P]
_lib.moe_layer_chain_noalloc.restype = ctypes.c_int
_lib.moe_layer_chain_noalloc.argtypes = [ctypes.POINTER(moe_dims), _I32, _I32,
                                         ctypes.POINTER(moe_layer_weights), _P, _P, _I32, _I32,
                                         _P, _P, _P]
_lib.lmhead_argmax.restype = ctypes.c_int
_lib.lmhead_argmax.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]
_lib.moe_expert_prefetch.restype = ctypes.c_int
_lib.moe_expert_prefetch.argtypes = [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_layer_weights),
                                     _P, _I32, _P]
_lib.moe_last_device_status.restype = ctypes.c_int
_lib.moe_last_device_status.argtypes = [_P, _SZ, _P]
_lib.moe_workspace_debug.restype = ctypes.c_int
_lib.moe_workspace_debug.argtypes = [_P, _SZ, ctypes.c_uint32, ctypes.c_uint32, _P]
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_status_str.argtypes = [ctypes.c_int]


class MoeError(RuntimeError):
    def __init__(self, status):
        super().__init__("libmoedecode: %s (%d)" % (moe_status_str(status), status))
        self.status = status


def check(status):
    if status != MOE_OK:
        raise MoeError(status)
    return status


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return ws_bytes
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def dims(hidden, n_experts, top_k, inter, n_shared, routed_scale=0.0,
         expert_format=MOE_EXPERT_BF16):
    """routed_scale 0 means 1 (the plain combine)."""
    return moe_dims(hidden, n_experts, top_k, inter, n_shared, routed_scale, expert_format)


def layer_weights(w_router, w_gate_up, w_down, router_bias=None, norm_gain=None,
                  s_gate_up=None, s_down=None):
    w = moe_layer_weights(_ptr(w_router), _ptr(w_gate_up), _ptr(w_down), _ptr(router_bias),
                          _ptr(norm_gain), _ptr(s_gate_up), _ptr(s_down))
    # the struct holds raw device addresses: keep the tensors they came from alive
    # for as long as the struct is (a temporary passed here would otherwise be
    # freed, and its memory handed to the next allocation, before the call runs)
    w._keep = (w_router, w_gate_up, w_down, router_bias, norm_gain, s_gate_up, s_down)
    return w


# ---- the C entry points, same names -------------------------------------------

def moe_status_str(status):
    return _lib.moe_status_str(int(status)).decode()


def moe_workspace_size(d, max_rows, n_layers):
    """Returns (status, bytes)."""
    out = _SZ(0)
    rc = _lib.moe_workspace_size(ctypes.byref(d) if d is not None else None, max_rows, n_layers,
                                 ctypes.byref(out))
    return rc, int(out.value)


def moe_workspace_init(ws, ws_bytes=None, stream=None):
    return _lib.moe_workspace_init(_ptr(ws), _nbytes(ws, ws_bytes), _stream(stream))


def moe_router_topk(d, M, x, w_router, router_bias, topk_idx, topk_gate, logits, ws,
                    ws_bytes=None, stream=None):
    return _lib.moe_router_topk(ctypes.byref(d) if d is not None else None, M, _ptr(x),
                                _ptr(w_router), _ptr(router_bias), _ptr(topk_idx),
                                _ptr(topk_gate), _ptr(logits), _ptr(ws), _nbytes(ws, ws_bytes),
                                _stream(stream))


def moe_experts_fused(d, M, x, topk_idx, topk_gate, w, out, out_dtype, ws, ws_bytes=None,
                      stream=None):
    return _lib.moe_experts_fused(ctypes.byref(d) if d is not None else None, M, _ptr(x),
                                  _ptr(topk_idx), _ptr(topk_gate),
                                  ctypes.byref(w) if w is not None else None, _ptr(out),
                                  out_dtype, _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream))


def moe_layer_chain(d, M, layers, x_in, out, out_dtype, mode, topk_idx_all, ws, ws_bytes=None,
                    stream=None, h_all=None):
    """layers: a sequence of moe_layer_weights (or None)."""
    if layers is None:
        arr, n = None, 0
    else:
        n = len(layers)
        arr = (moe_layer_weights * max(n, 1))(*layers)
    return _lib.moe_layer_chain(ctypes.byref(d) if d is not None else None, M, n, arr, _ptr(x_in),
                                _ptr(out), out_dtype, mode, _ptr(topk_idx_all), _ptr(h_all),
                                _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream))


def moe_layer_chain_noalloc(d, M, layers, x_in, out, out_dtype, mode, topk_idx_all, stream=None,
                            h_all=None):
    """moe_layer_chain on the library's static workspace (no workspace argument)."""
    if layers is None:
        arr, n = None, 0
    else:
        n = len(layers)
        arr = (moe_layer_weights * max(n, 1))(*layers)
    return _lib.moe_layer_chain_noalloc(ctypes.byref(d) if d is not None else None, M, n, arr,
                                        _ptr(x_in), _ptr(out), out_dtype, mode,
                                        _ptr(topk_idx_all), _ptr(h_all), _stream(stream))


def lmhead_argmax(M, H, V, h, w_lm, token, max_logit, ws, ws_bytes=None, stream=None):
    return _lib.lmhead_argmax(M, H, V, _ptr(h), _ptr(w_lm), _ptr(token), _ptr(max_logit),
                              _ptr(ws), _nbytes(ws, ws_bytes), _stream(stream))


def moe_expert_prefetch(d, w, expert_ids, n, stream=None):
    return _lib.moe_expert_prefetch(ctypes.byref(d) if d is not None else None,
                                    ctypes.byref(w) if w is not None else None, _ptr(expert_ids),
                                    n, _stream(stream))


def moe_last_device_status(ws, ws_bytes=None, stream=None):
    return _lib.moe_last_device_status(_ptr(ws), _nbytes(ws, ws_bytes), _stream(stream))


def moe_workspace_debug(ws, flags, deadline_us, ws_bytes=None, stream=None):
    return _lib.moe_workspace_debug(_ptr(ws), _nbytes(ws, ws_bytes), flags, deadline_us,
                                    _stream(stream))


# ---- device memory plumbing ------------------------------------------------------

def new_workspace(d, max_rows, n_layers, device="cuda"):
    """Allocate (torch) and zero a workspace for calls up to max_rows rows / n_layers layers."""
    import torch
    rc, nbytes = moe_workspace_size(d, max_rows, n_layers)
    check(rc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check(moe_workspace_init(ws))
    return ws
