"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Only input generation lives here (keys, the counter-based generator, the
workload shapes); none of the MoE arithmetic does.  Host generation goes
through libdg_host.so, device generation through libdg_device.so; both
produce identical bf16 bits for the same key and element index.
"""
import ctypes
import os

import numpy as np

from .build import HOST_SO, DEV_SO

# tensor families / ids used in keys
FAMILY_TINY = 1
FAMILY_LING = 2
TENSOR_X = 1
TENSOR_ROUTER = 2
TENSOR_GATE_UP = 3
TENSOR_DOWN = 4
TENSOR_LMHEAD = 5
TENSOR_BIAS = 6     # per-expert router selection bias
TENSOR_GAIN = 7     # RMSNorm gain in front of the router and experts
TENSOR_GATE_UP_FP8 = 8   # fp8 e4m3 codes of the gate/up projections
TENSOR_DOWN_FP8 = 9      # fp8 e4m3 codes of the down projections
TENSOR_SCALE_GU = 10     # block-128 scales of the gate/up projections
TENSOR_SCALE_D = 11      # block-128 scales of the down projections

FP8_MUL = 100            # fp8 codes ~ e4m3(N(0, 100^2)): amax of a 128x128 block near 4.3 sigma
FP8_BLOCK = 128

SIGMA_W = 0.02   # weights ~ N(0, 0.02^2)
SIGMA_X = 1.0    # inputs ~ N(0, 1)

_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            raise RuntimeError("libdg_host.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_SO)
        lib.dg_key_c.restype = ctypes.c_uint64
        lib.dg_key_c.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 5
        lib.dg_ih12_c.restype = ctypes.c_int32
        lib.dg_ih12_c.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.dg_fill_bf16.restype = None
        lib.dg_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_int64] * 5 + [ctypes.c_float]
        lib.dg_fill_fp8.restype = None
        lib.dg_fill_fp8.argtypes = [ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_int64] * 5 + [ctypes.c_int32]
        lib.dg_e4m3_code_c.restype = ctypes.c_uint8
        lib.dg_e4m3_code_c.argtypes = [ctypes.c_int32, ctypes.c_int32]
        lib.dg_fill_scales.restype = None
        lib.dg_fill_scales.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see moe_decode_amd)
        if not os.path.exists(DEV_SO):
            raise RuntimeError("libdg_device.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_SO)
        lib.dg_error_string.restype = ctypes.c_char_p
        lib.dg_error_string.argtypes = [ctypes.c_int]
        lib.dg_fill_bf16_dev.restype = ctypes.c_int
        lib.dg_fill_bf16_dev.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int] + \
            [ctypes.c_int64] * 6 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.dg_fill_fp8_dev.restype = ctypes.c_int
        lib.dg_fill_fp8_dev.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int] + \
            [ctypes.c_int64] * 6 + [ctypes.c_int32, ctypes.c_void_p]
        _dev = lib
    return _dev


def scale_for(sigma):
    """fp32 multiplier that maps an Irwin-Hall(12) integer to a sample of std sigma."""
    return float(np.float32(sigma / 65536.0))


def key(seed, family, layer, tensor, expert=0, attempt=0):
    return int(_host_lib().dg_key_c(seed, family, layer, tensor, expert, attempt))


def ih12(k, n):
    return int(_host_lib().dg_ih12_c(k, n))


def fill_host(k, rows, cols, sigma, row0=0, col0=0, ld_full=None):
    """bf16 bits (uint16 array [rows, cols]) of a slice of the keyed tensor."""
    if ld_full is None:
        ld_full = cols
    out = np.empty((rows, cols), dtype=np.uint16)
    _host_lib().dg_fill_bf16(out.ctypes.data, k, row0, col0, rows, cols, ld_full,
                             scale_for(sigma))
    return out


def fill_host_fp8(k, rows, cols, row0=0, col0=0, ld_full=None, mul=FP8_MUL):
    """fp8 e4m3 codes (uint8 [rows, cols]) of a slice of the keyed tensor."""
    if ld_full is None:
        ld_full = cols
    out = np.empty((rows, cols), dtype=np.uint8)
    _host_lib().dg_fill_fp8(out.ctypes.data, k, row0, col0, rows, cols, ld_full, mul)
    return out


def e4m3_code(s, mul):
    return int(_host_lib().dg_e4m3_code_c(int(s), int(mul)))


def fill_scales(k, shape, base):
    out = np.empty(shape, dtype=np.float32)
    _host_lib().dg_fill_scales(out.ctypes.data, k, out.size, float(base))
    return out


def fill_device_fp8(out_ptr, keys_dev_ptr, n_blocks, block_stride, rows, cols, row0=0, col0=0,
                    ld_full=None, stream=0, mul=FP8_MUL):
    if ld_full is None:
        ld_full = cols
    rc = _dev_lib().dg_fill_fp8_dev(out_ptr, keys_dev_ptr, n_blocks, block_stride, row0, col0,
                                    rows, cols, ld_full, mul, stream)
    if rc != 0:
        raise RuntimeError("dg_fill_fp8_dev failed (%d: %s)"
                           % (rc, _dev_lib().dg_error_string(rc).decode()))


def round_bf16_bits(f):
    """fp32 values -> bf16 bits, round to nearest even (finite inputs only)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def fill_device(out_ptr, keys_dev_ptr, n_blocks, block_stride, rows, cols, sigma,
                row0=0, col0=0, ld_full=None, stream=0, transposed=False):
    """Fill n_blocks device slices (block b at out_ptr + 2*b*block_stride bytes), each the
    rows x cols slice stored row-major, or column-major (its transpose) if `transposed`."""
    if ld_full is None:
        ld_full = cols
    rc = _dev_lib().dg_fill_bf16_dev(out_ptr, keys_dev_ptr, n_blocks, block_stride, row0, col0,
                                     rows, cols, ld_full, scale_for(sigma), int(transposed),
                                     stream)
    if rc != 0:
        raise RuntimeError("dg_fill_bf16_dev failed (%d: %s)"
                           % (rc, _dev_lib().dg_error_string(rc).decode()))
