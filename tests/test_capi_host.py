"""The C-ABI library on the host: it loads, exports what include/moe_decode.h
declares, and rejects bad arguments before anything reaches a device.

No call here launches a kernel: every call either is pure host arithmetic
(moe_workspace_size, moe_status_str) or fails validation, which runs before any
HIP call.  Fake device addresses are plain integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import moe_decode_amd as md

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")

A = 1 << 20          # a fake, 16-byte aligned device address
BAD = A + 2          # misaligned
LING = dict(hidden=2560, n_experts=512, top_k=8, inter=768, n_shared=1)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src,
                       flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_every_declared_function_is_exported():
    decl = declared_functions()
    assert set(decl) == set(md.EXPORTED), decl
    out = subprocess.run(["nm", "-D", "--defined-only", md.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in decl:
        assert name in exported, name
        assert hasattr(md._lib, name)


def test_library_links_only_the_hip_runtime_it_shares_with_torch():
    out = subprocess.run(["readelf", "-d", md.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"\[(.*?)\]", "\n".join(l for l in out.splitlines() if "NEEDED" in l))
    assert any(n.startswith("libamdhip64.so") for n in needed)
    assert not any("torch" in n or "c10" in n for n in needed)


def test_status_strings():
    for s in range(-7, 1):
        assert md.moe_status_str(s) != "unknown status"
    assert md.moe_status_str(-99) == "unknown status"


def test_workspace_size_layout_and_errors():
    d = md.dims(**LING)
    rc, b1 = md.moe_workspace_size(d, 1, 1)
    assert rc == md.MOE_OK
    rc, b6 = md.moe_workspace_size(d, 6, 16)
    assert rc == md.MOE_OK and b6 > b1

    def up(v):
        return (v + 255) // 256 * 256
    M, L, E, H, I, K, S = 6, 16, 512, 2560, 768, 8, 1
    C = 8  # the words every workgroup reads: one copy per XCD
    lg = 4096 + 256 * 32 * 8 + 512 * 16 * 2 * 8   # control words, phase stamps, lm_head slots
    hs = up(lg + L * C * M * E * 8)             # logits
    hr = up(hs + L * C * M * (I // 2) * 8)      # shared SwiGLU pairs
    y = up(hr + L * M * K * (I // 2) * 8)       # routed SwiGLU pairs
    res = up(y + L * M * K * H * 8)             # routed down outputs
    assert b6 == up(res + (L + 1) * C * M * (H // 2) * 8)
    assert md.moe_workspace_size(None, 1, 1)[0] == md.MOE_E_ARG
    assert md.moe_workspace_size(d, 0, 1)[0] == md.MOE_E_ARG
    assert md.moe_workspace_size(d, 17, 1)[0] == md.MOE_E_UNSUPPORTED
    assert md.moe_workspace_size(d, 16, 1)[0] == md.MOE_OK
    assert md.moe_workspace_size(d, 1, 65)[0] == md.MOE_E_UNSUPPORTED


@pytest.mark.parametrize("kw,rc", [
    (dict(n_shared=2), md.MOE_E_ARG),
    (dict(top_k=0), md.MOE_E_ARG),
    (dict(top_k=513), md.MOE_E_ARG),
    (dict(n_experts=2048, top_k=8), md.MOE_E_UNSUPPORTED),
    (dict(top_k=17), md.MOE_E_UNSUPPORTED),
    (dict(hidden=2500), md.MOE_E_UNSUPPORTED),
    (dict(inter=100), md.MOE_E_UNSUPPORTED),
    (dict(hidden=-256), md.MOE_E_ARG),
])
def test_dims_validation(kw, rc):
    d = md.dims(**dict(LING, **kw))
    assert md.moe_workspace_size(d, 1, 1)[0] == rc
    assert md.moe_router_topk(d, 1, A, A, None, A, A, None, A, 1 << 30, stream=0) == rc


def test_router_topk_validation():
    d = md.dims(**LING)
    big = 1 << 30
    assert md.moe_router_topk(d, 0, A, A, None, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert md.moe_router_topk(d, 17, A, A, None, A, A, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert md.moe_router_topk(d, 1, None, A, None, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert md.moe_router_topk(d, 1, A, None, None, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert md.moe_router_topk(d, 1, A, A, None, None, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert md.moe_router_topk(d, 1, BAD, A, None, A, A, None, A, big, stream=0) == md.MOE_E_ALIGN
    assert md.moe_router_topk(d, 1, A, BAD, None, A, A, None, A, big, stream=0) == md.MOE_E_ALIGN
    assert md.moe_router_topk(d, 1, A, A, None, A, A, None, None, big, stream=0) == md.MOE_E_WORKSPACE
    assert md.moe_router_topk(d, 1, A, A, None, A, A, None, BAD, big, stream=0) == md.MOE_E_ALIGN
    assert md.moe_router_topk(d, 1, A, A, None, A, A, None, A, 4096, stream=0) == md.MOE_E_WORKSPACE


def test_experts_fused_validation():
    d = md.dims(**LING)
    big = 1 << 30
    w = md.moe_layer_weights(0, A, A)
    f = md.moe_experts_fused
    assert f(d, 1, A, A, A, w, A, 2, A, big, stream=0) == md.MOE_E_ARG          # bad dtype
    assert f(d, 1, A, A, A, None, A, 0, A, big, stream=0) == md.MOE_E_ARG
    assert f(d, 1, A, A, A, md.moe_layer_weights(0, 0, A), A, 0, A, big, stream=0) == md.MOE_E_ARG
    assert f(d, 1, A, A, A, md.moe_layer_weights(0, BAD, A), A, 0, A, big, stream=0) == md.MOE_E_ALIGN
    assert f(d, 1, A, A + 1, A, w, A, 0, A, big, stream=0) == md.MOE_E_ALIGN     # idx not 4-aligned
    assert f(d, 1, A, A, A, w, BAD, 0, A, big, stream=0) == md.MOE_E_ALIGN
    assert f(d, 1, A, A, A, w, A, 0, A, 100, stream=0) == md.MOE_E_WORKSPACE


def test_layer_chain_validation():
    d = md.dims(**LING)
    big = 1 << 30
    lw = md.moe_layer_weights(A, A, A)
    c = md.moe_layer_chain
    R, LO, PN = md.MOE_CHAIN_RESIDUAL, md.MOE_CHAIN_LAYER_ONLY, md.MOE_CHAIN_PRENORM_RESIDUAL
    assert c(d, 1, [lw, lw], A, A, 0, LO, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert c(d, 1, [lw], A, A, 1, R, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert c(d, 1, [lw], A, A, 1, PN, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert c(d, 1, [lw], A, A, 0, 7, None, A, big, stream=0) == md.MOE_E_ARG
    assert c(d, 1, [], A, A, 0, R, None, A, big, stream=0) == md.MOE_E_ARG
    assert c(d, 1, [lw] * 65, A, A, 0, R, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert c(d, 1, [md.moe_layer_weights(A, 0, A)], A, A, 0, R, None, A, big,
             stream=0) == md.MOE_E_ARG
    assert c(d, 1, [md.moe_layer_weights(BAD, A, A)], A, A, 0, R, None, A, big,
             stream=0) == md.MOE_E_ALIGN
    assert c(d, 1, [lw], A, A, 0, R, A + 2, A, big, stream=0) == md.MOE_E_ALIGN
    rc, need = md.moe_workspace_size(d, 6, 16)
    assert c(d, 6, [lw] * 16, A, A, 0, R, None, A, need - 256, stream=0) == md.MOE_E_WORKSPACE


def test_router_front_validation():
    """Selection bias, norm gain and routed scale are checked on the host too."""
    assert ctypes.sizeof(md.moe_dims) == 28 and ctypes.sizeof(md.moe_layer_weights) == 56
    big = 1 << 30
    for bad in (float("nan"), float("inf"), -float("inf")):
        d = md.dims(**LING, routed_scale=bad)
        assert md.moe_workspace_size(d, 1, 1)[0] == md.MOE_E_ARG
        assert md.moe_router_topk(d, 1, A, A, None, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    d = md.dims(**LING, routed_scale=2.5)
    assert md.moe_workspace_size(d, 1, 1)[0] == md.MOE_OK
    assert md.moe_router_topk(d, 1, A, A, A + 2, A, A, None, A, big, stream=0) == md.MOE_E_ALIGN
    c = md.moe_layer_chain
    R, PN, PL = (md.MOE_CHAIN_RESIDUAL, md.MOE_CHAIN_PRENORM_RESIDUAL,
                 md.MOE_CHAIN_PRENORM_LAYER_ONLY)
    lw = md.layer_weights(A, A, A, A, A)
    assert c(d, 1, [lw, lw], A, A, 0, PL, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert c(d, 1, [lw], A, A, 0, PL, None, A, big, stream=0, h_all=A * 4) == md.MOE_E_ARG
    assert c(d, 1, [lw], A, A, 0, 4, None, A, big, stream=0) == md.MOE_E_ARG
    assert c(d, 1, [md.layer_weights(A, A, A, A + 1, A)], A, A, 0, R, None, A, big,
             stream=0) == md.MOE_E_ALIGN
    assert c(d, 1, [md.layer_weights(A, A, A, None, A + 2)], A, A, 0, PN, None, A, big,
             stream=0) == md.MOE_E_ALIGN
    assert c(d, 1, [md.layer_weights(A, A, A, None, A + 2)], A, A, 1, PL, None, A, big,
             stream=0) == md.MOE_E_ALIGN


def test_fp8_expert_validation():
    """fp8 block-128 experts: format code, the block-128 shape rule, and the scale tensors."""
    big = 1 << 30
    F8 = md.MOE_EXPERT_FP8_B128
    assert md.moe_workspace_size(md.dims(**LING, expert_format=7), 1, 1)[0] == md.MOE_E_ARG
    assert md.moe_workspace_size(md.dims(**LING, expert_format=F8), 1, 1)[0] == md.MOE_OK
    # I = 192 (a TP4 shard of 768) is not a whole number of 128-blocks
    tp4 = dict(LING, inter=192)
    assert md.moe_workspace_size(md.dims(**tp4, expert_format=F8), 1, 1)[0] == md.MOE_E_UNSUPPORTED
    assert md.moe_workspace_size(md.dims(**tp4), 1, 1)[0] == md.MOE_OK
    d8, d16 = md.dims(**LING, expert_format=F8), md.dims(**LING)
    f, c = md.moe_experts_fused, md.moe_layer_chain
    LO = md.MOE_CHAIN_LAYER_ONLY
    no_scales = md.layer_weights(A, A, A)
    one_scale = md.layer_weights(A, A, A, s_gate_up=A)
    bad_scale = md.layer_weights(A, A, A, s_gate_up=A, s_down=A + 2)
    with_scales = md.layer_weights(A, A, A, s_gate_up=A, s_down=A)
    assert f(d8, 1, A, A, A, no_scales, A, 0, A, big, stream=0) == md.MOE_E_ARG
    assert f(d8, 1, A, A, A, one_scale, A, 0, A, big, stream=0) == md.MOE_E_ARG
    assert f(d8, 1, A, A, A, bad_scale, A, 0, A, big, stream=0) == md.MOE_E_ALIGN
    assert f(d16, 1, A, A, A, with_scales, A, 0, A, big, stream=0) == md.MOE_E_ARG
    assert c(d8, 1, [no_scales], A, A, 0, LO, None, A, big, stream=0) == md.MOE_E_ARG
    assert c(d8, 1, [with_scales, bad_scale], A, A, 0, md.MOE_CHAIN_RESIDUAL, None, A, big,
             stream=0) == md.MOE_E_ALIGN
    assert c(d16, 1, [with_scales], A, A, 0, LO, None, A, big, stream=0) == md.MOE_E_ARG


def test_lmhead_validation():
    f = md.lmhead_argmax
    big = 1 << 30
    assert f(0, 2560, 100, A, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert f(17, 2560, 100, A, A, A, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert f(1, 2560, 0, A, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert f(1, 2560, 100, None, A, A, None, A, big, stream=0) == md.MOE_E_ARG
    assert f(1, 2560, 100, A, A, A, None, None, big, stream=0) == md.MOE_E_WORKSPACE
    assert f(1, 2560, 100, A, A, A, None, A, 100, stream=0) == md.MOE_E_WORKSPACE
    assert f(1, 2560, 100, BAD, A, A, None, A, big, stream=0) == md.MOE_E_ALIGN
    assert f(1, 2500, 100, A, A, A, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    # for 1 or 2 rows the dot-product kernel is built for H / 256 in {1, 2, 4, 8, 10}
    assert f(2, 768, 100, A, A, A, None, A, big, stream=0) == md.MOE_E_UNSUPPORTED
    assert f(1, 2560, 100, A, A, A + 2, None, A, big, stream=0) == md.MOE_E_ALIGN
    assert f(1, 2560, 100, A, A, A, A + 2, A, big, stream=0) == md.MOE_E_ALIGN


def test_expert_prefetch_validation():
    """The prefetch hint validates like the expert call; n = 0 enqueues nothing."""
    d16 = md.dims(**LING)
    d8 = md.dims(**LING, expert_format=md.MOE_EXPERT_FP8_B128)
    f = md.moe_expert_prefetch
    w = md.layer_weights(0, A, A)
    assert f(None, w, A, 1, stream=0) == md.MOE_E_ARG
    assert f(d16, None, A, 1, stream=0) == md.MOE_E_ARG
    assert f(d16, md.layer_weights(0, 0, A), A, 1, stream=0) == md.MOE_E_ARG
    assert f(d16, md.layer_weights(0, A, 0), A, 1, stream=0) == md.MOE_E_ARG
    assert f(d16, w, A, -1, stream=0) == md.MOE_E_ARG
    assert f(d16, w, None, 1, stream=0) == md.MOE_E_ARG
    assert f(d16, w, A, md.MOE_MAX_PREFETCH_IDS + 1, stream=0) == md.MOE_E_UNSUPPORTED
    assert f(d16, w, A + 2, 1, stream=0) == md.MOE_E_ALIGN
    assert f(d16, md.layer_weights(0, BAD, A), A, 1, stream=0) == md.MOE_E_ALIGN
    assert f(d16, md.layer_weights(0, A, BAD), A, 1, stream=0) == md.MOE_E_ALIGN
    assert f(d8, w, A, 1, stream=0) == md.MOE_E_ARG                      # fp8 needs scales
    assert f(d16, md.layer_weights(0, A, A, s_gate_up=A, s_down=A), A, 1,
             stream=0) == md.MOE_E_ARG                                    # bf16 takes none
    assert f(d8, md.layer_weights(0, A, A, s_gate_up=A, s_down=A + 2), A, 1,
             stream=0) == md.MOE_E_ALIGN
    assert f(md.dims(**dict(LING, hidden=2500)), w, A, 1, stream=0) == md.MOE_E_UNSUPPORTED
    # an empty list is a valid no-op and reaches no device
    assert f(d16, w, None, 0, stream=0) == md.MOE_OK
    assert f(d8, md.layer_weights(0, A, A, s_gate_up=A, s_down=A), A, 0, stream=0) == md.MOE_OK


def test_workspace_calls_validate_before_touching_the_device():
    assert md.moe_workspace_init(None, 1 << 20, stream=0) == md.MOE_E_WORKSPACE
    assert md.moe_workspace_init(BAD, 1 << 20, stream=0) == md.MOE_E_ALIGN
    assert md.moe_workspace_init(A, 16, stream=0) == md.MOE_E_WORKSPACE
    assert md.moe_last_device_status(None, 1 << 20, stream=0) == md.MOE_E_WORKSPACE
    assert md.moe_workspace_debug(A, 0, 16, stream=0, ws_bytes=16) == md.MOE_E_WORKSPACE
    assert md.moe_workspace_debug(A, 0, 50_000_000, ws_bytes=1 << 20,
                                  stream=0) == md.MOE_E_ARG


def test_one_hip_runtime_per_process():
    """Importing the binding first must not pull in a second HIP runtime."""
    code = ("import moe_decode_amd, datagen, torch\n"
            "datagen._dev_lib()\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len(set(l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l)))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout
    assert out.strip() == "1"


def test_plain_c_caller(tmp_path):
    """The boundary is usable from C alone: tests/capi_smoke.c includes only the
    header, links only the library, and checks host validation through it."""
    exe = tmp_path / "capi_smoke"
    lib_dir = os.path.dirname(md.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "capi_smoke.c"), "-L", lib_dir, "-lmoedecode",
                    "-Wl,-rpath," + lib_dir, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    assert out.strip() == "ok"


def test_noalloc_call_validates_before_touching_the_device():
    """The static-workspace variant rejects bad arguments, and any call whose workspace
    would not fit its MOE_NOALLOC_SCRATCH_BYTES buffer, before any HIP call."""
    d = md.dims(**LING)
    lw = md.layer_weights(16, 16, 16)
    rc, need = md.moe_workspace_size(d, 16, 64)
    assert rc == md.MOE_OK and need > md.MOE_NOALLOC_SCRATCH_BYTES
    assert md.moe_layer_chain_noalloc(d, 16, [lw] * 64, 16, 16, md.MOE_OUT_BF16,
                                      md.MOE_CHAIN_RESIDUAL, None, stream=0) == md.MOE_E_WORKSPACE
    rc, need = md.moe_workspace_size(d, 6, 16)
    assert rc == md.MOE_OK and need <= md.MOE_NOALLOC_SCRATCH_BYTES
    assert md.moe_layer_chain_noalloc(None, 1, [lw], 16, 16, 0, 1, None, stream=0) == md.MOE_E_ARG
    assert md.moe_layer_chain_noalloc(d, 0, [lw], 16, 16, 0, 1, None, stream=0) == md.MOE_E_ARG
    assert md.moe_layer_chain_noalloc(d, 1, [lw], BAD, 16, 0, 1, None, stream=0) == md.MOE_E_ALIGN
    assert md.moe_layer_chain_noalloc(d, 1, [lw], 16, 16, 0, 9, None, stream=0) == md.MOE_E_ARG
