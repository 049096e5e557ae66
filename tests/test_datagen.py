"""The seeded generator: published SplitMix64 outputs, slicing, and the value distribution."""
import numpy as np

import datagen
from datagen import workloads as W


def _mix64(z):
    M = (1 << 64) - 1
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
    return z ^ (z >> 31)


def test_splitmix64_published_outputs():
    # SplitMix64 seeded with 0 yields 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, ...;
    # dg_ih12(key, n) consumes outputs at key + GAMMA * (3n + t + 1), so with key 0
    # and n = 0 the first 16-bit digits come from exactly those outputs.
    G = 0x9E3779B97F4A7C15
    assert _mix64(G) == 0xE220A8397B1DCDAF
    assert _mix64((2 * G) & ((1 << 64) - 1)) == 0x6E789E6AA1B965F4
    s = 0
    for t in range(3):
        r = _mix64((G * (t + 1)) & ((1 << 64) - 1))
        s += sum((r >> (16 * q)) & 0xFFFF for q in range(4))
    assert datagen.ih12(0, 0) == s - 6 * 65535


def test_slices_agree_with_full_tensor():
    k = datagen.key(7, 1, 2, 3, 4, 5)
    full = datagen.fill_host(k, 40, 96, 0.02)
    part = datagen.fill_host(k, 10, 24, 0.02, row0=13, col0=48, ld_full=96)
    assert np.array_equal(part, full[13:23, 48:72])


def test_keys_are_distinct():
    ks = {datagen.key(1, f, l, t, e, a) for f in (1, 2) for l in range(3) for t in range(1, 6)
          for e in range(4) for a in range(2)}
    assert len(ks) == 2 * 3 * 5 * 4 * 2


def test_distribution_mean_std_support():
    k = datagen.key(99, 2, 0, 3, 0)
    a = datagen.fill_host(k, 512, 2048, 0.02)
    f = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f.mean()) < 0.02 * 0.01
    assert abs(f.std() / 0.02 - 1.0) < 0.01
    assert np.abs(f).max() <= 6 * 0.02 * 1.01
    # near-normal shape: fraction within one sigma close to 68.3 %
    assert abs(np.mean(np.abs(f) < 0.02) - 0.6827) < 0.01


def test_shard_slices_are_quarters_of_the_full_expert():
    full = W.expert_gate_up(W.C3, 0, 5)
    sh = W.expert_gate_up(W.C4, 0, 5)
    assert np.array_equal(sh[:192], full[:192])
    assert np.array_equal(sh[192:], full[768:768 + 192])
    assert np.array_equal(W.expert_down(W.C4, 0, 5), W.expert_down(W.C3, 0, 5)[:, :192])


def _torch_e4m3(v32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_codes_round_like_the_library():
    """dg_e4m3_code(s, mul) is the round-to-nearest-even e4m3 code of s * mul / 65536,
    saturated at 448: checked against torch's float32 -> float8_e4m3fn cast (exact
    float32 inputs only, below torch's NaN threshold of 480)."""
    k = datagen.key(5, 2, 0, datagen.TENSOR_GATE_UP_FP8, 1)
    s = np.array([datagen.ih12(k, n) for n in range(4000)], dtype=np.int64)
    for mul in (1, 100, 255):
        v = s * mul
        ok = np.abs(v) < (1 << 24)                 # exact in float32
        v32 = (v[ok].astype(np.float64) / 65536.0).astype(np.float32)
        keep = np.abs(v32) < 480
        mine = np.array([datagen.e4m3_code(int(a), mul) for a in s[ok][keep]], np.uint8)
        assert np.array_equal(mine, _torch_e4m3(v32[keep]))
    # midpoints round to the even code; zero keeps its sign; large values saturate
    mids = [(69632, 1), (-69632, 1), (65536 * 9 // 16 * 16 + 65536 // 32, 1), (1, 1)]
    for si, mul in mids:
        v32 = np.float32(si * mul / 65536.0)
        assert datagen.e4m3_code(si, mul) == int(_torch_e4m3(np.array([v32]))[0])
    assert datagen.e4m3_code(0, 100) == 0
    assert datagen.e4m3_code(480 * 65536, 1) == 0x7E
    assert datagen.e4m3_code(-10 ** 9, 1) == 0xFE
    assert datagen.e4m3_code(464 * 65536, 1) == 0x7E     # midpoint 448 / 480 goes to even 448


def test_fp8_slices_distribution_and_scales():
    k = datagen.key(7, 2, 0, datagen.TENSOR_DOWN_FP8, 3)
    full = datagen.fill_host_fp8(k, 64, 512)
    assert np.array_equal(datagen.fill_host_fp8(k, 8, 128, row0=5, col0=256, ld_full=512),
                          full[5:13, 256:384])
    import torch
    v = torch.from_numpy(full).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert not np.isnan(v).any()
    assert abs(v.std() / datagen.FP8_MUL - 1.0) < 0.03
    q, sc = W.expert_gate_up_fp8(W.C8, 0, 2)
    assert q.shape == (256, 256) and sc.shape == (2, 2)
    assert np.all(np.abs(sc / (0.02 / datagen.FP8_MUL) - 1.0) < 0.2)
