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
