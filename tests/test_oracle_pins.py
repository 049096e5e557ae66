"""Pins of the CPU oracle to things other than itself.

Each check is chosen so that a plausible mistake in the oracle (a dropped term,
a swapped gate/up half, a transposed operand, a wrong sign in silu, a wrong
tie-break, a double rounding) fails at least one of them:
exact rational arithmetic on dyadic inputs, float64 error bounds, brute-force
selection, library routines (torch's bf16 rounding, numpy's stable sort,
scipy's softmax), closed forms and invariants.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import runner
from datagen import workloads as W

U32 = 2.0 ** -24  # unit roundoff of fp32


def bf16_bits_torch(x64):
    """Library rounding: float64 -> bf16 via torch (round to nearest even)."""
    t = torch.tensor(np.asarray(x64, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def f32(bits):
    return oracle.bf16_to_f32(bits)


def to_bf16_bits_exact(vals):
    """bf16 bits of values that are exactly representable in bf16."""
    b = bf16_bits_torch(vals)
    assert np.array_equal(f32(b).astype(np.float64), np.asarray(vals, np.float64))
    return b


def dyadic(rng, shape, lim=16):
    """Values k/8 with |k| <= lim: exact in bf16, products and short sums exact in fp32."""
    return rng.integers(-lim, lim + 1, size=shape) / 8.0


def gamma(n):
    return n * U32 / (1 - n * U32)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_library(rng):
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38], np.float32),
    ])
    # exact halfway cases: bf16 value plus half an ulp (both even and odd neighbours)
    base = f32(rng.integers(0x3F00, 0x4100, 2000).astype(np.uint16))
    half = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, half])
    mine = oracle.f32_to_bf16(vals)
    ref = torch.tensor(vals).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(oracle.cast_bf16(vals), ref)


# ---------------------------------------------------------------- router GEMV

def test_router_logits_exact_on_dyadic_inputs(rng):
    M, H, E = 2, 8, 6
    x = dyadic(rng, (M, H))
    w = dyadic(rng, (E, H))
    lg = oracle.router_logits(to_bf16_bits_exact(x), to_bf16_bits_exact(w))
    for m in range(M):
        for e in range(E):
            exact = sum(Fraction(x[m, h]) * Fraction(w[e, h]) for h in range(H))
            assert Fraction(float(lg[m, e])) == exact


def test_router_logits_within_float64_bound(rng):
    wl = W.C3
    x = W.x_rows(wl, [0] * 3)
    w = W.router(wl)[:64]
    lg = oracle.router_logits(x, w).astype(np.float64)
    xf, wf = f32(x).astype(np.float64), f32(w).astype(np.float64)
    ref = xf @ wf.T
    bound = gamma(wl.H) * (np.abs(xf) @ np.abs(wf).T)
    assert np.all(np.abs(lg - ref) <= bound)
    # a transposed or shifted operand would be far outside the bound
    assert np.abs(lg - ref).max() < 1e-4


# ---------------------------------------------------------------- selection and gates

def test_selection_matches_bruteforce_and_stable_sort(rng):
    E, K = 7, 3
    for trial in range(200):
        lg = rng.integers(-3, 4, size=(1, E)).astype(np.float32)  # many exact ties
        idx, _ = oracle.select_gates(lg, K)
        S = list(idx[0])
        # brute force: exactly one K-subset dominates its complement under
        # (larger logit, then lower index); it must be the oracle's set
        def beats(a, b):
            return lg[0, a] > lg[0, b] or (lg[0, a] == lg[0, b] and a < b)
        winners = [c for c in itertools.combinations(range(E), K)
                   if all(beats(a, b) for a in c for b in range(E) if b not in c)]
        assert len(winners) == 1 and set(winners[0]) == set(S)
        # order: descending logit, lower index first among equals (numpy stable sort)
        assert S == list(np.argsort(-lg[0], kind="stable")[:K])


def test_gates_sum_to_one_and_closed_forms(rng):
    from scipy.special import softmax
    M, E, K = 6, 512, 8
    lg = (rng.standard_normal((M, E)) * 1.0).astype(np.float32)
    idx, g = oracle.select_gates(lg, K)
    assert np.all(np.abs(g.astype(np.float64).sum(1) - 1.0) <= 4 * K * U32)
    sm = softmax(lg.astype(np.float64), axis=1)
    ref = np.take_along_axis(sm, idx, 1)
    ref = ref / ref.sum(1, keepdims=True)
    assert np.all(np.abs(g - ref) <= 1e-6 * ref + 1e-12)
    # K = 1: the renormalised gate is exactly one
    _, g1 = oracle.select_gates(lg, 1)
    assert np.all(g1 == 1.0)
    # K = E: the gates are the full softmax, in selection order
    idxE, gE = oracle.select_gates(lg[:, :16], 16)
    smE = np.take_along_axis(softmax(lg[:, :16].astype(np.float64), axis=1), idxE, 1)
    assert np.all(np.abs(gE - smE) <= 1e-6 * smE)
    # two experts: g0 = 1 / (1 + exp(l1 - l0))
    two = np.array([[0.75, -0.5]], np.float32)
    _, g2 = oracle.select_gates(two, 2)
    assert abs(g2[0, 0] - 1.0 / (1.0 + math.exp(-1.25))) < 1e-7
    # a common shift of every logit leaves the gates unchanged (within rounding)
    _, gs = oracle.select_gates(lg + np.float32(3.0), K)
    assert np.all(np.abs(gs - g) <= 1e-6)



# ---------------------------------------------------------------- router front: selection bias

def test_selection_bias_matches_bruteforce(rng):
    """Selection on fp32(logit + bias), lower index first on equal scores; gates are the
    unbiased softmax renormalised over the chosen set (float64 closed form)."""
    E, K = 9, 3
    for trial in range(200):
        lg = (rng.integers(-6, 7, size=(2, E)) / 4.0).astype(np.float32)
        b = (rng.integers(-3, 4, size=E) / 4.0).astype(np.float32)   # exact sums, many ties
        idx, g = oracle.select_gates(lg, K, b)
        for m in range(2):
            sc = lg[m] + b
            order = sorted(range(E), key=lambda e: (-float(sc[e]), e))
            assert list(idx[m]) == order[:K]
            ex = np.exp(lg[m, idx[m]].astype(np.float64))
            assert np.all(np.abs(g[m] - ex / ex.sum()) <= 1e-6 * ex / ex.sum())


def test_selection_bias_special_cases(rng):
    M, E, K = 4, 512, 8
    lg = rng.standard_normal((M, E)).astype(np.float32)
    idx0, g0 = oracle.select_gates(lg, K)
    # zero bias is no bias, bit for bit
    idxz, gz = oracle.select_gates(lg, K, np.zeros(E, np.float32))
    assert np.array_equal(idxz, idx0) and np.array_equal(gz, g0)
    # a bias that dwarfs the logits selects by bias alone, and the gates are still the
    # unbiased softmax over that set (so they differ from a softmax of the biased scores)
    b = np.zeros(E, np.float32)
    forced = rng.choice(E, K, replace=False)
    b[forced] = 1000.0 + 100.0 * np.arange(K, dtype=np.float32)
    idx, g = oracle.select_gates(lg, K, b)
    assert np.all(idx == forced[np.argsort(-b[forced], kind="stable")][None, :])
    ex = np.exp(lg[:, forced[np.argsort(-b[forced], kind="stable")]].astype(np.float64))
    ref = ex / ex.sum(1, keepdims=True)
    assert np.all(np.abs(g - ref) <= 1e-6 * ref)
    # the gates of a set depend only on the set: same set, same gate per expert
    for m in range(M):
        if set(idx0[m]) == set(idx[m]):
            assert np.allclose(g0[m][np.argsort(idx0[m])], g[m][np.argsort(idx[m])], rtol=1e-6)


# ---------------------------------------------------------------- router front: routed scale

def test_routed_scale_combine_bound_and_power_of_two_exactness(rng):
    """acc = y_shared + s * sum_k g_k y_k: the shared expert is not scaled."""
    wl = W.C1
    x = W.x_rows(wl, [0, 1, 2])
    wr = W.router(wl)
    gu = {e: W.expert_gate_up(wl, 0, e) for e in range(wl.E + 1)}
    d = {e: W.expert_down(wl, 0, e) for e in range(wl.E + 1)}
    idx, gate, _ = oracle.router_topk(x, wr, wl.K)
    s = 2.5
    acc = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 1, s).astype(np.float64)
    for m in range(3):
        ysh = oracle.expert(x[m], gu[wl.E], d[wl.E])[0].astype(np.float64)
        ys = [oracle.expert(x[m], gu[idx[m, k]], d[idx[m, k]])[0].astype(np.float64)
              for k in range(wl.K)]
        R = sum(float(gate[m, k]) * ys[k] for k in range(wl.K))
        T = np.abs(ysh) + s * sum(float(gate[m, k]) * np.abs(ys[k]) for k in range(wl.K))
        assert np.all(np.abs(acc[m] - (ysh + s * R)) <= gamma(wl.K + 3) * T)
        # scaling the shared expert too would be far outside the bound
        assert np.max(np.abs(acc[m] - s * (ysh + R)) - gamma(wl.K + 3) * T) > 0
    # without a shared expert a power-of-two scale commutes with every rounding
    a1 = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 0, 1.0)
    a2 = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 0, 2.0)
    a8 = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 0, -0.125)
    assert np.array_equal(a2, 2 * a1) and np.array_equal(a8, -0.125 * a1)
    # scale zero leaves the shared expert alone
    a0 = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 1, 0.0)
    for m in range(3):
        assert np.array_equal(a0[m], oracle.expert(x[m], gu[wl.E], d[wl.E])[0])


# ---------------------------------------------------------------- router front: norm gain

def test_rmsnorm_gain_product_order_and_special_gains():
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    rng = np.random.default_rng(12)
    H = 2560
    h = bf16_bits_torch(rng.standard_normal((3, H)) * 1.3)
    g = bf16_bits_torch(1.0 + 0.1 * rng.standard_normal(H))
    u = oracle.rmsnorm(h, gain=g)
    hf = f32(h).astype(np.float64)
    for m in range(3):
        ss = sum(Fraction(float(v)) ** 2 for v in hf[m])
        ms = Decimal(ss.numerator) / Decimal(ss.denominator) / H + Decimal(oracle.RMS_EPS)
        r = np.float32(float(1 / ms.sqrt()))
        t = (f32(h[m]) * r).astype(np.float32) * f32(g)          # two fp32 products
        assert np.array_equal(u[m], bf16_bits_torch(t.astype(np.float64)))
    ones = to_bf16_bits_exact(np.ones(H))
    assert np.array_equal(oracle.rmsnorm(h, gain=ones), oracle.rmsnorm(h))
    twos = to_bf16_bits_exact(np.full(H, 2.0))
    assert np.array_equal(f32(oracle.rmsnorm(h, gain=twos)), 2 * f32(oracle.rmsnorm(h)))
    # the gain scales each channel, not each row
    gv = f32(g).astype(np.float64)
    ratio = f32(u).astype(np.float64) / f32(oracle.rmsnorm(h)).astype(np.float64)
    ok = np.abs(f32(oracle.rmsnorm(h))) > 0.05
    assert np.all(np.abs(ratio - gv[None, :])[ok] <= 2 ** -6 * gv[None, :].repeat(3, 0)[ok])


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_exhaustive_over_bf16(rng):
    """All finite bf16 a with b = 1: h = bf16(silu(a)) up to a rounding-boundary tie."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    a = f32(bits)
    finite = np.isfinite(a)
    a = a[finite]
    lib = oracle.lib()
    mine = np.array([lib.oracle_swiglu(float(v), 1.0) for v in a], dtype=np.uint16)
    a64 = a.astype(np.float64)
    with np.errstate(over="ignore"):
        s64 = a64 / (1.0 + np.exp(-a64))
    ref = bf16_bits_torch(s64)
    diff = mine != ref
    # a difference is allowed only where silu lies within two fp32 ulps of a bf16 midpoint
    lo = f32(ref[diff]).astype(np.float64)
    other = f32(mine[diff]).astype(np.float64)
    mid = (lo + other) / 2
    assert np.all(np.abs(s64[diff] - mid) <= 2 * U32 * np.abs(s64[diff]) + 1e-45)
    assert diff.sum() <= 8
    # silu is asymmetric: swapping gate and up, or dropping the minus sign, is caught
    assert lib.oracle_swiglu(-2.0, 1.0) != lib.oracle_swiglu(2.0, 1.0)
    assert oracle.swiglu(2.0, 3.0) != oracle.swiglu(3.0, 2.0)


def test_swiglu_random_pairs_against_float64(rng):
    a = (rng.standard_normal(4000) * 3).astype(np.float32)
    b = (rng.standard_normal(4000) * 3).astype(np.float32)
    mine = np.array([oracle.swiglu(x, y) for x, y in zip(a, b)], dtype=np.uint16)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    v = a64 / (1.0 + np.exp(-a64)) * b64
    ref = bf16_bits_torch(v)
    diff = mine != ref
    assert diff.sum() <= 4
    if diff.any():
        mid = (f32(ref[diff]).astype(np.float64) + f32(mine[diff]).astype(np.float64)) / 2
        assert np.all(np.abs(v[diff] - mid) <= 4 * U32 * np.abs(v[diff]))


# ---------------------------------------------------------------- one expert

def test_expert_gate_up_exact_and_down_within_bound(rng):
    H, I = 8, 4
    x = dyadic(rng, (H,))
    wgu = dyadic(rng, (2 * I, H))
    wd = dyadic(rng, (H, I))
    y, h = oracle.expert(to_bf16_bits_exact(x), to_bf16_bits_exact(wgu), to_bf16_bits_exact(wd))
    for j in range(I):
        a = sum(Fraction(x[k]) * Fraction(wgu[j, k]) for k in range(H))
        b = sum(Fraction(x[k]) * Fraction(wgu[I + j, k]) for k in range(H))
        # a and b are exact fp32 numbers; h must be SwiGLU of exactly these (gate rows first)
        assert h[j] == oracle.swiglu(float(a), float(b))
    hf = f32(h).astype(np.float64)
    for n in range(H):
        exact = sum(Fraction(float(hf[j])) * Fraction(wd[n, j]) for j in range(I))
        terms = sum(abs(float(hf[j]) * wd[n, j]) for j in range(I))
        assert abs(float(y[n]) - float(exact)) <= gamma(I) * terms


def test_identity_like_top1_reduces_to_swiglu_of_input(rng):
    """K=1, zero shared expert, identical routed experts with W_g = W_u = [I | 0]
    and W_d = [I ; 0]: out_n = bf16(silu(x_n) * x_n) for n < I, else 0."""
    H, I, E, K = 64, 16, 4, 1
    x = bf16_bits_torch(rng.standard_normal((2, H)) * 2)
    eye_gu = np.zeros((2 * I, H))
    eye_gu[np.arange(I), np.arange(I)] = 1.0
    eye_gu[I + np.arange(I), np.arange(I)] = 1.0
    eye_d = np.zeros((H, I))
    eye_d[np.arange(I), np.arange(I)] = 1.0
    gu = {e: to_bf16_bits_exact(eye_gu) for e in range(E)}
    d = {e: to_bf16_bits_exact(eye_d) for e in range(E)}
    gu[E] = np.zeros((2 * I, H), np.uint16)
    d[E] = np.zeros((H, I), np.uint16)
    wr = bf16_bits_torch(rng.standard_normal((E, H)) * 0.02)
    idx, gate, _ = oracle.router_topk(x, wr, K)
    assert np.all(gate == 1.0)
    out = oracle.cast_bf16(oracle.experts_combine(x, idx, gate, gu, d, E, 1))
    xf = f32(x).astype(np.float64)
    ref = bf16_bits_torch(xf[:, :I] / (1.0 + np.exp(-xf[:, :I])) * xf[:, :I])
    assert np.mean(out[:, :I] == ref) > 0.97
    mism = out[:, :I] != ref
    assert np.all(np.abs(f32(out[:, :I][mism]) - f32(ref[mism])) <=
                  np.abs(f32(ref[mism])) * 2.0 ** -7)
    assert np.all(f32(out[:, I:]) == 0.0)


def test_top1_identical_experts_is_a_dense_swiglu_mlp(rng):
    H, I, E = 256, 64, 8
    wl = W.C1
    x = W.x_rows(wl, [0, 1])
    wgu = W.expert_gate_up(wl, 0, 0)
    wd = W.expert_down(wl, 0, 0)
    gu = {e: wgu for e in range(E)}
    d = {e: wd for e in range(E)}
    wr = W.router(wl)[:E]
    idx, gate, _ = oracle.router_topk(x, wr, 1)
    acc = oracle.experts_combine(x, idx, gate, gu, d, E, 0)
    xf, gf, df = f32(x).astype(np.float64), f32(wgu).astype(np.float64), f32(wd).astype(np.float64)
    for m in range(2):
        a = gf[:I] @ xf[m]
        b = gf[I:] @ xf[m]
        h_ref = bf16_bits_torch(a / (1 + np.exp(-a)) * b)
        y, h = oracle.expert(x[m], wgu, wd)
        assert np.mean(h == h_ref) > 0.98          # rare 1-ulp flips at rounding boundaries
        hf = f32(h).astype(np.float64)
        ref = df @ hf
        assert np.all(np.abs(y - ref) <= gamma(I) * (np.abs(df) @ np.abs(hf)))
        assert np.array_equal(acc[m], y)           # gate 1, no shared expert: acc = 0 + 1*y


# ---------------------------------------------------------------- combine invariants

def _tiny_layer(rng, S=1, zero_x=False, M=2):
    wl = W.C1
    x = np.zeros((M, wl.H), np.uint16) if zero_x else W.x_rows(wl, list(range(M)))
    return wl, x


def test_zero_input_gives_zero_output():
    wl = W.C1
    x = np.zeros((3, wl.H), np.uint16)
    r = runner.layer(wl, x)
    assert np.all(r["idx"] == np.arange(wl.K)[None, :])    # all logits tie at +0
    assert np.all(r["gate"] == np.float32(1.0 / wl.K))
    assert np.all(r["acc"] == 0.0)
    out = runner.layer_output(wl, r)
    assert np.all((out == 0x0000) | (out == 0x8000))


def test_identical_routed_experts_make_output_independent_of_router(rng):
    wl = W.C1
    x = W.x_rows(wl, [0, 1])
    wgu = W.expert_gate_up(wl, 0, 3)
    wd = W.expert_down(wl, 0, 3)
    gu = {e: wgu for e in range(wl.E)}
    d = {e: wd for e in range(wl.E)}
    gu[wl.E] = W.expert_gate_up(wl, 0, wl.E)
    d[wl.E] = W.expert_down(wl, 0, wl.E)
    outs = []
    for K, seed_layer in ((1, 0), (2, 0), (4, 1), (8, 2)):
        wr = W.router(wl, seed_layer)
        idx, gate, _ = oracle.router_topk(x, wr, K)
        outs.append(oracle.experts_combine(x, idx, gate, gu, d, wl.E, 1).astype(np.float64))
    y_sh = np.stack([oracle.expert(x[m], gu[wl.E], d[wl.E])[0] for m in range(2)])
    y_r = np.stack([oracle.expert(x[m], wgu, wd)[0] for m in range(2)])
    scale = np.abs(y_sh) + np.abs(y_r)
    for o in outs:
        assert np.all(np.abs(o - (y_sh + y_r)) <= 24 * U32 * scale + 1e-30)


def test_expert_permutation_with_index_remap(rng):
    wl = W.C1
    x = W.x_rows(wl, [0, 1, 2])
    wr = W.router(wl)
    gu = {e: W.expert_gate_up(wl, 0, e) for e in range(wl.E + 1)}
    d = {e: W.expert_down(wl, 0, e) for e in range(wl.E + 1)}
    idx, gate, _ = oracle.router_topk(x, wr, wl.K)
    acc = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 1)
    perm = rng.permutation(wl.E)
    wr_p = np.empty_like(wr)
    wr_p[perm] = wr
    gu_p = {int(perm[e]): gu[e] for e in range(wl.E)}
    d_p = {int(perm[e]): d[e] for e in range(wl.E)}
    gu_p[wl.E], d_p[wl.E] = gu[wl.E], d[wl.E]
    idx_p, gate_p, _ = oracle.router_topk(x, wr_p, wl.K)
    assert np.array_equal(idx_p, perm[idx])
    assert np.all(np.abs(gate_p - gate) <= 4 * U32 * gate)
    acc_p = oracle.experts_combine(x, idx_p, gate_p, gu_p, d_p, wl.E, 1)
    # the gates may move by a few ulps (the softmax sum runs in the new index
    # order); bound the change by the magnitude of the terms being combined
    for m in range(3):
        T = np.abs(oracle.expert(x[m], gu[wl.E], d[wl.E])[0]).astype(np.float64)
        for k in range(wl.K):
            T += gate[m, k] * np.abs(oracle.expert(x[m], gu[idx[m, k]], d[idx[m, k]])[0])
        assert np.all(np.abs(acc_p[m] - acc[m]) <= 8 * (wl.K + 1) * U32 * T)


def test_rows_are_independent():
    wl = W.C1
    x = W.x_rows(wl, list(range(6)))
    full = runner.layer(wl, x)
    for m in range(6):
        one = runner.layer(wl, x[m:m + 1])
        assert np.array_equal(one["idx"][0], full["idx"][m])
        assert np.array_equal(one["gate"][0], full["gate"][m])
        assert np.array_equal(one["acc"][0], full["acc"][m])


def test_tp_shards_sum_to_full_layer():
    from dataclasses import replace
    full_wl = replace(W.C1, M=3, x_seed=777)
    x = W.x_rows(full_wl, [0, 1, 2])
    full = runner.layer(full_wl, x)
    parts = []
    for r in range(4):
        sh = replace(full_wl, I=16, n_shards=4, shard=r, out_f32=True)
        parts.append(runner.layer(sh, x)["acc"].astype(np.float64))
        assert np.array_equal(runner.layer(sh, x)["idx"], full["idx"])
    tot = sum(parts)
    ref = full["acc"].astype(np.float64)
    scale = sum(np.abs(p) for p in parts) + np.abs(ref)
    assert np.all(np.abs(tot - ref) <= 64 * 12 * U32 * scale + 1e-9)


def test_thread_count_does_not_change_results():
    wl = W.C1
    x = W.x_rows(wl, [0, 1, 2])
    oracle.set_threads(1)
    a = runner.layer(wl, x)
    w = W.lmhead_rows(W.C5, 0, 3000)
    h = W.x_rows(W.C5, [0, 1])
    t1 = oracle.lmhead_argmax(h, w)
    oracle.set_threads(4)
    b = runner.layer(wl, x)
    t4 = oracle.lmhead_argmax(h, w)
    oracle.set_threads(os.cpu_count() or 1)
    assert np.array_equal(a["acc"], b["acc"]) and np.array_equal(a["gate"], b["gate"])
    assert np.array_equal(t1[0], t4[0]) and np.array_equal(t1[1], t4[1])


# ---------------------------------------------------------------- residual chain

def test_residual_rounds_once():
    rng = np.random.default_rng(5)
    h = bf16_bits_torch(rng.standard_normal(5000))
    acc = (rng.standard_normal(5000) * 0.05).astype(np.float32)
    out = oracle.residual(h, acc)
    v = f32(h).astype(np.float64) + acc.astype(np.float64)
    ref = bf16_bits_torch(v)
    diff = out != ref
    assert diff.sum() <= 3   # only where fp32 rounding of h + acc lands on a bf16 midpoint
    assert np.array_equal(oracle.residual(h, np.zeros(5000, np.float32)), h)


def test_rmsnorm_scale_is_the_correctly_rounded_exact_value():
    """r must be the fp32 rounding of 1/sqrt(exact mean square + eps), and u = bf16(h * r)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    rng = np.random.default_rng(11)
    H = 2560
    h = bf16_bits_torch(rng.standard_normal((4, H)) * 1.7)
    u = oracle.rmsnorm(h)
    hf = f32(h).astype(np.float64)
    for m in range(4):
        ss = sum(Fraction(float(v)) ** 2 for v in hf[m])
        ms = Decimal(ss.numerator) / Decimal(ss.denominator) / H + Decimal(oracle.RMS_EPS)
        r = np.float32(float(1 / ms.sqrt()))
        ref = bf16_bits_torch((f32(h[m]) * r).astype(np.float64))   # fp32 product, then bf16
        assert np.array_equal(u[m], ref)
    # unit mean square after the norm; a constant row maps to (about) +-1
    uf = f32(u).astype(np.float64)
    assert np.all(np.abs((uf ** 2).mean(1) - 1) < 0.01)
    c = bf16_bits_torch(np.full((2, 256), [[1.0], [-3.0]]))
    assert np.all(f32(oracle.rmsnorm(c)) == np.array([[1.0], [-1.0]], np.float32))


def test_chain_with_zero_weights_is_identity():
    wl = W.C1
    x = W.x_rows(wl, [0, 1])
    zero_gu = {e: np.zeros((2 * wl.I, wl.H), np.uint16) for e in range(wl.E + 1)}
    zero_d = {e: np.zeros((wl.H, wl.I), np.uint16) for e in range(wl.E + 1)}
    h = x
    for _ in range(3):
        idx, gate, _ = oracle.router_topk(h, np.zeros((wl.E, wl.H), np.uint16), wl.K)
        acc = oracle.experts_combine(h, idx, gate, zero_gu, zero_d, wl.E, 1)
        h = oracle.residual(h, acc)
    assert np.array_equal(h, x)


# ---------------------------------------------------------------- lm_head argmax

def test_argmax_exact_with_ties_goes_to_lowest_index(rng):
    M, H, V = 3, 8, 50
    hx = dyadic(rng, (M, H), lim=4)
    w = dyadic(rng, (V, H), lim=4)
    w[37] = w[11]           # planted exact tie: the lower index must win
    w[11] = np.abs(w[11]) + 0.0
    w[37] = w[11]
    hx[:, :] = np.abs(hx)   # nonnegative h makes rows 11/37 large
    tok, mx = oracle.lmhead_argmax(to_bf16_bits_exact(hx), to_bf16_bits_exact(w))
    for m in range(M):
        z = [sum(Fraction(hx[m, k]) * Fraction(w[v, k]) for k in range(H)) for v in range(V)]
        best = max(z)
        assert tok[m] == z.index(best) and Fraction(float(mx[m])) == best


def test_argmax_matches_float64_when_margin_is_clear():
    wl = W.C5
    w = W.lmhead_rows(wl, 0, 20000)
    h = W.x_rows(wl, [0, 1, 2, 3])
    tok, _ = oracle.lmhead_argmax(h, w)
    z = f32(h).astype(np.float64) @ f32(w).astype(np.float64).T
    srt = -np.sort(-z, axis=1)
    for m in range(4):
        if srt[m, 0] - srt[m, 1] > 1e-3:
            assert tok[m] == int(np.argmax(z[m]))


# ---------------------------------------------------------------- byte counts vs the pages

def test_byte_counts_match_the_numbers_the_pages_print():
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")) as f:
        pc = json.load(f)
    wl = W.C2
    assert (wl.H, wl.E, wl.S, wl.K, wl.I) == (pc["hidden_size"]["value"], pc["routed_experts"]["value"],
                                              pc["shared_experts"]["value"], pc["top_k"]["value"],
                                              pc["moe_intermediate_size"]["value"])
    assert abs(wl.V if wl.V else W.C5.V - pc["vocab_approx"]["value"]) <= \
        pc["vocab_approx"]["rel_tol"] * pc["vocab_approx"]["value"]
    assert abs(wl.router_bytes() / 1e6 - pc["router_weight_mb_bf16"]["value"]) <= \
        pc["router_weight_mb_bf16"]["abs_tol"]
    # one token routed to 8 distinct experts reads about 94 MB of expert weights
    idx = np.arange(8, dtype=np.int32)[None, :] * 3
    b, U = oracle.unique_weight_bytes(wl.H, wl.E, wl.K, wl.I, 0, idx, include_router=False)
    assert U == 8 and abs(b / 1e6 - pc["activated_expert_mb_per_layer"]["value"]) <= \
        pc["activated_expert_mb_per_layer"]["abs_tol"]
    # MoE weights of all layers on one of four ranks: about 63 GB
    per_rank = pc["layers"]["value"] * wl.layer_bytes() / pc["tp_degree"]["value"] / 1e9
    assert abs(per_rank / pc["weights_gb_per_rank_tp4"]["value"] - 1) <= \
        pc["weights_gb_per_rank_tp4"]["rel_tol"]
    # the shard's intermediate size is a quarter of 768
    assert W.C4.I * pc["tp_degree"]["value"] == pc["moe_intermediate_size"]["value"]
    assert W.C3.M == pc["verify_rows"]["value"] and W.C3.M <= pc["max_rows_per_tile"]["value"]
    # full M=1 layer call: router + 8 experts + shared expert
    b1, _ = oracle.unique_weight_bytes(wl.H, wl.E, wl.K, wl.I, 1, idx, include_router=True)
    assert b1 == 108_789_760


# ---------------------------------------------------------------- fp8 block-128 experts

def _f8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)


def test_fp8_decode_matches_library():
    c = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_decode(c)
    ref = _f8(c).float().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))   # -0 stays -0


def _finite_codes(rng, shape):
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C                      # no NaN codes
    return q


def test_fp8_dequant_block_indexing_and_rounding(rng):
    rows, cols = 384, 256                             # 3 x 2 blocks: a transposed index fails
    q = _finite_codes(rng, (rows, cols))
    dec = _f8(q).double()
    # unit scales: the codes' values; power-of-two scales: exact scaling per block
    assert np.array_equal(oracle.dequant_fp8(q, np.ones((3, 2), np.float32)), dec.float().numpy())
    p2 = np.array([[0.5, 4.0], [2.0 ** -12, 1.0], [8.0, 0.25]], np.float32)
    big = np.kron(p2, np.ones((128, 128))).astype(np.float64)
    assert np.array_equal(oracle.dequant_fp8(q, p2), (dec.numpy() * big).astype(np.float32))
    # arbitrary scales: the exact product rounded once to fp32 (library float64 -> float32)
    s = (rng.random((3, 2)) * 1e-3 + 1e-4).astype(np.float32)
    full = torch.from_numpy(np.kron(s.astype(np.float64), np.ones((128, 128))))
    assert np.array_equal(oracle.dequant_fp8(q, s), (dec * full).float().numpy())


def test_fp8_expert_with_unit_scales_is_the_bf16_expert(rng):
    """Codes are exact in bf16 and every product of a bf16 input and a code value is exact
    in fp32, so with unit scales the fp8 expert must equal the pinned bf16 expert bit for bit."""
    H, I = 256, 128
    x = W.x_rows(W.C8, [0])[0]
    qgu = _finite_codes(rng, (2 * I, H)) & 0xBF        # exponent field <= 7: |v| < 2
    qd = _finite_codes(rng, (H, I)) & 0xBF
    one_gu, one_d = np.ones((2, 2), np.float32), np.ones((2, 1), np.float32)
    y8, h8 = oracle.expert_fp8(x, qgu, one_gu, qd, one_d)
    wgu = to_bf16_bits_exact(_f8(qgu).double().numpy())
    wd = to_bf16_bits_exact(_f8(qd).double().numpy())
    y, h = oracle.expert(x, wgu, wd)
    assert np.array_equal(h8, h) and np.array_equal(y8, y)


def test_fp8_expert_within_float64_bound_with_block_scales(rng):
    wl = W.C8
    x = W.x_rows(wl, [1])[0]
    (qgu, sgu), (qd, sd) = W.expert_gate_up_fp8(wl, 0, 4), W.expert_down_fp8(wl, 0, 4)
    y, h = oracle.expert_fp8(x, qgu, sgu, qd, sd)
    wgu = _f8(qgu).double().numpy() * np.kron(sgu.astype(np.float64), np.ones((128, 128)))
    wd = _f8(qd).double().numpy() * np.kron(sd.astype(np.float64), np.ones((128, 128)))
    xf = f32(x).astype(np.float64)
    a, b = wgu[:wl.I] @ xf, wgu[wl.I:] @ xf
    h_ref = bf16_bits_torch(a / (1 + np.exp(-a)) * b)
    assert np.mean(h == h_ref) > 0.97
    mism = h != h_ref
    assert np.all(np.abs(f32(h[mism]) - f32(h_ref[mism])) <= np.abs(f32(h_ref[mism])) * 2.0 ** -7)
    hf = f32(h).astype(np.float64)
    # the oracle's down weights are the dequantised values rounded once to fp32
    ref = wd @ hf
    bound = (gamma(wl.I) + 2 * U32) * (np.abs(wd) @ np.abs(hf))
    assert np.all(np.abs(y - ref) <= bound)
    # a block scale applied to the wrong block would be far outside the bound
    wd_t = _f8(qd).double().numpy() * np.kron(sd.astype(np.float64)[::-1], np.ones((128, 128)))
    assert np.max(np.abs(y - wd_t @ hf) - bound) > 0


def test_fp8_combine_with_unit_scales_is_the_bf16_combine(rng):
    wl = W.C8
    x = W.x_rows(wl, [0, 1, 2])
    idx, gate, _ = oracle.router_topk(x, W.router(wl), wl.K)
    gu8, d8, gu, d = {}, {}, {}, {}
    for e in sorted(set(idx.ravel().tolist())) + [wl.E]:
        qgu = _finite_codes(rng, (2 * wl.I, wl.H)) & 0xBF
        qd = _finite_codes(rng, (wl.H, wl.I)) & 0xBF
        gu8[e], d8[e] = (qgu, np.ones((2, 2), np.float32)), (qd, np.ones((2, 1), np.float32))
        gu[e] = to_bf16_bits_exact(_f8(qgu).double().numpy())
        d[e] = to_bf16_bits_exact(_f8(qd).double().numpy())
    for scale in (1.0, 2.5):
        a8 = oracle.experts_combine_fp8(x, idx, gate, gu8, d8, wl.E, 1, scale)
        a = oracle.experts_combine(x, idx, gate, gu, d, wl.E, 1, scale)
        assert np.array_equal(a8, a)


# ---------------------------------------------------------------- chain and router-front compositions
#
# runner.chain and runner.front_layer decide where the norm sits, what feeds the
# router and the experts, and what the residual adds to.  They are pinned with
# identity-like experts, whose layer output has a closed form (every sum has one
# nonzero term), and with zero experts, whose chain must return its input.

def _identity_experts(monkeypatch, H, I, E, shared_zero=True):
    """Every routed expert: W_g = W_u = [I_I | 0], W_d = [I_I ; 0]; the shared one zero."""
    eye_gu = np.zeros((2 * I, H))
    eye_gu[np.arange(I), np.arange(I)] = 1.0
    eye_gu[I + np.arange(I), np.arange(I)] = 1.0
    eye_d = np.zeros((H, I))
    eye_d[np.arange(I), np.arange(I)] = 1.0
    gu_bits, d_bits = to_bf16_bits_exact(eye_gu), to_bf16_bits_exact(eye_d)

    def gu(wl, layer, e):
        return np.zeros((2 * I, H), np.uint16) if (e == E and shared_zero) else gu_bits

    def dn(wl, layer, e):
        return np.zeros((H, I), np.uint16) if (e == E and shared_zero) else d_bits

    monkeypatch.setattr(W, "expert_gate_up", gu)
    monkeypatch.setattr(W, "expert_down", dn)


def _swiglu_self_closed_form(u, I):
    """bf16(silu(u_n) * u_n) for n < I, 0 beyond: the identity-like top-1 layer output,
    in float64 rounded once to bf16 (rare 1-ulp differences from the fp32 path)."""
    uf = f32(u).astype(np.float64)
    s = np.zeros_like(uf)
    s[:, :I] = uf[:, :I] / (1.0 + np.exp(-uf[:, :I])) * uf[:, :I]
    return bf16_bits_torch(s)


def _tiny_front_wl(**kw):
    from dataclasses import replace
    a = dict(name="tiny_chain_pin", K=1, M=3, n_layers=3, residual=True, prenorm=True,
             bias_sigma=0.0, gain_sigma=0.1, routed_scale=1.0)
    a.update(kw)
    return replace(W.C6, **a)


def test_runner_chain_with_zero_experts_returns_its_input(monkeypatch):
    """All expert weights zero: every layer adds an exact +-0, so h_L = x bit for bit,
    with and without the pre-norm (and whatever the router chooses)."""
    wl = _tiny_front_wl(K=2, bias_sigma=0.25, routed_scale=2.5)
    monkeypatch.setattr(W, "expert_gate_up",
                        lambda wl_, layer, e: np.zeros((2 * wl_.I, wl_.H), np.uint16))
    monkeypatch.setattr(W, "expert_down",
                        lambda wl_, layer, e: np.zeros((wl_.H, wl_.I), np.uint16))
    x = W.x_rows(wl, [0, 1, 2])
    for prenorm in (True, False):
        h, per = runner.chain(wl, x, prenorm=prenorm)
        assert np.array_equal(h, x)
        assert len(per) == wl.n_layers
        for r in per:
            assert np.array_equal(r["h_in"], x)
            assert np.all(r["acc"] == 0.0)


def test_runner_chain_identity_experts_closed_form(monkeypatch):
    """Identity-like top-1 experts with a zero shared expert and per-layer gains: layer l
    must (i) norm h_l with layer l's gain, (ii) feed that u_l to the router (its logits)
    and to the experts (acc = bf16(silu(u)*u) on the first I channels), and (iii) add acc
    to h_l, not to u_l.  The input is scaled by 3, so u_l differs from h_l and each wrong
    composition fails."""
    wl = _tiny_front_wl()
    _identity_experts(monkeypatch, wl.H, wl.I, wl.E)
    x = bf16_bits_torch(f32(W.x_rows(wl, [0, 1, 2])).astype(np.float64) * 3.0)
    h, per = runner.chain(wl, x)
    assert np.array_equal(per[0]["h_in"], x)
    close = 0
    for l, r in enumerate(per):
        hl = r["h_in"]
        gain = W.norm_gain(wl, l)
        # each layer has a gain of its own, so a gain taken from the wrong layer fails
        assert gain is not None and np.any(gain != W.norm_gain(wl, (l + 1) % wl.n_layers))
        u = oracle.rmsnorm(hl, gain=gain)
        assert np.array_equal(r["u_in"], u)
        assert not np.array_equal(u, hl)
        # the router sees u (its logits), not h
        assert np.array_equal(r["logits"], oracle.router_logits(u, W.router(wl, l)))
        assert not np.allclose(r["logits"], oracle.router_logits(hl, W.router(wl, l)))
        assert np.all(r["gate"] == 1.0)
        # the experts see u: acc is the closed form of u (to one bf16 ulp where the
        # float64 and fp32 roundings of silu(u)*u part)
        ref = _swiglu_self_closed_form(u, wl.I)
        acc_bits = bf16_bits_torch(r["acc"].astype(np.float64))
        assert np.all(f32(acc_bits[:, wl.I:]) == 0.0)
        same = acc_bits == ref
        assert same.mean() > 0.97
        assert np.all(np.abs(f32(acc_bits[~same]) - f32(ref[~same])) <=
                      np.abs(f32(ref[~same])) * 2.0 ** -7)
        # the residual adds acc to h_l (exact sums of two bf16 values, rounded once)
        nxt = per[l + 1]["h_in"] if l + 1 < len(per) else h
        want = bf16_bits_torch(f32(hl).astype(np.float64) + r["acc"].astype(np.float64))
        close += int(np.sum(nxt == want))
        assert np.mean(nxt == want) > 0.99
        wrong = bf16_bits_torch(f32(u).astype(np.float64) + r["acc"].astype(np.float64))
        assert np.mean(nxt == wrong) < 0.5
    assert close > 0


def test_runner_chain_one_layer_and_three_layers_by_hand():
    """With real random weights, a selection bias, per-layer gains and a routed scale:
    chain(L=1) = residual(x, layer(rmsnorm(x, gain_0)).acc), and three layers composed
    by hand from the pinned oracle functions equal chain(L=3) bit for bit."""
    wl = _tiny_front_wl(K=2, bias_sigma=0.25, routed_scale=2.5)
    x = W.x_rows(wl, [0, 1, 2])
    h1, per1 = runner.chain(wl, x, n_layers=1)
    u0 = oracle.rmsnorm(x, gain=W.norm_gain(wl, 0))
    idx, gate, _ = oracle.router_topk(u0, W.router(wl, 0), wl.K, W.router_bias(wl, 0))
    gu = {e: W.expert_gate_up(wl, 0, e) for e in range(wl.E + 1)}
    d = {e: W.expert_down(wl, 0, e) for e in range(wl.E + 1)}
    acc = oracle.experts_combine(u0, idx, gate, gu, d, wl.E, wl.S, wl.routed_scale)
    assert np.array_equal(per1[0]["idx"], idx)
    assert np.array_equal(per1[0]["acc"], acc)
    assert np.array_equal(h1, oracle.residual(x, acc))
    # the residual must not be taken on u
    assert not np.array_equal(h1, oracle.residual(u0, acc))
    h = x
    for l in range(3):
        u = oracle.rmsnorm(h, gain=W.norm_gain(wl, l))
        idx, gate, _ = oracle.router_topk(u, W.router(wl, l), wl.K, W.router_bias(wl, l))
        gu = {e: W.expert_gate_up(wl, l, e) for e in range(wl.E + 1)}
        d = {e: W.expert_down(wl, l, e) for e in range(wl.E + 1)}
        h = oracle.residual(h, oracle.experts_combine(u, idx, gate, gu, d, wl.E, wl.S,
                                                      wl.routed_scale))
    h3, _ = runner.chain(wl, x, n_layers=3)
    assert np.array_equal(h3, h)
    # without the pre-norm the layers see h itself
    h_plain, per_plain = runner.chain(wl, x, n_layers=1, prenorm=False)
    idx, gate, _ = oracle.router_topk(x, W.router(wl, 0), wl.K, W.router_bias(wl, 0))
    gu = {e: W.expert_gate_up(wl, 0, e) for e in range(wl.E + 1)}
    d = {e: W.expert_down(wl, 0, e) for e in range(wl.E + 1)}
    assert np.array_equal(h_plain, oracle.residual(
        x, oracle.experts_combine(x, idx, gate, gu, d, wl.E, wl.S, wl.routed_scale)))


def test_runner_front_layer_feeds_the_same_normed_input_to_router_and_experts(monkeypatch):
    """front_layer: the router's logits are those of u = bf16(RMSNorm(x) * gain), and the
    experts read u too: with identity-like experts, channels the gain zeroes come out 0
    while the others follow the closed form of u.  With unit gain it is layer(rmsnorm(x))."""
    from dataclasses import replace
    wl = _tiny_front_wl(n_layers=1)
    _identity_experts(monkeypatch, wl.H, wl.I, wl.E)
    x = bf16_bits_torch(f32(W.x_rows(wl, [0, 1, 2])).astype(np.float64) * 3.0)
    gain = np.array(W.norm_gain(wl, 0), copy=True)
    gain[:8] = 0                                    # bf16 +0: these channels of u vanish
    monkeypatch.setattr(W, "norm_gain", lambda wl_, layer=0: gain)
    r = runner.front_layer(wl, x)
    u = oracle.rmsnorm(x, gain=gain)
    assert np.array_equal(r["u_in"], u)
    assert np.array_equal(r["logits"], oracle.router_logits(u, W.router(wl, 0)))
    acc_bits = bf16_bits_torch(r["acc"].astype(np.float64))
    assert np.all(r["acc"][:, :8] == 0.0)
    assert np.all(f32(x[:, :8]) != 0.0)                # x itself is nonzero there
    ref = _swiglu_self_closed_form(u, wl.I)
    assert np.mean(acc_bits == ref) > 0.97
    # unit gain: front_layer is the plain layer on rmsnorm(x); a workload without the
    # pre-norm passes x through unchanged
    monkeypatch.undo()
    wl1 = replace(_tiny_front_wl(n_layers=1, K=2, bias_sigma=0.25), gain_sigma=0.0)
    x1 = W.x_rows(wl1, [0, 1, 2])
    a = runner.front_layer(wl1, x1)
    b = runner.layer(wl1, oracle.rmsnorm(x1))
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["acc"], b["acc"])
    wl0 = replace(wl1, prenorm=False)
    c = runner.front_layer(wl0, x1)
    assert np.array_equal(c["u_in"], x1)
    assert np.array_equal(c["acc"], runner.layer(wl0, x1)["acc"])
