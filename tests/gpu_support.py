"""Shared helpers of the GPU tests: device weights, tie-free inputs, comparisons."""
import json
import os
import sys

import numpy as np

from datagen import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))

_TIEFREE = None


def tiefree_attempts(wl, n=None):
    global _TIEFREE
    if _TIEFREE is None:
        with open(os.path.join(HERE, "golden", "tiefree_rows.json")) as f:
            _TIEFREE = json.load(f)
    a = _TIEFREE["workloads"][wl.name]
    return a if n is None else a[:n]


def x_tiefree(wl, M):
    return W.x_rows(wl, tiefree_attempts(wl, M))


def say(msg):
    """Name the case before each GPU step (flushed, so a lost box still shows it)."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rel_err_normwise(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i|  (the 1e-2 bar for bf16 outputs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def frac_beyond_one_ulp(got_bits, ref_bits, floor_rel=1e-3):
    """Fraction of bf16 elements that differ by more than one bf16 ulp of the
    reference (plus floor_rel * max|ref|): a stricter diagnostic than the bar."""
    g = f32(got_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    ulp = np.abs(r) * 2.0 ** -7
    tol = ulp + floor_rel * np.abs(r).max()
    return float(np.mean(np.abs(g - r) > tol))


def same_sets(a, b):
    return np.array_equal(np.sort(np.asarray(a), axis=-1), np.sort(np.asarray(b), axis=-1))


def order_agrees(gpu_idx, ref_idx, logits, min_gap=1e-5):
    """Ranks agree wherever the reference's adjacent logits are min_gap apart."""
    for m in range(ref_idx.shape[0]):
        lv = logits[m, ref_idx[m]]
        for k in range(ref_idx.shape[1]):
            lo = lv[k] - lv[k + 1] if k + 1 < ref_idx.shape[1] else np.inf
            hi = lv[k - 1] - lv[k] if k > 0 else np.inf
            if min(lo, hi) >= min_gap and gpu_idx[m, k] != ref_idx[m, k]:
                return False
    return True


def free_running_report(wl, x, ids_gpu, h_gpu, tok_gpu, lm_host, routers=None, tag=""):
    """Compare a free-running GPU chain with the oracle's free-running chain from the
    same input rows (no teacher forcing): per row, the first layer whose selected expert
    set differs, the norm-wise error of the final hidden state, and whether the greedy
    tokens agree.  Reported, not gated: the method gives no error bound across a chain,
    and a single bf16 ulp that flips one selection makes the two runs part ways.
    The report is printed and, when MOE_RESULTS_DIR is set, written there as JSON."""
    import oracle
    from oracle import runner
    h_ref, per = runner.chain(wl, x, routers=routers)
    tok_ref, _ = oracle.lmhead_argmax(h_ref, lm_host)
    rows = []
    for m in range(x.shape[0]):
        first = None
        for l in range(len(per)):
            if set(int(e) for e in ids_gpu[l, m]) != set(int(e) for e in per[l]["idx"][m]):
                first = l
                break
        rows.append({"row": m, "first_selection_difference_layer": first,
                     "h_final_rel_err_normwise": rel_err_normwise(f32(h_gpu[m]), f32(h_ref[m])),
                     "token_gpu": int(tok_gpu[m]), "token_oracle": int(tok_ref[m]),
                     "token_match": bool(int(tok_gpu[m]) == int(tok_ref[m]))})
    rep = {"workload": wl.name, "layers": len(per), "rows": rows,
           "rows_same_routing_all_layers": sum(r["first_selection_difference_layer"] is None
                                               for r in rows),
           "tokens_matching": sum(r["token_match"] for r in rows)}
    for r in rows:
        say("chain-drift %s%s row %d: first selection difference at layer %s, |h_L err| %.3e, "
            "token %d vs oracle %d" % (wl.name, tag, r["row"],
                                       r["first_selection_difference_layer"],
                                       r["h_final_rel_err_normwise"], r["token_gpu"],
                                       r["token_oracle"]))
    out_dir = os.environ.get("MOE_RESULTS_DIR")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "chain_drift_%s%s.json" % (wl.name, tag)), "w") as f:
            json.dump(rep, f, indent=1)
    return rep
