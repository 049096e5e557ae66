"""Write tiefree_rows.json: per workload, the generator attempt index of each
input row such that the oracle's routing has no near-tie (K-th minus (K+1)-th
selection score >= DELTA at every layer; the score is the logit plus the
selection bias, on the normed input where the workload has the router front)
and, for the lm_head workload, no near-tie in the argmax (top two float64
logits DELTA apart).

Calls only the oracle and the seeded generator.  Usage:
    python tests/golden/make_tiefree.py [workload names to recompute]
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from datagen import workloads as W  # noqa: E402
from oracle import rmsnorm, router_topk, runner  # noqa: E402

DELTA = 1e-3
ROWS = {W.C1.name: 16, W.C2.name: 8, W.C3.name: 6, W.C4.name: 6, W.C5.name: 6,
        W.C6.name: 8, W.C7.name: 8, W.C8.name: 8, W.C9.name: 8, W.C10.name: 8, W.C11.name: 6,
        W.C12.name: 16, W.C13.name: 16}


def row_ok_single(wl, xrow, wr):
    u = xrow[None, :]
    if wl.prenorm:
        u = rmsnorm(u, gain=W.norm_gain(wl, 0))
    bias = W.router_bias(wl, 0)
    _, _, lg = router_topk(u, wr, wl.K, bias)
    return runner.router_margin(lg, wl.K, bias)[0] >= DELTA


def row_ok_chain(wl, xrow, routers, lm):
    h, per = runner.chain(wl, xrow[None, :], routers=routers)
    if any(runner.router_margin(r["logits"], wl.K)[0] < DELTA for r in per):
        return False
    return runner.lmhead_margin(h, lm)[0] >= DELTA


def main():
    path = os.path.join(HERE, "tiefree_rows.json")
    out = {"delta": DELTA, "workloads": {}}
    only = set(sys.argv[1:])          # optional: recompute just these workloads
    if only and os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    for wl in W.ALL + W.FRONT + W.FP8 + W.WIDE:
        if only and wl.name not in only:
            continue
        n = ROWS[wl.name]
        attempts = []
        if wl.n_layers == 1:
            wr = W.router(wl, 0)
            for m in range(n):
                a = 0
                while not row_ok_single(wl, W.x_row(wl, m, a), wr):
                    a += 1
                attempts.append(a)
        else:
            routers = [W.router(wl, l) for l in range(wl.n_layers)]
            lm = W.lmhead(wl)
            for m in range(n):
                a = 0
                while not row_ok_chain(wl, W.x_row(wl, m, a), routers, lm):
                    a += 1
                attempts.append(a)
                print(wl.name, "row", m, "attempt", a, flush=True)
        out["workloads"][wl.name] = attempts
        print(wl.name, attempts, flush=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
