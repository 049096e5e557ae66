"""Benchmark of the small-M MoE decoder step on one MI355X.

Headline (the JSON `value`): the Ling-3.0-flash-shaped MoE layer at M=1
(hidden 2560, 512 routed + 1 shared experts, top-8, intermediate 768), one
persistent launch per layer (router -> softmax top-k -> expert union ->
gate/up+SwiGLU -> down -> combine), reported as effective HBM GB/s of the
unique weight bytes the call must stream (router + every selected expert +
the shared expert, each once), with microseconds per layer beside it.

Cold weights: each timed step runs a different one of 16 distinct layers
(97.7 GB in all, far beyond the 256 MB Infinity Cache) on a different input
row set, so no step finds its weights in any cache; inputs and weights are
resident in HBM before timing starts and nothing else runs in the timed
region.  Secondary figures on the same protocol: the same layer at M=6, the
tensor-parallel shard (I=192, fp32 partial) at M=6, and the 16-layer
pre-norm residual chain at M=6 followed by the 157184-row lm_head argmax.

The CPU oracle is timed on a bounded sample of the headline workload on the
host's cores (cpu_baseline); it is a reported reference, not a target.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/MoE layer and effective HBM GB/s (% of peak) at M=1 and M=6, cold weights"
HBM_PEAK_GBS = 8000.0
N_LAYERS = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="rocprofv3 FETCH/WRITE_SIZE summary for the roofline traffic field")
    ap.add_argument("--profile-run", choices=sorted(PROFILE_WORKLOADS),
                    help="untimed launches of one workload for rocprofv3 (after one known-size "
                         "reference copy); prints no JSON")
    ap.add_argument("--ingest-profiles", metavar="DIR",
                    help="read rocprofv3 CSV output under DIR and write the summaries in profiles/")
    return ap.parse_args()


# Workloads of --profile-run: (workload name, rows, fp32 partial output)
PROFILE_WORKLOADS = {"m1": ("ling_moe_layer_m1", 1, False),
                     "m6": ("ling_moe_layer_m6", 6, False),
                     "tp4": ("ling_tp4_shard_moe_layer_m6", 6, True),
                     "front": ("ling_moe_layer_front_m6", 6, False),
                     "fp8m1": ("ling_fp8_moe_layer_m1", 1, False),
                     "fp8m6": ("ling_fp8_moe_layer_m6", 6, False),
                     "m16": ("ling_moe_layer_m16", 16, False),
                     "lmhead1": ("lmhead_v157184_m1", 1, False),
                     "lmhead": ("lmhead_v157184_m6", 6, False),
                     "lmhead16": ("lmhead_v157184_m16", 16, False),
                     "prefetch": ("ling_moe_layer_m1_prefetch", 1, False)}
# kernel profiled by each workload (the layer kernel unless named here)
PROFILE_KERNELS = {"lmhead1": "moe_lmhead_kernel", "lmhead": "moe_lmhead_mfma_kernel",
                   "lmhead16": "moe_lmhead_mfma_kernel",
                   "prefetch": "moe_prefetch_kernel"}
COPY_BYTES = 256 << 20   # reference copy for the counter scale
PROFILE_CALLS = 64


def main():
    args = parse()
    if args.ingest_profiles:
        ingest_profiles(args.ingest_profiles)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.profile_run:
        profile_run(args.profile_run)
        return

    import numpy as np
    import torch

    import moe_decode_amd as md
    from datagen import device as D
    from datagen import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- weights: 16 distinct Ling layers (+ shards, + lm_head)
    t0 = time.time()
    layers = [D.make_layer(W.C2, l) for l in range(N_LAYERS)]
    print("generated %d layers in %.1f s" % (N_LAYERS, time.time() - t0), file=sys.stderr,
          flush=True)
    lw = [md.layer_weights(L.w_router, L.w_gate_up, L.w_down) for L in layers]

    def x_pool(wl, n_steps, M):
        rows = [W.x_rows(wl, [s * M + m for m in range(M)]) for s in range(n_steps)]
        return torch.stack([D.to_device(r) for r in rows])

    def time_layer(wl, lws, M, steps, warmup, out_f32=False, mode=None):
        """Cold rotating per-layer timing; returns dict of figures."""
        mode = md.MOE_CHAIN_LAYER_ONLY if mode is None else mode
        d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                    md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
        ws = md.new_workspace(d, M, 1)
        n = steps + warmup
        xs = x_pool(wl, n, M)
        out = torch.empty((M, wl.H), dtype=torch.float32 if out_f32 else torch.int16, device=dev)
        idx = torch.empty((n, M, wl.K), dtype=torch.int32, device=dev)
        dt = md.MOE_OUT_F32 if out_f32 else md.MOE_OUT_BF16

        def call(i):
            return md.moe_layer_chain(d, M, [lws[i % len(lws)]], xs[i], out, dt, mode, idx[i],
                                      ws)

        for i in range(warmup):
            md.check(call(i))
        torch.cuda.synchronize()
        # timed region: exactly `steps` back-to-back launches between two events
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        e0.record()
        for i in range(steps):
            md.check(call(warmup + i))
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        md.check(md.moe_last_device_status(ws))
        us_per = e0.elapsed_time(e1) * 1e3 / steps
        # spread: a separate, untimed pass with an event after every launch
        # (each event adds its own small cost, so these sit a little above us_per)
        ne = min(steps, 50)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(ne + 1)]
        evs[0].record()
        for i in range(ne):
            md.check(call(warmup + i))
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(ne)]) * 1e3
        ids = idx.cpu().numpy()[warmup:]
        U = np.array([len(np.unique(ids[i])) for i in range(steps)])
        bytes_per = wl.router_bytes() + (U + wl.S) * wl.expert_bytes() + wl.front_bytes()
        gbs = bytes_per.mean() / (us_per * 1e-6) / 1e9
        return {
            "us_per_layer": float(us_per),
            "per_call_event_us_median": float(np.median(per)),
            "per_call_event_us_p10": float(np.percentile(per, 10)),
            "per_call_event_us_p90": float(np.percentile(per, 90)),
            "wall_ms_per_step": wall * 1e3 / steps,
            "effective_gbs": float(gbs),
            "pct_of_hbm_peak": float(100.0 * gbs / HBM_PEAK_GBS),
            "mean_union_experts": float(U.mean()),
            "unique_bytes_per_call": float(bytes_per.mean()),
            "floor_us_at_peak": float(bytes_per.mean() / HBM_PEAK_GBS / 1e3),
        }

    # ---------------- headline: M=1
    head = time_layer(W.C2, lw, 1, args.steps, args.warmup)
    print("M=1: %.2f us/layer, %.0f GB/s (%.1f %% of 8 TB/s)"
          % (head["us_per_layer"], head["effective_gbs"], head["pct_of_hbm_peak"]),
          file=sys.stderr, flush=True)

    secondary = {}

    def report_prefetch(name, r):
        secondary[name] = r
        print("%s: layer %.1f us cold, %.1f / %.1f / %.1f us after a prefetch at 100 / 75 / 0 %% "
              "routed hits; prefetch %.1f us (%.0f GB/s)"
              % (name, r["cold"]["layer_us_mean"], r["hit100"]["layer_us_mean"],
                 r["hit75"]["layer_us_mean"], r["hit0"]["layer_us_mean"],
                 r["hit100"]["prefetch_us_mean"], r["hit100"]["prefetch_gbs"]),
              file=sys.stderr, flush=True)
        print("%s: back-to-back %.1f us per layer, %.1f us with the next call's experts "
              "prefetched on a second stream during each call"
              % (name, r["pipelined_no_prefetch_us_per_layer"],
                 r["pipelined_prefetch_next_us_per_layer"]), file=sys.stderr, flush=True)

    if not args.no_secondary:
        report_prefetch(W.C2.name + "_prefetch",
                        time_prefetch(md, np, torch, dev, W.C2, lw, x_pool(W.C2, 176, 1)))
        s3 = time_layer(W.C3, lw, 6, args.steps, args.warmup)
        secondary[W.C3.name] = s3
        print("M=6: %.2f us/layer, %.0f GB/s (%.1f %%), U=%.1f"
              % (s3["us_per_layer"], s3["effective_gbs"], s3["pct_of_hbm_peak"],
                 s3["mean_union_experts"]), file=sys.stderr, flush=True)
        s12 = time_layer(W.C12, lw, 16, args.steps, args.warmup)
        secondary[W.C12.name] = s12
        print("M=16: %.2f us/layer, %.0f GB/s (%.1f %%), U=%.1f"
              % (s12["us_per_layer"], s12["effective_gbs"], s12["pct_of_hbm_peak"],
                 s12["mean_union_experts"]), file=sys.stderr, flush=True)
        shards = [D.make_layer(W.C4, l) for l in range(N_LAYERS)]
        lws = [md.layer_weights(L.w_router, L.w_gate_up, L.w_down) for L in shards]
        s4 = time_layer(W.C4, lws, 6, args.steps, args.warmup, out_f32=True)
        secondary[W.C4.name] = s4
        print("TP4 shard M=6: %.2f us/layer, %.0f GB/s (%.1f %%)"
              % (s4["us_per_layer"], s4["effective_gbs"], s4["pct_of_hbm_peak"]),
              file=sys.stderr, flush=True)
        del shards, lws
        # the router front (RMSNorm with gain, selection bias, routed scale) fused in
        fronts = [(D.to_device(W.router_bias(W.C7, l)), D.to_device(W.norm_gain(W.C7, l)))
                  for l in range(N_LAYERS)]
        lwf = [md.layer_weights(L.w_router, L.w_gate_up, L.w_down, b, g)
               for L, (b, g) in zip(layers, fronts)]
        s7 = time_layer(W.C7, lwf, 6, args.steps, args.warmup,
                        mode=md.MOE_CHAIN_PRENORM_LAYER_ONLY)
        secondary[W.C7.name] = s7
        print("front M=6: %.2f us/layer, %.0f GB/s (%.1f %%)"
              % (s7["us_per_layer"], s7["effective_gbs"], s7["pct_of_hbm_peak"]),
              file=sys.stderr, flush=True)
        del fronts, lwf
        # fp8 e4m3 experts with 128 x 128 block scales (bf16 router), 16 distinct layers
        f8 = [D.make_layer_fp8(W.C9, l) for l in range(N_LAYERS)]
        lw8 = [md.layer_weights(L.w_router, L.w_gate_up, L.w_down, None, None, L.s_gate_up,
                                L.s_down) for L in f8]
        for wl8, M8 in ((W.C9, 1), (W.C10, 6), (W.C13, 16)):
            r8 = time_layer(wl8, lw8, M8, args.steps, args.warmup)
            secondary[wl8.name] = r8
            print("fp8 M=%d: %.2f us/layer, %.0f GB/s (%.1f %%)"
                  % (M8, r8["us_per_layer"], r8["effective_gbs"], r8["pct_of_hbm_peak"]),
                  file=sys.stderr, flush=True)
        report_prefetch(W.C9.name + "_prefetch",
                        time_prefetch(md, np, torch, dev, W.C9, lw8, x_pool(W.C9, 176, 1)))
        c8 = time_chain(md, D, W, np, torch, dev, lw8, steps=10, warmup=2, wl=W.C11)
        secondary[W.C11.name] = c8
        print("fp8 chain16+lm_head M=6: %.1f us (floor %.1f us, ratio %.2f)"
              % (c8["us_per_step"], c8["floor_us_at_peak"], c8["ratio_to_floor"]),
              file=sys.stderr, flush=True)
        del f8, lw8
        torch.cuda.empty_cache()
        secondary[W.C5.name] = time_chain(md, D, W, np, torch, dev, lw, steps=10, warmup=2)
        c = secondary[W.C5.name]
        print("chain16+lm_head M=6: %.1f us (floor %.1f us, ratio %.2f)"
              % (c["us_per_step"], c["floor_us_at_peak"], c["ratio_to_floor"]),
              file=sys.stderr, flush=True)
        # one token row through the same 16-layer chain: the per-layer cost when
        # the launch is paid once per step, not once per layer
        from dataclasses import replace as _replace
        wl1 = _replace(W.C5, name="ling_chain16_lmhead_m1", M=1)
        c1 = time_chain(md, D, W, np, torch, dev, lw, steps=10, warmup=2, wl=wl1)
        c1["chain_us_per_layer"] = c1["chain_us"] / wl1.n_layers
        secondary[wl1.name] = c1
        print("chain16+lm_head M=1: %.1f us (chain %.1f us = %.2f us per layer, lm_head %.1f us)"
              % (c1["us_per_step"], c1["chain_us"], c1["chain_us_per_layer"], c1["lmhead_us"]),
              file=sys.stderr, flush=True)
        lmr = time_lmhead(md, D, W, np, torch, dev)
        secondary["lmhead_v%d" % W.C5.V] = lmr
        print("lm_head alone: " + ", ".join("M=%s %.1f us (%.0f GB/s)" % (k[2:], v["us"], v["gbs"])
                                              for k, v in lmr.items()),
              file=sys.stderr, flush=True)

    traffic = None
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            tj = json.load(f)
        if tj.get("kernel_source_sha") == kernel_source_sha():
            traffic = tj.get("workloads", {}).get(W.C2.name, {}).get("bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(head["effective_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; weights ~N(0,0.02^2), inputs ~N(0,1))",
        "config": {"workload": W.C2.name, "hidden": 2560, "routed_experts": 512,
                   "shared_experts": 1, "top_k": 8, "inter": 768, "rows": 1,
                   "cold": "rotating over 16 distinct layers, 97.7 GB"},
        "us_per_layer": round(head["us_per_layer"], 3),
        "pct_of_hbm_peak": round(head["pct_of_hbm_peak"], 2),
        "roofline": {"bound": "hbm", "achieved": round(head["effective_gbs"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["effective_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "headline_detail": head,
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def time_chain(md, D, W, np, torch, dev, lw, steps, warmup, wl=None):
    """16-layer pre-norm residual chain (one launch) + lm_head argmax (one launch)."""
    wl = W.C5 if wl is None else wl
    M = wl.M
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
    ws = md.new_workspace(d, M, wl.n_layers)
    lm = D.make_lmhead(wl)
    n = steps + warmup
    xs = torch.stack([D.to_device(W.x_rows(wl, [s * M + m for m in range(M)]))
                      for s in range(n)])
    h = torch.empty((M, wl.H), dtype=torch.int16, device=dev)
    idx = torch.empty((n, wl.n_layers, M, wl.K), dtype=torch.int32, device=dev)
    tok = torch.empty((M,), dtype=torch.int32, device=dev)

    def call(i):
        md.check(md.moe_layer_chain(d, M, lw[:wl.n_layers], xs[i], h, md.MOE_OUT_BF16,
                                    md.MOE_CHAIN_PRENORM_RESIDUAL, idx[i], ws))
        md.check(md.lmhead_argmax(M, wl.H, wl.V, h, lm, tok, None, ws))

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    e[0].record()
    for i in range(steps):
        md.check(md.moe_layer_chain(d, M, lw[:wl.n_layers], xs[warmup + i], h, md.MOE_OUT_BF16,
                                    md.MOE_CHAIN_PRENORM_RESIDUAL, idx[warmup + i], ws))
        e[2 * i + 1].record()
        md.check(md.lmhead_argmax(M, wl.H, wl.V, h, lm, tok, None, ws))
        e[2 * i + 2].record()
    torch.cuda.synchronize()
    md.check(md.moe_last_device_status(ws))
    chain_us = np.array([e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(steps)]) * 1e3
    lm_us = np.array([e[2 * i + 1].elapsed_time(e[2 * i + 2]) for i in range(steps)]) * 1e3
    ids = idx.cpu().numpy()[warmup:]
    chain_bytes = []
    for i in range(steps):
        b = 0
        for l in range(wl.n_layers):
            U = len(np.unique(ids[i, l]))
            b += wl.router_bytes() + (U + wl.S) * wl.expert_bytes()
        chain_bytes.append(b)
    chain_bytes = np.array(chain_bytes, dtype=np.float64)
    lm_bytes = wl.V * wl.H * 2
    total_bytes = chain_bytes.mean() + lm_bytes
    floor_us = total_bytes / HBM_PEAK_GBS / 1e3
    tot_us = chain_us.mean() + lm_us.mean()
    del lm
    return {
        "us_per_step": float(tot_us),
        "chain_us": float(chain_us.mean()),
        "lmhead_us": float(lm_us.mean()),
        "chain_effective_gbs": float(chain_bytes.mean() / (chain_us.mean() * 1e-6) / 1e9),
        "lmhead_effective_gbs": float(lm_bytes / (lm_us.mean() * 1e-6) / 1e9),
        "unique_bytes_per_step": float(total_bytes),
        "floor_us_at_peak": float(floor_us),
        "ratio_to_floor": float(tot_us / floor_us),
    }


def time_prefetch(md, np, torch, dev, wl, lws, xs, calls=160, warmup=16):
    """Layer time after a speculative prefetch of its experts, against cold.

    Calls rotate over the distinct layers in `lws`, so each call's weights were
    last read many gigabytes ago.  A first untimed pass records every call's
    routing; then, per call, the guess lists the chosen experts with a share
    replaced by experts the call does not pick (routed hit rate 100, 75 or 0 %),
    plus the shared expert.  moe_expert_prefetch runs just before the layer on
    the same stream; events around each kernel give the layer's and the
    prefetch's time.  "cold" is the same loop with no prefetch."""
    M = xs.shape[1]
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
    ws = md.new_workspace(d, M, 1)
    n = calls + warmup
    nl = len(lws)
    out = torch.empty((M, wl.H), dtype=torch.int16, device=dev)
    idx = torch.empty((n, M, wl.K), dtype=torch.int32, device=dev)

    def layer(i):
        md.check(md.moe_layer_chain(d, M, [lws[i % nl]], xs[i], out, md.MOE_OUT_BF16,
                                    md.MOE_CHAIN_LAYER_ONLY, idx[i], ws))

    for i in range(n):
        layer(i)
    torch.cuda.synchronize()
    md.check(md.moe_last_device_status(ws))
    chosen = [np.unique(r) for r in idx.cpu().numpy()]
    rng = np.random.default_rng(20240607)
    res = {}
    for label, hit in (("cold", None), ("hit100", 1.0), ("hit75", 0.75), ("hit0", 0.0)):
        ids = None
        if hit is not None:
            lists = []
            for ch in chosen:
                keep = int(round(hit * len(ch)))
                pool = np.setdiff1d(np.arange(wl.E), ch)
                wrong = rng.choice(pool, len(ch) - keep, replace=False)
                lists.append(np.concatenate([ch[:keep], wrong, np.arange(wl.E, wl.E + wl.S)]))
            width = max(len(l) for l in lists)
            pad = np.full((n, width), -1, dtype=np.int32)   # -1 is skipped by the prefetch
            for i, l in enumerate(lists):
                pad[i, :len(l)] = l
            ids = torch.from_numpy(pad).to(dev)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            evs[i][0].record()
            if ids is not None:
                md.check(md.moe_expert_prefetch(d, lws[i % nl], ids[i], ids.shape[1]))
            evs[i][1].record()
            layer(i)
            evs[i][2].record()
        torch.cuda.synchronize()
        md.check(md.moe_last_device_status(ws))
        lay = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(warmup, n)]) * 1e3
        pf = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(warmup, n)]) * 1e3
        r = {"layer_us_mean": float(lay.mean()), "layer_us_median": float(np.median(lay))}
        if ids is not None:
            nb = float(np.mean([len(l) for l in lists])) * wl.expert_bytes()
            r.update({"prefetch_us_mean": float(pf.mean()), "prefetch_bytes": nb,
                      "prefetch_gbs": float(nb / (pf.mean() * 1e-6) / 1e9)})
        res[label] = r
    res["saving_us_at_hit100"] = res["cold"]["layer_us_mean"] - res["hit100"]["layer_us_mean"]

    # Overlapped: the next call's experts (a correct guess, plus the shared expert)
    # prefetched on a second stream while the current call runs; the next call
    # waits for that prefetch.  Against the same loop with no prefetch.
    nxt = np.full((n, max(len(c) for c in chosen) + wl.S), -1, dtype=np.int32)
    for i, ch in enumerate(chosen):
        row = np.concatenate([ch, np.arange(wl.E, wl.E + wl.S)])
        nxt[i, :len(row)] = row
    nxt = torch.from_numpy(nxt).to(dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for label, with_pf in (("pipelined_no_prefetch", False), ("pipelined_prefetch_next", True)):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(n):
            if i == warmup:
                e0.record(main)
            go = torch.cuda.Event()
            go.record(main)
            layer(i)
            if with_pf and i + 1 < n:
                side.wait_event(go)
                md.check(md.moe_expert_prefetch(d, lws[(i + 1) % nl], nxt[i + 1], nxt.shape[1],
                                                stream=side.cuda_stream))
                done = torch.cuda.Event()
                done.record(side)
                main.wait_event(done)
        e1.record(main)
        torch.cuda.synchronize()
        md.check(md.moe_last_device_status(ws))
        res[label + "_us_per_layer"] = e0.elapsed_time(e1) * 1e3 / calls
    return res


def time_lmhead(md, D, W, np, torch, dev, rows=(1, 6, 16), calls=30, warmup=3):
    """The lm_head argmax alone (V = 157184, H = 2560), back-to-back calls at each
    row count: the dot-product kernel for 1 or 2 rows, the matrix-core kernel above.
    The 805 MB matrix exceeds every cache, so every call streams it from HBM."""
    wl = W.C5
    lm = D.make_lmhead(wl)
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S)
    ws = md.new_workspace(d, max(rows), 1)
    out = {}
    for M in rows:
        hs = [D.to_device(W.x_rows(wl, [s * M + m for m in range(M)]))
              for s in range(calls + warmup)]
        tok = torch.empty((M,), dtype=torch.int32, device=dev)
        for i in range(warmup):
            md.check(md.lmhead_argmax(M, wl.H, wl.V, hs[i], lm, tok, None, ws))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(warmup, warmup + calls):
            md.check(md.lmhead_argmax(M, wl.H, wl.V, hs[i], lm, tok, None, ws))
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        out["M=%d" % M] = {"us": float(us), "gbs": float(wl.V * wl.H * 2 / us / 1e3),
                           "pct_of_hbm_peak": float(100.0 * wl.V * wl.H * 2 / us / 1e3
                                                    / HBM_PEAK_GBS)}
    md.check(md.moe_last_device_status(ws))
    del lm
    return out


def profile_run(key):
    """One reference copy of COPY_BYTES, then PROFILE_CALLS cold layer launches of
    one workload (rotating over 16 distinct layers), for rocprofv3."""
    import torch

    import benchsupport as bs
    import moe_decode_amd as md
    from datagen import device as D
    from datagen import workloads as W

    name, M, f32 = PROFILE_WORKLOADS[key]
    if key == "prefetch":
        return profile_run_prefetch(name)
    if key in PROFILE_KERNELS:
        return profile_run_lmhead(name, M)
    wl = {w.name: w for w in (W.C2, W.C3, W.C4, W.C7, W.C9, W.C10, W.C12)}[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    make = D.make_layer_fp8 if wl.fp8 else D.make_layer
    layers = [make(wl, l) for l in range(N_LAYERS)]
    keep = []
    lws = []
    for l, L in enumerate(layers):
        b, g = W.router_bias(wl, l), W.norm_gain(wl, l)
        b = None if b is None else D.to_device(b)
        g = None if g is None else D.to_device(g)
        keep.append((b, g))
        lws.append(md.layer_weights(L.w_router, L.w_gate_up, L.w_down, b, g, L.s_gate_up,
                                    L.s_down))
    mode = md.MOE_CHAIN_PRENORM_LAYER_ONLY if wl.prenorm else md.MOE_CHAIN_LAYER_ONLY
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
    ws = md.new_workspace(d, M, 1)
    xs = torch.stack([D.to_device(W.x_rows(wl, [s * M + m for m in range(M)]))
                      for s in range(PROFILE_CALLS)])
    out = torch.empty((M, wl.H), dtype=torch.float32 if f32 else torch.int16, device=dev)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    bs.copy(src, dst, 2048, st)
    idx = torch.empty((PROFILE_CALLS, M, wl.K), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for i in range(PROFILE_CALLS):
        md.check(md.moe_layer_chain(d, M, [lws[i % N_LAYERS]], xs[i], out,
                                    md.MOE_OUT_F32 if f32 else md.MOE_OUT_BF16, mode, idx[i], ws))
    torch.cuda.synchronize()
    md.check(md.moe_last_device_status(ws))
    ids = idx.cpu().numpy()
    U = [len(set(ids[i].ravel().tolist())) for i in range(PROFILE_CALLS)]
    alg = wl.router_bytes() + (sum(U) / len(U) + wl.S) * wl.expert_bytes() + wl.front_bytes()
    print("profile run %s: 1 copy of %d bytes, %d layer launches" % (key, COPY_BYTES,
                                                                      PROFILE_CALLS))
    print("algorithmic bytes per launch: %.0f (mean union %.2f experts)" % (alg, sum(U) / len(U)),
          flush=True)


def profile_run_prefetch(name):
    """One reference copy, PROFILE_CALLS cold Ling layer launches at M=1 to learn
    each call's routing, then PROFILE_CALLS pairs of (moe_expert_prefetch of that
    call's 8 routed experts and the shared expert, the layer launch), rotating over
    16 distinct layers."""
    import numpy as np
    import torch

    import benchsupport as bs
    import moe_decode_amd as md
    from datagen import device as D
    from datagen import workloads as W

    wl = W.C2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = [D.make_layer(wl, l) for l in range(N_LAYERS)]
    lws = [md.layer_weights(L.w_router, L.w_gate_up, L.w_down) for L in layers]
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale)
    ws = md.new_workspace(d, 1, 1)
    xs = torch.stack([D.to_device(W.x_rows(wl, [s])) for s in range(PROFILE_CALLS)])
    out = torch.empty((1, wl.H), dtype=torch.int16, device=dev)
    idx = torch.empty((PROFILE_CALLS, 1, wl.K), dtype=torch.int32, device=dev)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    bs.copy(src, dst, 2048, torch.cuda.current_stream().cuda_stream)

    def layer(i):
        md.check(md.moe_layer_chain(d, 1, [lws[i % N_LAYERS]], xs[i], out, md.MOE_OUT_BF16,
                                    md.MOE_CHAIN_LAYER_ONLY, idx[i], ws))

    for i in range(PROFILE_CALLS):
        layer(i)
    torch.cuda.synchronize()
    ids = torch.cat([idx.view(PROFILE_CALLS, wl.K),
                     torch.full((PROFILE_CALLS, 1), wl.E, dtype=torch.int32, device=dev)], 1)
    ids = ids.contiguous()
    n = wl.K + wl.S
    for i in range(PROFILE_CALLS):
        md.check(md.moe_expert_prefetch(d, lws[i % N_LAYERS], ids[i], n))
        layer(i)
    torch.cuda.synchronize()
    md.check(md.moe_last_device_status(ws))
    print("profile run %s: 1 copy of %d bytes, %d prefetch + layer pairs" % (name, COPY_BYTES,
                                                                            PROFILE_CALLS))
    print("algorithmic bytes per launch: %.0f (%d experts, each once)"
          % (n * wl.expert_bytes(), n), flush=True)


def profile_run_lmhead(name, M):
    """One reference copy, then PROFILE_CALLS lm_head argmax launches (V = 157184, H = 2560;
    the 805 MB weight is larger than every cache, so each launch reads it from HBM)."""
    import torch

    import benchsupport as bs
    import moe_decode_amd as md
    from datagen import device as D
    from datagen import workloads as W

    wl = W.C5
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lm = D.make_lmhead(wl)
    ws = md.new_workspace(md.dims(wl.H, wl.E, wl.K, wl.I, wl.S), M, 1)
    hs = torch.stack([D.to_device(W.x_rows(wl, [s * M + m for m in range(M)]))
                      for s in range(PROFILE_CALLS)])
    tok = torch.empty((M,), dtype=torch.int32, device=dev)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    bs.copy(src, dst, 2048, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for i in range(PROFILE_CALLS):
        md.check(md.lmhead_argmax(M, wl.H, wl.V, hs[i], lm, tok, None, ws))
    torch.cuda.synchronize()
    md.check(md.moe_last_device_status(ws))
    print("profile run %s: 1 copy of %d bytes, %d lm_head launches" % (name, COPY_BYTES,
                                                                        PROFILE_CALLS))
    print("algorithmic bytes per launch: %.0f (the V x H bf16 weight, once)"
          % (wl.V * wl.H * 2), flush=True)


def _csv_rows(root, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True))
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return files, rows


def ingest_profiles(root):
    """rocprofv3 output of the profile runs -> profiles/*.txt and profiles/traffic.json.

    Expected layout under root: kt_<key>/ (--kernel-trace --stats), pmc_fetch_<key>/
    (--pmc FETCH_SIZE) and pmc_write_<key>/ (--pmc WRITE_SIZE) for each key of
    PROFILE_WORKLOADS that was run.  FETCH_SIZE and WRITE_SIZE are KiB per dispatch;
    each is scaled to bytes by what it reads for the reference copy of COPY_BYTES."""
    import numpy as np
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    traffic = {"kernel_source_sha": kernel_source_sha(), "copy_bytes": COPY_BYTES,
               "workloads": {}}
    for key, (name, M, _) in sorted(PROFILE_WORKLOADS.items()):
        kname = PROFILE_KERNELS.get(key, "moe_layer_kernel")
        cmd_kt = ("rocprofv3 --kernel-trace --stats --output-format csv -d %s/kt_%s -o kt "
                  "-- python3 bench.py --profile-run %s" % (root, key, key))
        alg = None
        logf = os.path.join(root, "kt_%s.log" % key)
        if os.path.exists(logf):
            for ln in open(logf):
                if ln.startswith("algorithmic bytes per launch:"):
                    alg = float(ln.split(":")[1].split()[0])
        kt_files, kt = _csv_rows(os.path.join(root, "kt_" + key), "kernel_trace.csv")
        st_files, stats = _csv_rows(os.path.join(root, "kt_" + key), "kernel_stats.csv")
        if not kt_files:
            continue
        lay = [r for r in kt if kname in r.get("Kernel_Name", "")]
        durs = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in lay],
                        dtype=np.float64) * 1e-3
        lines = ["# %s: %s, %d cold launches" % (name, kname, len(durs)),
                 "command: %s" % cmd_kt,
                 "per-launch kernel duration (us, kernel_trace.csv): mean %.2f  median %.2f  "
                 "min %.2f  max %.2f" % (durs.mean(), np.median(durs), durs.min(), durs.max()),
                 "", "kernel_stats.csv:"]
        for r in stats:
            lines.append("  %-60s calls %5s  avg %10.0f ns  total %12s ns  %6s %%"
                         % (r["Name"][:60], r["Calls"], float(r["AverageNs"]),
                            r["TotalDurationNs"], r["Percentage"]))
        w = {"mean_kernel_us": float(durs.mean()), "median_kernel_us": float(np.median(durs))}
        for ctr, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            files, rows = _csv_rows(os.path.join(root, "pmc_%s_%s" % (tag, key)),
                                    "counter_collection.csv")
            if not files:
                continue
            ref = [float(r["Counter_Value"]) for r in rows
                   if "bs_copy" in r["Kernel_Name"] and r["Counter_Name"] == ctr]
            vals = [float(r["Counter_Value"]) for r in rows
                    if kname in r["Kernel_Name"] and r["Counter_Name"] == ctr]
            if not ref or not vals:
                continue
            scale = COPY_BYTES / ref[0]          # bytes per counter unit
            per = float(np.mean(vals)) * scale
            w[tag + "_bytes_per_launch"] = per
            w[tag + "_counter_per_launch"] = float(np.mean(vals))
            w[tag + "_scale_bytes_per_unit"] = scale
            lines.append("")
            lines.append("%s: command: rocprofv3 --pmc %s --output-format csv -d %s/pmc_%s_%s "
                         "-o pmc -- python3 bench.py --profile-run %s" % (ctr, ctr, root, tag, key,
                                                                          key))
            lines.append("  reference copy of %d bytes (read once, written once): %.1f units "
                         "-> %.2f bytes per unit" % (COPY_BYTES, ref[0], scale))
            lines.append("  %s: %.1f units per launch (mean of %d) = %.3f MB per launch"
                         % (kname, np.mean(vals), len(vals), per / 1e6))
        if "fetch_bytes_per_launch" in w:
            w["bytes_per_launch"] = w["fetch_bytes_per_launch"] + w.get("write_bytes_per_launch", 0.0)
        if alg:
            w["algorithmic_bytes_per_launch"] = alg
            lines.append("")
            what = {"prefetch": "the 9 listed experts, each once"}.get(
                key, "the V x H weight, once" if key in PROFILE_KERNELS
                else "router + union + shared expert, each once")
            lines.append("algorithmic bytes per launch (%s): %.3f MB" % (what, alg / 1e6))
            if "bytes_per_launch" in w:
                lines.append("measured HBM traffic / algorithmic bytes: %.4f"
                             % (w["bytes_per_launch"] / alg))
            lines.append("achieved at the mean kernel duration: %.0f GB/s (%.1f %% of 8 TB/s)"
                         % (alg / (durs.mean() * 1e-6) / 1e9,
                            100 * alg / (durs.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS))
        traffic["workloads"][name] = w
        with open(os.path.join(out_dir, "%s_%s.txt" % (kname, name)), "w") as f:
            f.write("\n".join(lines) + "\n")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps(traffic, indent=1))


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("moe_device.hpp", "moe_layer.hpp", "moe_lmhead.hpp", "moe_prefetch.hpp",
              "moe_capi.hip"):
        with open(os.path.join(ROOT, "moe_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(seconds):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    headline workload (Ling layer, M=1); weight generation is not timed."""
    import numpy as np

    import oracle
    from oracle import runner
    from datagen import workloads as W

    wl = W.C2
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    # a pool of 16 problems (one per layer, each with its own input row and its
    # selected experts' weights generated once), cycled until the time budget
    # is spent: ~1.7 GB of weights, well beyond the host caches
    pool = []
    for l in range(N_LAYERS):
        x = W.x_rows(wl, [1000 + l])
        wr = W.router(wl, l)
        idx, _, _ = oracle.router_topk(x, wr, wl.K)
        used = sorted(set(int(e) for e in idx.ravel())) + [wl.E]
        gu = {e: W.expert_gate_up(wl, l, e) for e in used}
        dn = {e: W.expert_down(wl, l, e) for e in used}
        pool.append((x, wr, gu, dn, wl.router_bytes() + len(used) * wl.expert_bytes()))
    times, nbytes = [], []
    t_total = 0.0
    s = 0
    while t_total < seconds:
        x, wr, gu, dn, nb = pool[s % len(pool)]
        t0 = time.perf_counter()
        idx, gate, _ = oracle.router_topk(x, wr, wl.K)
        acc = oracle.experts_combine(x, idx, gate, gu, dn, wl.E, wl.S)
        oracle.cast_bf16(acc)
        dt = time.perf_counter() - t0
        times.append(dt)
        nbytes.append(nb)
        t_total += dt
        s += 1
    times = np.array(times)
    gbs = float(np.sum(nbytes) / np.sum(times) / 1e9)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_layer": round(float(times.mean() * 1e6), 1),
            "sample": "%d Ling MoE layer calls at M=1 (router, top-k, 8 routed + shared "
                      "experts, combine) cycling over 16 pre-generated problems; %.1f s of "
                      "oracle time" % (len(times), times.sum())}


if __name__ == "__main__":
    main()
