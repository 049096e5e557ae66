"""Benchmark of the small-M MoE decoder step on one MI355X.

Headline (the JSON `value`): the Ling-3.0-flash-shaped MoE layer at M=1
(hidden 2560, 512 routed + 1 shared experts, top-8, intermediate 768), one
persistent launch per layer (router -> softmax top-k -> expert union ->
gate/up+SwiGLU -> down -> combine), reported as effective HBM GB/s of the
unique weight bytes the call must stream (router + every selected expert +
the shared expert, each once), with microseconds per layer beside it.  Every
time in the record comes from HIP events on the launch stream.

Cold weights: each timed step runs a different one of 16 distinct layers
(97.7 GB in all, far beyond the 256 MB Infinity Cache) on a different input
row set, so no step finds its weights in any cache; inputs and weights are
resident in HBM before timing starts and nothing else runs in the timed
region.  Beside it: the same call hot (one layer, one input, repeated: its
109 MB stay in the Infinity Cache), and the achievable streaming-read rate of
the chip from a plain read kernel.  Secondary figures on the cold protocol:
the layer at M=6 (independent rows, and perturbed copies of one row), M=16,
the tensor-parallel shard (I=192, fp32 partial) at M=6, the router front,
fp8 experts, the 16-layer pre-norm residual chains followed by the 157184-row
lm_head argmax, the lm_head alone, and speculative expert prefetch on a
time-correlated decode walk guessed from the previous step's routing.

The CPU oracle is timed on bounded samples of the same workloads on the host's
cores (cpu_baseline); it is a reported reference, not a target.
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
PERTURB_RHO = 0.9       # correlation of each perturbed row with the batch's base row


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

    def time_layer(wl, lws, M, steps, warmup, out_f32=False, mode=None, xs=None, hot=False):
        """Per-layer timing, cold (call i runs layer i mod 16 on input set i) or hot
        (every call runs layer 0 on input set 0, so its weights stay in the caches when
        they fit); returns dict of figures, all from events on the launch stream."""
        mode = md.MOE_CHAIN_LAYER_ONLY if mode is None else mode
        d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                    md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
        ws = md.new_workspace(d, M, 1)
        n = steps + warmup
        xs = x_pool(wl, n, M) if xs is None else xs
        assert xs.shape[0] >= n and xs.shape[1] == M
        out = torch.empty((M, wl.H), dtype=torch.float32 if out_f32 else torch.int16, device=dev)
        idx = torch.empty((n, M, wl.K), dtype=torch.int32, device=dev)
        dt = md.MOE_OUT_F32 if out_f32 else md.MOE_OUT_BF16

        def call(i):
            j = 0 if hot else i
            return md.moe_layer_chain(d, M, [lws[j % len(lws)]], xs[j], out, dt, mode, idx[i],
                                      ws)

        for i in range(warmup):
            md.check(call(i))
        torch.cuda.synchronize()
        # timed region: exactly `steps` back-to-back launches between two events
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            md.check(call(warmup + i))
        e1.record()
        torch.cuda.synchronize()
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
            "effective_gbs": float(gbs),
            "pct_of_hbm_peak": float(100.0 * gbs / HBM_PEAK_GBS),
            "mean_union_experts": float(U.mean()),
            "unique_bytes_per_call": float(bytes_per.mean()),
            "floor_us_at_peak": float(bytes_per.mean() / HBM_PEAK_GBS / 1e3),
        }

    # ---------------- headline: M=1, cold; the same call hot beside it
    head = time_layer(W.C2, lw, 1, args.steps, args.warmup)
    hot = time_layer(W.C2, lw, 1, args.steps, args.warmup, hot=True)
    head["hot_us_per_layer"] = hot["us_per_layer"]
    print("M=1: %.2f us/layer cold (%.0f GB/s, %.1f %% of 8 TB/s), %.2f us hot"
          % (head["us_per_layer"], head["effective_gbs"], head["pct_of_hbm_peak"],
             hot["us_per_layer"]), file=sys.stderr, flush=True)
    ceiling = stream_ceiling(torch, dev)
    print("streaming-read ceiling: %.0f GB/s (%s)" % (ceiling["gbs"], ceiling["grid"]),
          file=sys.stderr, flush=True)

    secondary = {}

    def report_prefetch(name, r):
        secondary[name] = r
        print("%s: rho %.2f, previous-step guess hits %.0f %%; layer %.1f us cold, %.1f us after "
              "prefetch (+%.1f us prefetch = %.1f); exact guess %.1f + %.1f = %.1f us"
              % (name, r["rho"], 100 * r["hit_rate_previous_step"], r["cold_layer_us"],
                 r["previous"]["layer_us"], r["previous"]["prefetch_us"],
                 r["previous"]["total_us"], r["exact"]["layer_us"], r["exact"]["prefetch_us"],
                 r["exact"]["total_us"]), file=sys.stderr, flush=True)

    chain_probe = None
    if not args.no_secondary:
        report_prefetch(W.C2.name + "_prefetch_walk",
                        time_prefetch(md, np, torch, dev, W.C2, lw))
        s3 = time_layer(W.C3, lw, 6, args.steps, args.warmup)
        secondary[W.C3.name] = s3
        print("M=6: %.2f us/layer, %.0f GB/s (%.1f %%), U=%.1f"
              % (s3["us_per_layer"], s3["effective_gbs"], s3["pct_of_hbm_peak"],
                 s3["mean_union_experts"]), file=sys.stderr, flush=True)
        # six rows that are perturbed copies of one row: correlated routing, smaller union
        n3 = args.steps + args.warmup
        xp = torch.stack([D.to_device(W.x_perturbed(W.C3, 6, PERTURB_RHO, s)) for s in range(n3)])
        s3p = time_layer(W.C3, lw, 6, args.steps, args.warmup, xs=xp)
        s3p["rho"] = PERTURB_RHO
        secondary[W.C3.name + "_perturbed"] = s3p
        del xp
        print("M=6 perturbed rows (rho %.2f): %.2f us/layer, %.0f GB/s (%.1f %%), U=%.1f"
              % (PERTURB_RHO, s3p["us_per_layer"], s3p["effective_gbs"], s3p["pct_of_hbm_peak"],
                 s3p["mean_union_experts"]), file=sys.stderr, flush=True)
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
        c8, _ = time_chain(md, D, W, np, torch, dev, lw8, steps=10, warmup=2, wl=W.C11)
        secondary[W.C11.name] = c8
        print("fp8 chain16+lm_head M=6: %.1f us (floor %.1f us, ratio %.2f)"
              % (c8["us_per_step"], c8["floor_us_at_peak"], c8["ratio_to_floor"]),
              file=sys.stderr, flush=True)
        del f8, lw8
        torch.cuda.empty_cache()
        secondary[W.C5.name], chain_probe = time_chain(md, D, W, np, torch, dev, lw, steps=10,
                                                       warmup=2)
        c = secondary[W.C5.name]
        print("chain16+lm_head M=6: %.1f us (floor %.1f us, ratio %.2f)"
              % (c["us_per_step"], c["floor_us_at_peak"], c["ratio_to_floor"]),
              file=sys.stderr, flush=True)
        # one token row through the same 16-layer chain: the per-layer cost when
        # the launch is paid once per step, not once per layer
        from dataclasses import replace as _replace
        wl1 = _replace(W.C5, name="ling_chain16_lmhead_m1", M=1)
        c1, _ = time_chain(md, D, W, np, torch, dev, lw, steps=10, warmup=2, wl=wl1)
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
        cpu = cpu_baseline(args.cpu_seconds, chain_probe)

    rec = {
        "metric": METRIC,
        "value": round(head["effective_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_layer"] * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; weights ~N(0,0.02^2), inputs ~N(0,1))",
        "config": {"workload": W.C2.name, "hidden": 2560, "routed_experts": 512,
                   "shared_experts": 1, "top_k": 8, "inter": 768, "rows": 1,
                   "cold": "rotating over 16 distinct layers, 97.7 GB"},
        "us_per_layer": round(head["us_per_layer"], 3),
        "hot_us_per_layer": round(head["hot_us_per_layer"], 3),
        "pct_of_hbm_peak": round(head["pct_of_hbm_peak"], 2),
        "roofline": {"bound": "hbm", "achieved": round(head["effective_gbs"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["effective_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "achievable": round(ceiling["gbs"], 1),
                     "frac_of_achievable": round(head["effective_gbs"] / ceiling["gbs"], 4),
                     "achievable_kernel": ceiling["kernel"]},
        "headline_detail": head,
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def stream_ceiling(torch, dev, gib=4, reps=4, grids=(256, 1024, 2048)):
    """Achievable streaming-read rate of the chip: bs_stream_read (whole 16 KiB chunks
    per wave, 1 KiB non-temporal loads, 16 in flight) over a buffer far larger than
    every cache, best of a few grid sizes, timed with events on the launch stream."""
    import benchsupport as bs
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    best = (0.0, None)
    for g in grids:
        bs.stream_read(buf, sink, g, st.cuda_stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            bs.stream_read(buf, sink, g, st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        gbs = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(best, (gbs, g), key=lambda t: t[0])
    del buf
    torch.cuda.empty_cache()
    return {"gbs": best[0], "grid": "%d x 512 threads" % best[1],
            "kernel": "bs_stream_read over %d GiB: 16 KiB per wave, 1 KiB non-temporal loads, "
                      "16 in flight" % gib}


def time_chain(md, D, W, np, torch, dev, lw, steps, warmup, wl=None):
    """16-layer pre-norm residual chain (one launch) + lm_head argmax (one launch).

    Returns (figures, probe): probe holds the tokens and per-layer routing of one more
    call on the first input set (rows 0..M-1), for comparison with the CPU oracle."""
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
    call(0)
    torch.cuda.synchronize()
    probe = {"rows": [m for m in range(M)], "tokens": tok.cpu().numpy().copy(),
             "idx": idx[0].cpu().numpy().copy()}
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
    }, probe


def time_prefetch(md, np, torch, dev, wl, lws, rho=0.95, n_steps=12):
    """Speculative expert prefetch on a decode-like, time-correlated input.

    One row per step from W.x_walk (correlation rho between consecutive steps);
    each step runs the distinct layers of `lws` in turn on that row (layer-only
    calls), so every call's weights were last read one step, i.e. more than
    1.5 GB of other layers, ago.  Step 0 is untimed.  Three passes over the same
    calls, all on one stream (no kernel may run beside a layer call):
      cold      the layer calls alone;
      previous  before each call, moe_expert_prefetch of the experts the same
                layer chose at the previous step, plus the shared expert;
      exact     the same with the call's own routing (the best any guess can do).
    Reports per-call layer time, prefetch time and their sum against cold, the
    realized hit rate of the previous-step guess, and whether every pass routed
    identically (a prefetch never changes results)."""
    from datagen import device as D
    from datagen import workloads as W
    nl = len(lws)
    d = md.dims(wl.H, wl.E, wl.K, wl.I, wl.S, wl.routed_scale,
                md.MOE_EXPERT_FP8_B128 if wl.fp8 else md.MOE_EXPERT_BF16)
    ws = md.new_workspace(d, 1, 1)
    xs = torch.stack([D.to_device(r[None]) for r in W.x_walk(wl, n_steps, rho)])
    out = torch.empty((1, wl.H), dtype=torch.int16, device=dev)
    n = n_steps * nl
    shared = np.arange(wl.E, wl.E + wl.S)

    def run(guess):
        idx = torch.empty((n, 1, wl.K), dtype=torch.int32, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            ev[i][0].record()
            if guess is not None and i >= nl:
                md.check(md.moe_expert_prefetch(d, lws[i % nl], guess[i], guess.shape[1]))
            ev[i][1].record()
            md.check(md.moe_layer_chain(d, 1, [lws[i % nl]], xs[i // nl], out, md.MOE_OUT_BF16,
                                        md.MOE_CHAIN_LAYER_ONLY, idx[i], ws))
            ev[i][2].record()
        torch.cuda.synchronize()
        md.check(md.moe_last_device_status(ws))
        pf = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(nl, n)]) * 1e3
        lay = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(nl, n)]) * 1e3
        return idx.view(n, wl.K).cpu().numpy(), pf, lay

    ids, _, cold = run(None)
    chosen = [np.unique(r) for r in ids]

    def guess_table(src):
        t = np.full((n, wl.K + wl.S), -1, dtype=np.int32)   # -1 entries are skipped
        for i in range(nl, n):
            row = np.concatenate([chosen[src(i)], shared])
            t[i, :len(row)] = row
        return torch.from_numpy(t).to(dev)

    hits = [len(np.intersect1d(chosen[i - nl], chosen[i])) / len(chosen[i]) for i in range(nl, n)]
    res = {"rho": rho, "steps": n_steps, "layers": nl, "timed_calls": n - nl,
           "hit_rate_previous_step": float(np.mean(hits)),
           "cold_layer_us": float(cold.mean())}
    same = True
    for label, src in (("previous", lambda i: i - nl), ("exact", lambda i: i)):
        g = guess_table(src)
        ids2, pf, lay = run(g)
        same = same and bool(np.array_equal(ids2, ids))
        nb = wl.expert_bytes() * float(np.mean([(g[i] >= 0).sum().item() for i in range(nl, n)]))
        res[label] = {"prefetch_us": float(pf.mean()), "layer_us": float(lay.mean()),
                      "total_us": float(pf.mean() + lay.mean()),
                      "saving_us": float(cold.mean() - pf.mean() - lay.mean()),
                      "prefetch_gbs": float(nb / (pf.mean() * 1e-6) / 1e9)}
    res["routing_identical_in_all_passes"] = same
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


def cpu_baseline(seconds, chain_probe=None):
    """The oracle as it stands, on the host cores, over bounded samples; weight
    generation is never timed.

    value: the headline workload (Ling layer, M=1) on every core, as GB/s of the
    unique weight bytes a call needs.  extra: the same layer at M=6 on every core;
    single-thread figures for the tiny layer and the Ling layer at M=1; and one
    16-layer pre-norm chain + lm_head at M=6 on every core, on the rows of the GPU
    chain's probe call, with the oracle's tokens and routing set against the GPU's."""
    import numpy as np

    import oracle
    from datagen import workloads as W

    cores = len(os.sched_getaffinity(0))

    def pool_of(wl, n):
        # n problems, each on its own layer and input rows, with the selected
        # experts' weights generated once
        pool = []
        for l in range(n):
            x = W.x_rows(wl, [1000 + l * wl.M + m for m in range(wl.M)])
            wr = W.router(wl, l)
            idx, _, _ = oracle.router_topk(x, wr, wl.K)
            used = sorted(set(int(e) for e in idx.ravel())) + list(range(wl.E, wl.E + wl.S))
            gu = {e: W.expert_gate_up(wl, l, e) for e in used}
            dn = {e: W.expert_down(wl, l, e) for e in used}
            pool.append((x, wr, gu, dn, wl.router_bytes() + len(used) * wl.expert_bytes()))
        return pool

    def run(wl, pool, budget, threads):
        oracle.set_threads(threads)
        times, nbytes = [], []
        s = 0
        while sum(times) < budget or s < 2:
            x, wr, gu, dn, nb = pool[s % len(pool)]
            t0 = time.perf_counter()
            idx, gate, _ = oracle.router_topk(x, wr, wl.K)
            acc = oracle.experts_combine(x, idx, gate, gu, dn, wl.E, wl.S)
            oracle.cast_bf16(acc)
            times.append(time.perf_counter() - t0)
            nbytes.append(nb)
            s += 1
        t = np.array(times)
        return {"calls": len(t), "us_per_layer": round(float(t.mean() * 1e6), 1),
                "gbs": round(float(np.sum(nbytes) / t.sum() / 1e9), 3), "threads": threads,
                "seconds": round(float(t.sum()), 2)}

    # headline workload: ~1.7 GB of weights over 16 problems, well beyond the host caches
    p2 = pool_of(W.C2, N_LAYERS)
    head = run(W.C2, p2, 0.5 * seconds, cores)
    extra = {W.C2.name + "_1thread": run(W.C2, p2, 0.2 * seconds, 1)}
    del p2
    p1 = pool_of(W.C1, N_LAYERS)
    extra[W.C1.name + "_1thread"] = run(W.C1, p1, 0.05 * seconds, 1)
    p3 = pool_of(W.C3, 4)
    extra[W.C3.name] = run(W.C3, p3, 0.25 * seconds, cores)
    del p3
    if chain_probe is not None:
        extra[W.C5.name] = _cpu_chain(W.C5, chain_probe, cores)
    return {"value": head["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_layer": head["us_per_layer"],
            "sample": "%d Ling MoE layer calls at M=1 (router, top-k, 8 routed + shared experts, "
                      "combine) cycling over 16 pre-generated problems, %.1f s of oracle time; "
                      "extra: the same at M=6, single-thread tiny and Ling M=1 layers, one "
                      "16-layer chain + lm_head at M=6" % (head["calls"], head["seconds"]),
            "extra": extra}


def _cpu_chain(wl, probe, cores):
    """One free-running oracle chain (pre-norm, residual, 16 layers, then the lm_head
    argmax) on the probe's rows, composed as the oracle's own chain runner composes it;
    only the arithmetic is timed.  Reports the first layer whose routing differs from
    the GPU's (as sets per row) and how many of the tokens agree."""
    import numpy as np

    import oracle
    from datagen import workloads as W

    oracle.set_threads(cores)
    h = W.x_rows(wl, probe["rows"])
    t = 0.0
    first_diff = None
    for l in range(wl.n_layers):
        gain, wr, bias = W.norm_gain(wl, l), W.router(wl, l), W.router_bias(wl, l)
        t0 = time.perf_counter()
        u = oracle.rmsnorm(h, gain=gain) if wl.prenorm else h
        idx, gate, _ = oracle.router_topk(u, wr, wl.K, bias)
        t += time.perf_counter() - t0
        used = sorted(set(int(e) for e in idx.ravel())) + list(range(wl.E, wl.E + wl.S))
        gu = {e: W.expert_gate_up(wl, l, e) for e in used}
        dn = {e: W.expert_down(wl, l, e) for e in used}
        t0 = time.perf_counter()
        acc = oracle.experts_combine(u, idx, gate, gu, dn, wl.E, wl.S, wl.routed_scale)
        h = oracle.residual(h, acc)
        t += time.perf_counter() - t0
        if first_diff is None and not all(
                set(idx[m].tolist()) == set(probe["idx"][l, m].tolist()) for m in range(wl.M)):
            first_diff = l
    lm = W.lmhead(wl)
    t0 = time.perf_counter()
    tok, _ = oracle.lmhead_argmax(h, lm)
    t += time.perf_counter() - t0
    return {"us_per_step": round(t * 1e6, 1), "threads": cores,
            "tokens_equal_to_gpu": "%d/%d" % (int(np.sum(tok == probe["tokens"])), wl.M),
            "first_layer_routing_differs_from_gpu": first_diff}


if __name__ == "__main__":
    main()
