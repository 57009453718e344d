"""Benchmark: one clustered-sparse-attention layer (all four stages) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload cog76k] [--no-cpu] [--no-dense]

A step is one cold layer call on seeded synthetic Q/K/V already resident in HBM
(3 warm-up + 20 timed steps by default; per-step median/p10/p90 from HIP events,
and the latency/density spread over seeds 1 and 2):
cluster_q -> cluster_k (threshold-adaptive) -> select (TensorQuest + top-p) ->
sparse_attn. The headline value is the dense-equivalent throughput
4 H N^2 D / t_layer of that cold call. The warm-start steady state (later
denoising steps on drifted inputs, starting from the previous centres) is
reported beside it, with the latency amortised over the denoising schedule.
Prints one JSON line (last line of stdout).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "clustered-attn layer latency (ms) + dense-equiv TFLOP/s at 75.6K tokens"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
CALIB_BYTES = 512 << 20   # plain copy used to calibrate the memory counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_layer(torch, adc, q, k, v, cfg, stream, prev=None, select_kw=None, want_lse=True,
                serial=False):
    """One layer as the package schedules it (the two clusterings overlapped on
    two streams, then selection and attention), with timing events. Returns
    (Q, K, S, out, times) where times() gives the layer and per-stage
    milliseconds once the stream has finished. serial: the query clustering,
    then the key clustering, on the one stream (each stage's kernels alone on
    the GPU, for profiles)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    ev[0].record(stream)
    if serial and prev is None:
        ev[1].record(stream)
        Q = adc.cluster_q(q, cfg.q_clusters, cfg.iters, cfg.init, cfg.seed)
        ev[2].record(stream)
        ev[3].record(stream)
        K = adc.cluster_k(k, v, cfg.k_base, cfg.k_max, cfg.iters, cfg.tau_mult, cfg.adaptive, cfg.init,
                          cfg.seed)
        ev[4].record(stream)
        ev[5].record(stream)
    else:
        Q, K = adc.cluster_layer(q, k, v, cfg, prev=prev, events=ev[1:6])
    S = adc.select(Q["qrep"], K, cfg.top_p, q_offsets=Q["offsets"], **(select_kw or {}))
    ev[6].record(stream)
    out, _ = adc.sparse_attn(q, Q["perm"], Q["offsets"], K["k_perm"], K["v_perm"], K["offsets"],
                             S["mask"], want_lse=want_lse)
    ev[7].record(stream)

    def times():
        return {"layer": ev[0].elapsed_time(ev[7]), "cluster_q": ev[1].elapsed_time(ev[2]),
                "cluster_k": ev[3].elapsed_time(ev[4]), "select": ev[5].elapsed_time(ev[6]),
                "sparse_attn": ev[6].elapsed_time(ev[7])}
    return Q, K, S, out, times


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="cog76k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparisons")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the latency/density spread over seeds 1 and 2")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the 65-q-cluster / top-k / centroid-score variants")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the per-layer count / Nmax calibration on a synthetic layer stack")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm-start steady-state steps (drifted inputs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (a few layers each)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured GEMM and copy ceilings")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-captured layer (LayerGraph replays)")
    ap.add_argument("--cpu-heads", default=None,
                    help="heads the oracle baseline runs: 'all', or a comma list (default: 4 spread heads)")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only warmup + timed steps (for profiler runs)")
    ap.add_argument("--serial-clustering", action="store_true",
                    help="run the query and key clusterings one after the other on one stream")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the heads of a layer would be split across GPUs, with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import clustered_sparse_attention_cosine_amd as adc
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    g = synth.generate(w, seed=args.seed)
    log(f"generated {w.name} inputs in {time.time() - t0:.1f}s")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = (to_dev(g[t]) for t in "qkv")
    nmax = w.k_max
    cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=nmax, top_p=w.top_p,
                          iters=w.iters, init=w.init, adaptive=w.k_adaptive, seed=args.seed)
    stream = torch.cuda.current_stream(dev)

    def step(record=None):
        Q, K, S, out, times = timed_layer(torch, adc, q, k, v, cfg, stream, serial=args.serial_clustering)
        if record is not None:
            record.append(times)
        return Q, K, S, out

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    events = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        Q, K, S, out = step(events)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {t_total:.3f}s")
    ms = t_total * 1e3 / args.steps
    stage_names = ["cluster_q", "cluster_k", "select", "sparse_attn"]
    events = [t() for t in events]
    stage_ms = {n: float(np.mean([e[n] for e in events])) for n in stage_names}
    per_step = np.array([e["layer"] for e in events])
    layer_stats = {"median": round(float(np.median(per_step)), 4),
                   "p10": round(float(np.percentile(per_step, 10)), 4),
                   "p90": round(float(np.percentile(per_step, 90)), 4)}

    # workload facts from the last step (query-key pairs counted by adacluster_select)
    pairs = float(S["pairs"].sum().item())
    density = pairs / (w.B * w.H * float(w.N) ** 2)
    slots = K["n_clusters"].flatten().tolist()
    full_heads = int(K["full"].sum().item())
    dense_flops = w.dense_flops()
    value = dense_flops / (ms * 1e-3) / 1e12
    attn_flops = 4.0 * w.D * pairs
    attn_tflops = attn_flops / (stage_ms["sparse_attn"] * 1e-3) / 1e12
    if args.profile_steps:
        # a plain device copy of known size, to calibrate memory counters
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        # shapes of the timed layer's assignment passes, for counter summaries:
        # rows, centres per query/key stage-0 round, and the final key
        # assignment's slots (every slot up to the last one holding a centre)
        ss = K["stage_sizes"].cpu().numpy().reshape(-1, 8)
        meff = []
        for row in ss:
            base, t, last = 0, 0, 0
            while base < nmax and t < 8 and row[t] > 0:
                mt = min(w.k_base if t == 0 else w.k_base << (t - 1), nmax - base)
                last = base + min(mt, int(row[t]))
                base += mt
                t += 1
            meff.append(last)
        log(json.dumps(dict(ms_per_step=ms, stages_ms=stage_ms, calib_copy_bytes=CALIB_BYTES,
                            schedule="serial" if args.serial_clustering else "two streams",
                            shapes=dict(rows=w.B * w.H * w.N, D=w.D, q_clusters=w.q_clusters,
                                        k_base=w.k_base, k_max=nmax, heads=w.B * w.H,
                                        elem_bytes=2 if w.dtype == "bf16" else 4, iters=w.iters,
                                        k_final_slots_mean=float(np.mean(meff))))))
        return

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s (dense-equivalent, 4*H*N^2*D / layer time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded smooth fields + noise, shapes of the workload)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} D={w.D} grid={w.grid}",
                   "q_clusters": w.q_clusters,
                   "k_clusters": f"adaptive {{{w.k_base},{2 * w.k_base},{4 * w.k_base}}}"
                   if w.k_adaptive else str(w.k_base),
                   "top_p": w.top_p, "lloyd_iters": w.iters, "init": w.init,
                   "layer_ms": round(ms, 4)},
        "stages_ms": {k2: round(v2, 4) for k2, v2 in stage_ms.items()},
        "schedule": ("cluster_q, then cluster_k, on one stream, then select and sparse_attn"
                     if args.serial_clustering else
                     "cluster_q on a side stream beside cluster_k (their stage times overlap), then select and sparse_attn"),
        "layer_ms_events": layer_stats,
        "selection": {"pairs": pairs, "density": round(density, 5), "full_heads": full_heads,
                      "k_slots": {str(s): slots.count(s) for s in sorted(set(slots))}},
        "roofline": {"kernel": "sparse_attn (run build + work list + attention)",
                     "bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "algorithmic_flops": attn_flops},
        "stage_rooflines": stage_rooflines(w.name),
    }

    if not args.no_graph:
        result["graph"] = graph_replay(torch, adc, q, k, v, cfg, out, args.steps, dense_flops)

    if not args.no_dense:
        result["dense"] = dense_compare(torch, adc, q, k, v, w, dev, stream)

    if not args.no_variants:
        bits = np.unpackbits(S["mask"].cpu().numpy().view(np.uint8), bitorder="little")
        mean_slots = float(bits.sum()) / (w.B * w.H * w.q_clusters)
        result["variants"] = variants(torch, adc, w, cfg, q, k, v, stream, args.seed, mean_slots)

    if not args.no_warm:
        result["warm_steady_state"] = warm_steady_state(
            torch, adc, synth, w, cfg, dev, stream, layer_stats["median"], q, k, v, args.seed)

    if not args.no_calib:
        result["calibration"] = calibration(torch, adc, synth, dev, stream)

    if not args.no_spread or not args.no_configs or not args.no_ceilings:
        del q, k, v, Q, K, S, out
    if not args.no_spread:
        result["spread"] = seed_spread(torch, adc, synth, w, cfg, dev, stream)

    if not args.no_configs:
        result["configs"] = other_configs(torch, adc, synth, dev, stream)

    if not args.no_ceilings:
        result["ceilings"] = ceilings(torch, dev, stream)

    if not args.no_cpu:
        heads = args.cpu_heads
        if heads not in (None, "all"):
            heads = [int(x) for x in heads.split(",")]
        result["cpu_baseline"] = cpu_baseline(w, g, args.seed, heads)

    print(json.dumps(result), flush=True)


def graph_replay(torch, adc, q, k, v, cfg, eager_out, steps, dense_flops):
    """The same layer captured once in a HIP graph (LayerGraph) and replayed
    `steps` times on the same inputs: wall time per replay, and whether the
    replays' output equals the eager layer's bit for bit."""
    lg = adc.LayerGraph(q, k, v, cfg)
    lg.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        out, _, _ = lg.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    same = bool(torch.equal(out, eager_out))
    del lg
    torch.cuda.empty_cache()
    log(f"graph replay {ms:.3f} ms per layer, same output as eager: {same}")
    return {"layer_ms": round(ms, 4), "dense_equiv_tflops": round(dense_flops / (ms * 1e-3) / 1e12, 3),
            "same_output_as_eager": same, "steps": steps,
            "note": "every kernel of the layer recorded once (LayerGraph), one graph launch per layer"}


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary
    (profiles/attn_<workload>_pmc.txt), or None when that summary is missing or
    was taken on a different attention kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_{workload}_pmc.txt")
    src = os.path.join(ROOT, "clustered_sparse_attention_cosine_amd", "csrc", "attn.hip")
    if not os.path.exists(path):
        return None
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    text = open(path).read()
    if f"attn.hip sha256[:16] = {digest}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_bytes = "):
            return int(line.split("=")[1])
    return None


def seed_spread(torch, adc, synth, w, cfg, dev, stream, seeds=(1, 2), steps=5):
    """Layer latency and achieved density on other seeds of the same workload."""
    out = []
    for seed in seeds:
        g = synth.generate(w, seed=seed)
        q, k, v = (torch.from_numpy(g[t].view(np.int16)).view(torch.bfloat16).to(dev)
                   if g[t].dtype == np.uint16 else torch.from_numpy(g[t]).to(dev) for t in "qkv")
        del g
        times = []
        cs = dataclasses.replace(cfg, seed=seed)
        for i in range(2 + steps):
            Q, K, S, _, tm = timed_layer(torch, adc, q, k, v, cs, stream, want_lse=False)
            torch.cuda.synchronize()
            if i >= 2:
                times.append(tm()["layer"])
        pairs = float(S["pairs"].sum().item())
        out.append({"seed": seed, "layer_ms_median": round(float(np.median(times)), 4),
                    "density": round(pairs / (w.B * w.H * float(w.N) ** 2), 5),
                    "full_heads": int(K["full"].sum().item())})
        log(f"seed {seed}: {out[-1]}")
        del q, k, v, Q, K, S
    return out


def warm_steady_state(torch, adc, synth, w, cfg, dev, stream, cold, q0, k0, v0, seed,
                      n_steps=4, warm_iters=(1, 5)):
    """Denoising steps after the first (section 3.2.2): inputs drift (the
    generator's steps 1..n_steps), both clusterings start from the previous
    step's centres and the keys keep their per-head counts and flags. Each chain
    (cold step on step 0, then the warm steps) runs twice; the second is timed.
    Reports the warm-step latency, the latency amortised over the model's
    denoising schedule (30 steps for HunyuanVideo, 50 otherwise), and the key
    clusterings' compactness (mean MSE and Davies-Bouldin index over heads, the
    diagnostics of section 3.2.1 and Fig. 10) beside a cold clustering of the
    last step."""
    t0 = time.time()
    steps = []
    for s in range(1, n_steps + 1):
        g = synth.generate(w, seed=seed, step=s)
        steps.append(tuple(torch.from_numpy(g[t].view(np.int16)).view(torch.bfloat16).to(dev)
                           if g[t].dtype == np.uint16 else torch.from_numpy(g[t]).to(dev)
                           for t in "qkv"))
        del g
    log(f"generated {n_steps} drifted steps in {time.time() - t0:.1f}s")
    names = ["cluster_q", "cluster_k", "select", "sparse_attn"]
    total_steps = 30 if w.name.startswith("hun") else 50
    res = {"drift_rad_per_step": synth.DRIFT, "denoising_steps": total_steps,
           "cold_layer_ms": round(cold, 4)}
    for wi in warm_iters:
        for rep in range(2):
            prev = None
            rows = []
            cw = dataclasses.replace(cfg, seed=seed, warm_iters=wi)
            for s, (q, k, v) in enumerate([(q0, k0, v0)] + steps):
                Q, K, S, _, tm = timed_layer(torch, adc, q, k, v, cw, stream, prev=prev,
                                             want_lse=False)
                prev = dict(Q=Q, K=K)
                torch.cuda.synchronize()
                tm = tm()
                pairs = float(S["pairs"].sum().item())
                C = adc.compactness(K["k_perm"], K["offsets"], K["centroids"])
                rows.append(dict(t=[tm[n] for n in names], layer=tm["layer"],
                                 density=pairs / (w.B * w.H * float(w.N) ** 2),
                                 key_mse=float(C["mse"].mean().item()),
                                 key_db=float(C["db"].mean().item())))
        warm = rows[1:]
        layer = [r["layer"] for r in warm]
        wm = float(np.median(layer))
        res[f"lloyd_iters_{wi}"] = {
            "warm_layer_ms_median": round(wm, 4),
            "warm_layer_ms_per_step": [round(x, 4) for x in layer],
            "stages_ms_median": {n: round(float(np.median([r["t"][i] for r in warm])), 4)
                                 for i, n in enumerate(names)},
            "density_per_step": [round(r["density"], 5) for r in warm],
            "key_mse_per_step": [round(r["key_mse"], 5) for r in warm],
            "key_db_per_step": [round(r["key_db"], 5) for r in warm],
            "amortized_layer_ms": round((cold + (total_steps - 1) * wm) / total_steps, 4),
        }
        log(f"warm steady state, {wi} Lloyd round(s): {res[f'lloyd_iters_{wi}']}")
    # a cold clustering of the last drifted step, for the compactness comparison,
    # and the cost of the diagnostic itself
    q, k, v = steps[-1]
    K = adc.cluster_k(k, v, cfg.k_base, cfg.k_max, cfg.iters, cfg.tau_mult, cfg.adaptive,
                      cfg.init, seed)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    adc.compactness(K["k_perm"], K["offsets"], K["centroids"])
    ev[0].record(stream)
    C = adc.compactness(K["k_perm"], K["offsets"], K["centroids"])
    ev[1].record(stream)
    torch.cuda.synchronize()
    res["cold_last_step"] = {"key_mse": round(float(C["mse"].mean().item()), 5),
                             "key_db": round(float(C["db"].mean().item()), 5),
                             "comp": round(float(C["comp"][0].item()), 6)}
    res["compactness_ms"] = round(ev[0].elapsed_time(ev[1]), 4)
    log(f"cold clustering of step {n_steps}: {res['cold_last_step']}, "
        f"diagnostic {res['compactness_ms']} ms")
    del steps, K, C
    return res


def variants(torch, adc, w, cfg, q, k, v, stream, seed, mean_slots, steps=5):
    """Cold-layer latency under the pages' other settings: 65 query clusters
    (section 4.1), the argtopk rule of Algorithm 3 step 7 with k equal to the
    mean number of slots top-p selected above, and the centroid score of the
    prior clustering method (section 2.3)."""
    top_k = max(1, int(round(mean_slots)))
    settings = {"q_clusters_65": dict(cq=65, score="quest", rule="topp"),
                f"topk_{top_k}": dict(cq=cfg.q_clusters, score="quest", rule="topk"),
                "centroid_score": dict(cq=cfg.q_clusters, score="centroid", rule="topp")}
    res = {"topk_k": top_k}
    for name, st in settings.items():
        rows = []
        cv = dataclasses.replace(cfg, seed=seed, q_clusters=st["cq"])
        for i in range(2 + steps):
            Q, K, S, _, tm = timed_layer(torch, adc, q, k, v, cv, stream,
                                         select_kw=dict(score=st["score"], rule=st["rule"],
                                                        top_k=top_k), want_lse=False)
            torch.cuda.synchronize()
            if i >= 2:
                rows.append(tm())
        pairs = float(S["pairs"].sum().item())
        res[name] = {"layer_ms_median": round(float(np.median([r["layer"] for r in rows])), 4),
                     "stages_ms_median": {n: round(float(np.median([r[n] for r in rows])), 4)
                                          for n in ["cluster_q", "cluster_k", "select",
                                                    "sparse_attn"]},
                     "density": round(pairs / (w.B * w.H * float(w.N) ** 2), 5)}
        log(f"variant {name}: {res[name]}")
        del Q, K, S
    return res


def calibration(torch, adc, synth, dev, stream, n_layers=8, top_frac=0.15, comp_clusters=400):
    """The per-layer study of sections 3.2.1 and 4.1 on a synthetic stack of
    CogVideoX-17.7K-shaped layers (keys more scattered and heavier-tailed from
    layer to layer): each layer's required key-cluster count (Algorithm 1 with a
    16 m0 cap), its compactness Comp_l at 400 centres (Fig. 4), the cap that
    sends the top 15 % of layers to full attention, and the heads on full
    attention at that cap."""
    from clustered_sparse_attention_cosine_amd import calibrate
    w = synth.WORKLOADS["cog17k"]
    t0 = time.time()
    layers = []
    for lw, seed in synth.layer_stack(w, n_layers):
        g = synth.generate(lw, seed=seed)
        layers.append(tuple(torch.from_numpy(g[t].view(np.int16)).view(torch.bfloat16).to(dev)
                            for t in "kv"))
        del g
    log(f"generated {n_layers} stacked layers in {time.time() - t0:.1f}s")
    m0 = w.k_base
    calibrate.calibrate_stack(layers[:1], m0, 16 * m0, top_frac, comp_clusters=comp_clusters)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    res = calibrate.calibrate_stack(layers, m0, 16 * m0, top_frac, comp_clusters=comp_clusters)
    e1.record(stream)
    torch.cuda.synchronize()
    out = {"workload": f"{w.name} stack of {n_layers} layers: B=1 H={w.H} N={w.N} D={w.D}",
           "m0": m0, "probe_cap": 16 * m0, "top_frac": top_frac, "kmax": res["kmax"],
           "ms": round(e0.elapsed_time(e1), 3), "layers": []}
    for (lw, _), p in zip(synth.layer_stack(w, n_layers), res["layers"]):
        out["layers"].append({"noise_std": round(lw.noise_std, 4), "noise_df": round(lw.noise_df, 3),
                              "required": p["required"], "comp": round(p["comp"], 5),
                              "head_counts": {str(c): int((p["head_counts"] == c).sum())
                                              for c in sorted(set(p["head_counts"].tolist()))},
                              "full_heads_at_kmax": int(p["full_at_kmax"].sum())})
    log(f"calibration: kmax {res['kmax']}, " + "; ".join(
        f"req {l['required']} comp {l['comp']} full {l['full_heads_at_kmax']}" for l in out["layers"]))
    del layers
    return out


def other_configs(torch, adc, synth, dev, stream, names=("tiny", "cog17k", "wan33k", "hun119k"),
                  steps=5, warmup=2):
    """The other workloads, a few cold layers each on seed 0: layer and stage
    latency, density, the sparse attention's useful rate (4 D pairs / its
    time) against the bf16 peak, and dense attention on the same inputs (this
    library's kernel with everything selected; PyTorch SDPA, flash backend)."""
    res = {}
    for name in names:
        w = synth.WORKLOADS[name]
        t0 = time.time()
        g = synth.generate(w, seed=0)
        q, k, v = (torch.from_numpy(g[t].view(np.int16)).view(torch.bfloat16).to(dev)
                   if g[t].dtype == np.uint16 else torch.from_numpy(g[t]).to(dev) for t in "qkv")
        del g
        cfg = adc.LayerConfig(q_clusters=w.q_clusters, k_base=w.k_base, k_max=w.k_max,
                              top_p=w.top_p, iters=w.iters, init=w.init, adaptive=w.k_adaptive)
        rows = []
        for i in range(warmup + steps):
            Q, K, S, _, tm = timed_layer(torch, adc, q, k, v, cfg, stream, want_lse=False)
            torch.cuda.synchronize()
            if i >= warmup:
                rows.append(tm())
        pairs = float(S["pairs"].sum().item())
        stages = {n: round(float(np.median([r[n] for r in rows])), 4)
                  for n in ["cluster_q", "cluster_k", "select", "sparse_attn"]}
        lm = float(np.median([r["layer"] for r in rows]))
        useful = 4.0 * w.D * pairs / (stages["sparse_attn"] * 1e-3) / 1e12
        slots = K["n_clusters"].flatten().tolist()
        entry = {"workload": f"B={w.B} H={w.H} N={w.N} D={w.D} {w.dtype}",
                 "layer_ms_median": round(lm, 4),
                 "dense_equiv_tflops": round(w.dense_flops() / (lm * 1e-3) / 1e12, 2),
                 "stages_ms_median": stages, "density": round(pairs / (w.B * w.H * float(w.N) ** 2), 5),
                 "full_heads": int(K["full"].sum().item()),
                 "k_slots": {str(c): slots.count(c) for c in sorted(set(slots))},
                 "sparse_attn_useful_tflops": round(useful, 2),
                 "sparse_attn_frac_bf16_peak": round(useful / PEAK_BF16_TFLOPS, 4)}
        del Q, K, S
        entry["dense"] = dense_compare(torch, adc, q, k, v, w, dev, stream)
        res[name] = entry
        log(f"config {name} ({time.time() - t0:.1f}s): {entry}")
        del q, k, v
    return res


def dense_compare(torch, adc, q, k, v, w, dev, stream):
    """Dense attention on the same GPU: this library's kernel with everything
    selected, and PyTorch's fused SDPA (flash backend only)."""
    res = {}
    B, H, N, D = q.shape
    ident = torch.arange(N, dtype=torch.int32, device=dev).repeat(B, H, 1).contiguous()
    offs = torch.tensor([0, N], dtype=torch.int32, device=dev).repeat(B, H, 1).contiguous()
    mask = torch.ones(B, H, 1, 1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    adc.sparse_attn(q, ident, offs, k, v, offs, mask, want_lse=False)
    torch.cuda.synchronize()
    e0.record(stream)
    adc.sparse_attn(q, ident, offs, k, v, offs, mask, want_lse=False)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1)
    res["own_select_all_ms"] = round(t, 3)
    res["own_select_all_tflops"] = round(w.dense_flops() / (t * 1e-3) / 1e12, 2)
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(q, k, v)
            torch.cuda.synchronize()
            e0.record(stream)
            torch.nn.functional.scaled_dot_product_attention(q, k, v)
            e1.record(stream)
            torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        res["torch_sdpa_flash_ms"] = round(t, 3)
        res["torch_sdpa_flash_tflops"] = round(w.dense_flops() / (t * 1e-3) / 1e12, 2)
    except Exception as exc:  # flash backend unavailable: report, never fall back to math
        res["torch_sdpa_flash_ms"] = None
        res["torch_sdpa_error"] = str(exc)[:200]
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, g, seed, heads=None):
    """The CPU oracle (as it stands) on a sample of heads of the same workload,
    all four stages, each timed on its own; scaled to the dense-equivalent unit
    as (4 N^2 D) x heads / t. The sample keeps the default run to about 20 s of
    host time; heads="all" times the whole layer. Threads: the host's share
    for one GPU (at most 16, the worker budget of a one-GPU machine), OpenMP over
    independent outputs."""
    import oracle
    import synth
    nproc = len(os.sched_getaffinity(0))
    threads = min(nproc, 16)
    oracle.set_threads(threads)
    if heads == "all":
        heads = list(range(w.H))
    elif heads is None:
        heads = sorted({0, w.H // 3, (2 * w.H) // 3, w.H - 1})
    scale = 1.0 / math.sqrt(w.D)
    st = {"cluster_q": 0.0, "cluster_k": 0.0, "select": 0.0, "sparse_attn": 0.0}
    t0 = time.perf_counter()
    for h in heads:
        qh, kh, vh = (synth.as_f32(g[t][0, h]) for t in "qkv")
        ta = time.perf_counter()
        Q = oracle.cluster_q(qh, w.q_clusters, w.iters, init=w.init, seed=seed, h=h)
        tb = time.perf_counter()
        K = oracle.cluster_k(kh, w.k_base, w.k_max if w.k_adaptive else w.k_base, w.iters,
                             adaptive=w.k_adaptive, init=w.init, seed=seed, h=h)
        tc = time.perf_counter()
        ck = K["n_slots"]
        S = oracle.quest_scores(Q["qrep"], K["kmax"][:ck], K["kmin"][:ck], K["sizes"][:ck])
        sel = oracle.select_topp(S, K["sizes"][:ck], scale, w.top_p, full=bool(K["full"]))
        td = time.perf_counter()
        oracle.sparse_attn(qh, kh, vh, Q["lab"], K["lab"], w.q_clusters, ck, sel["mask"], scale)
        te = time.perf_counter()
        for n, dt in zip(st, (tb - ta, tc - tb, td - tc, te - td)):
            st[n] += dt
        log(f"oracle head {h} done at {time.perf_counter() - t0:.1f}s")
    t = time.perf_counter() - t0
    flops = 4.0 * float(w.N) ** 2 * w.D * len(heads)
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s (dense-equivalent)",
            "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"heads {heads} of {w.H}, all four stages, N={w.N}: {t:.1f} s "
                      f"(layer estimate {t * w.H / len(heads):.0f} s)",
            "seconds": round(t, 2), "layer_seconds_estimate": round(t * w.H / len(heads), 1),
            "stage_seconds": {n: round(v, 2) for n, v in st.items()},
            "nproc": nproc, "cpu_model": cpu_model()}


def ceilings(torch, dev, stream):
    """Measured ceilings of this GPU beside the spec peaks: a large bf16 GEMM
    (torch.matmul, 8192^3) and a 1 GiB device-to-device copy (bytes read plus
    bytes written)."""
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    res["bf16_gemm_tflops"] = round(2.0 * n ** 3 / (t * 1e-3) / 1e12, 1)
    res["bf16_gemm_shape"] = f"{n}x{n}x{n} torch.matmul"
    del a, b
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    res["copy_gbs"] = round(2.0 * src.numel() * 4 / (t * 1e-3) / 1e9, 1)
    res["copy_bytes"] = src.numel() * 4
    res["spec_peaks"] = {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    del src, dst
    return res


def stage_rooflines(workload):
    """Per-kernel roofline entries of the other stages (k-means assignment on
    the matrix cores; centroid update and cluster gather against HBM), read
    from the committed counter summary profiles/clustering_<workload>_pmc.txt
    while the kmeans.hip, permute.hip and select.hip it was taken on are the
    ones in the tree; None otherwise."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"clustering_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    for src in ("kmeans.hip", "permute.hip", "select.hip"):
        with open(os.path.join(ROOT, "clustered_sparse_attention_cosine_amd", "csrc", src), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()[:16]
        if f"{src} sha256[:16] = {digest}" not in text:
            return None
    out = []
    for line in text.splitlines():
        if line.startswith("roofline "):
            out.append(json.loads(line[len("roofline "):]))
    return out or None


if __name__ == "__main__":
    main()
