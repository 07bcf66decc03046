#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on one MI355X.

One step = one moe_run (route planner, MXFP8 quantiser, GEMM1 + SwiGLU +
requantiser, GEMM2 + combine) over one batch, inputs already resident in HBM.
Steps cycle through --layers independent copies of the expert weights so the
decode working set (about 0.22 GB of distinct experts per layer) cannot be
served from the 256 MB last-level cache, as in a real stack of layers.

Prints ONE JSON line. `value` is tokens/s per layer (live tokens / median layer
time) of the headline workload (the 8-token decode batch); `ms_per_step` is the
median over --samples replays of one captured graph that runs exactly --steps
layers, with p10 / p90 beside it; `roofline` is for the dominant kernel, timed
live with HIP events recorded by the library on the launch stream;
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload
on this host's cores. `secondary` carries the same measurement for the prefill
batch (both combine modes) and the NVFP4 and hybrid workloads, each with its own
roofline.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_scaled_fp4_histogram_amd import inputs as I  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
METRIC = "routed-MoE tokens/s per layer + % HBM peak (decode) / % MFMA peak (prefill)"
STAGES = ("route", "gemm1", "gemm2", "combine")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(fmt, K, N):
    """(w13+s13, w2+s2) bytes of one expert in the checkpoint format."""
    if fmt == I.FMT_MXFP4:
        per = lambda rows, cols: rows * cols // 2 + rows * cols // 32
    elif fmt == I.FMT_NVFP4:
        per = lambda rows, cols: rows * cols // 2 + rows * cols // 16
    else:
        per = lambda rows, cols: rows * cols // 8 * 3 + rows * cols // 32
    return per(2 * N, K), per(K, N)


def algorithmic(prob):
    """Algorithmic bytes and flops of one layer and of each GEMM kernel: weights of the
    distinct experts touched (each read once), activations in, results out."""
    c = prob.cfg
    ids = prob.ids
    valid = (ids >= 0) & (ids < c.E)
    live = int(valid.any(axis=1).sum())
    routes = int(valid.sum())
    distinct = np.unique(ids[valid])
    w1 = w2 = 0
    for g in distinct:
        for t in prob.tiers:
            e = int(g) if t.emap is None else int(t.emap[g])
            if 0 <= e < t.E:
                a, b = expert_bytes(t.fmt, c.K, c.N)
                w1 += a
                w2 += b
                break
    a8 = prob.tiers[0].fmt == I.FMT_MXFP4
    x_in = live * c.K * ((1 + 1 / 32) if a8 else 2)        # activation operand as GEMM1 reads it
    h_bytes = routes * c.N * ((1 + 1 / 32) if a8 else 2)   # intermediate written by GEMM1, read by GEMM2
    out_bytes = live * c.K * 2                              # bf16 output rows
    flops1 = 2.0 * routes * 2 * c.N * c.K
    flops2 = 2.0 * routes * c.K * c.N
    return dict(live=live, routes=routes, distinct=int(len(distinct)),
                layer_bytes=w1 + w2 + live * c.K * 2 + out_bytes,
                gemm1_bytes=w1 + x_in + h_bytes, gemm2_bytes=w2 + h_bytes + out_bytes,
                gemm1_flops=flops1, gemm2_flops=flops2, layer_flops=flops1 + flops2)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("moe_kernels.hip", "moe_decode.hip", "moe_prefill.hip", "moe_device.h", "moe_common.h"):
        with open(os.path.join(ROOT, "block_scaled_fp4_histogram_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel, per_launch_units):
    """HBM bytes per launch of `kernel` from the committed PMC summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def pmc_summary(args):
    """HBM bytes per launch of one kernel from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE; counter_collection.csv each), scaled by what the same counters read for a
    plain device copy of known size (bench.py --copy-calib) run under the same counters."""
    import csv
    fetch, write, cfetch, cwrite = args.pmc_csv

    def kib(path, name_part):
        vals = {}
        for r in csv.DictReader(open(path)):
            if name_part in r["Kernel_Name"]:
                key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        if not vals:
            raise SystemExit(f"no dispatch of {name_part!r} in {path}")
        return sum(vals.values()) / len(vals), len(vals)

    copy_bytes = args.copy_calib_bytes
    f_copy, _ = kib(cfetch, "copyBuffer")
    w_copy, _ = kib(cwrite, "copyBuffer")
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    f_k, n_f = kib(fetch, args.pmc_kernel)
    w_k, n_w = kib(write, args.pmc_kernel)
    read_b, write_b = f_k * 1024.0 * f_scale, w_k * 1024.0 * w_scale
    return {"kernel": args.pmc_kernel, "workload": args.config + ("_det" if args.deterministic else ""),
            "kernel_source_sha256_16": kernel_source_hash(),
            "dispatches": [n_f, n_w], "fetch_kib_per_dispatch": round(f_k, 1),
            "write_kib_per_dispatch": round(w_k, 1),
            "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(f_copy, 1), "write_kib": round(w_copy, 1),
                                 "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
            "hbm_read_bytes_per_launch": round(read_b), "hbm_write_bytes_per_launch": round(write_b),
            "hbm_bytes_per_launch": round(read_b + write_b)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(prob, seconds, live_rows):
    """The oracle, as it stands, on a bounded sample of the workload's rows."""
    import oracle as O
    O.lib()
    rows = live_rows
    t0 = time.perf_counter()
    done = 0
    reps = 0
    while True:
        O.moe_problem(prob, rows=rows)
        done += len(rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return done / el, O.num_threads(), reps, el


# workloads whose weights are the same tensors (same format, geometry and seed):
# one set of prepared layer copies serves all of them
def weight_key(cfg):
    return (cfg.fmt, cfg.E, cfg.K, cfg.N, cfg.hybrid_nvfp4, cfg.e8m0_exp)


def problem(name, tiers_cache):
    """The named workload; its weights come from tiers_cache when another workload of
    the same weights generated them already (they are deterministic in the seed)."""
    cfg = I.CONFIGS[name]
    key = weight_key(cfg)
    if key not in tiers_cache:
        tiers_cache.clear()
        tiers_cache[key] = I.make_problem(name).tiers
    x = I.make_x(cfg.T, cfg.K)
    ids, wts = I.make_routing(cfg.T, cfg.E, cfg.topk, 0, cfg.zipf_s, cfg.pad_rows)
    return I.Problem(cfg, x, ids, wts, tiers_cache[key])


class LayerCopies:
    """`n` independent prepared copies of a problem's expert weights on the GPU."""

    def __init__(self, M, prob, plan, n, dev):
        import torch
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.key = weight_key(prob.cfg)
        host = []
        for t in prob.tiers:
            w = t.weights
            host.append(({k: up(w[k]) for k in ("w13", "s13", "w2", "s2")},
                         None if w["g13"] is None else up(w["g13"]), None if w["g2"] is None else up(w["g2"]),
                         None if t.emap is None else up(t.emap), t))
        self.layers = []
        for li in range(n):
            tiers = []
            for ws, g13, g2, emap, t in host:
                # copies are cloned from the checkpoint-layout upload before any is repacked
                # in place; the last copy repacks the upload itself
                ts = {k: (v if li == n - 1 else v.clone()) for k, v in ws.items()}
                tiers.append((ts, M.Experts(plan, t.fmt, t.E, ts["w13"], ts["s13"], ts["w2"], ts["s2"], g13, g2),
                              emap))
            self.layers.append(tiers)
        log(f"{n} layer copies of {prob.cfg.name}'s weights prepared")
        self.run_tiers = [[(ex, emap) for _, ex, emap in tiers] for tiers in self.layers]


def measure(M, prob, copies, deterministic, args, dev):
    """One workload: median / p10 / p90 layer time over args.samples replays of a graph of
    exactly args.steps layers (cycling the layer copies), per-stage times from the
    library's events, and the roofline of the dominant kernel."""
    import torch
    cfg = prob.cfg
    alg = algorithmic(prob)
    a8 = prob.tiers[0].fmt == I.FMT_MXFP4
    plan = M.Plan(cfg.E, cfg.K, cfg.N, cfg.topk, cfg.limit, M.A_MXFP8 if a8 else M.A_BF16, max_tokens=cfg.T)
    x = torch.from_numpy(prob.x).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(prob.ids).to(dev)
    wts = torch.from_numpy(prob.wts).to(dev)
    out = torch.empty_like(x)
    scratch = M.scratch_for(plan, cfg.T, deterministic, dev)
    rt = copies.run_tiers

    def step(i):
        M.run(plan, rt[i % len(rt)], x, ids, wts, out, deterministic, scratch)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # one graph = exactly args.steps layers, cycling the copies
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for i in range(len(rt)):   # warm the capture stream outside the graph
            step(i)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    samples = args.samples if cfg.T <= 64 else max(10, args.samples // 3)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    us = np.array([1000.0 * e0.elapsed_time(e1) / args.steps for e0, e1 in evs])
    del graph
    med, p10, p90 = (float(np.percentile(us, q)) for q in (50, 10, 90))

    # per-stage durations from events the library records on its launch stream (eager runs)
    nrec = min(args.timing_runs, max(args.steps, 8 * len(rt)))
    plan.enable_stage_timing(nrec)
    for i in range(nrec):
        step(i)
    stage_ms, runs = plan.stage_times()
    plan.enable_stage_timing(0)
    stage_us = {s: 1000.0 * v / max(runs, 1) for s, v in zip(STAGES, stage_ms)}
    sequence = ("decode", "general", "prefill", "prefill_narrow")[plan.sequence(cfg.T) - 1]
    if sequence == "decode":
        # two launches, no route planner or combine kernel: the events bracketing those
        # empty stages measure only their own overhead
        stage_us["route"] = stage_us["combine"] = 0.0

    dominant = max(("gemm1", "gemm2"), key=lambda s: stage_us[s])
    dom_s = stage_us[dominant] * 1e-6
    # the binding roofline of the dominant kernel: the larger of its algorithmic
    # bytes at peak HBM bandwidth and its flops at the peak MFMA rate of its dtype
    mfma_peak = MFMA_PEAK_TFLOPS["fp8" if a8 else "bf16"]
    t_hbm = alg[f"{dominant}_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg[f"{dominant}_flops"] / (mfma_peak * 1e12)
    if t_hbm >= t_mfma:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = alg[f"{dominant}_bytes"] / dom_s / 1e9
    else:
        bound, unit, peak = "mfma", "TFLOP/s", mfma_peak
        achieved = alg[f"{dominant}_flops"] / dom_s / 1e12
    traffic = measured_traffic(cfg.name + ("_det" if deterministic else ""), dominant, 1)
    fmt = "MXFP4 W4A8" if a8 else ("NVFP4+NF3 hybrid" if cfg.hybrid_nvfp4 else "NVFP4 W4A16")
    workload = (f"{cfg.name}: T={cfg.T} ({alg['live']} live), E={cfg.E}, K={cfg.K}, N={cfg.N}, top-{cfg.topk}, "
                f"{fmt}, {'deterministic' if deterministic else 'atomic'} combine")
    log(f"{workload}: median {med:.1f} us per layer (p10 {p10:.1f}, p90 {p90:.1f}); stages " +
        ", ".join(f"{k} {v:.1f}" for k, v in stage_us.items()))
    return {
        "workload": workload, "deterministic": bool(deterministic), "tokens": cfg.T, "live_tokens": alg["live"],
        "experts": cfg.E, "hidden": cfg.K, "intermediate": cfg.N, "top_k": cfg.topk,
        "distinct_experts": alg["distinct"], "layer_copies_cycled": len(rt), "launch": "hipGraph replay",
        "sequence": sequence, "samples": samples, "steps_per_sample": args.steps,
        "us_per_layer": round(med, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2),
        "tokens_per_s": round(alg["live"] / (med * 1e-6), 1),
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "layer_hbm_frac": round(alg["layer_bytes"] / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(alg["layer_flops"] / (med * 1e-6) / 1e12 / mfma_peak, 4),
        "roofline": {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic},
        "dtype": "mxfp4*mxfp8->f32" if a8 else (
            "f16(dequant nvfp4/nf3)*f16(bf16 rows scaled by 2^-e)->f32" if sequence == "decode" else
            "bf16(dequant nvfp4/nf3)*bf16->f32 (NVFP4 route-buffer down GEMM in f16)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="layers per timed sample (one graph replay)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--samples", type=int, default=30, help="timed graph replays of the headline workload "
                    "(a third as many, at least 10, for batches above 64 tokens)")
    ap.add_argument("--config", default="decode", choices=sorted(I.CONFIGS))
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--secondary", default="prefill:det,prefill:atomic,nvfp4_decode:atomic,nvfp4_prefill:det,"
                    "hybrid:det", help="further workloads NAME:det|atomic measured the same way ('' = none)")
    ap.add_argument("--layers", type=int, default=8, help="independent weight copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle budget (0 = skip)")
    ap.add_argument("--cpu-rows", type=int, default=16, help="token rows in the CPU oracle sample")
    ap.add_argument("--timing-runs", type=int, default=200, help="runs with per-stage HIP events")
    ap.add_argument("--tune", default="", metavar="T1,T2,...",
                    help="race the launch sequences at the capacity of each batch size (moe_plan_autotune) on "
                         "the workload's geometry and print the times instead of the benchmark line")
    ap.add_argument("--tune-reps", type=int, default=10, help="timed runs per sequence in --tune")
    ap.add_argument("--tune-file", default="", help="with --tune: save the pinned rungs to this file")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference kernel that "
                         "scales HBM byte counters)")
    ap.add_argument("--pmc-csv", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only summarise rocprofv3 counter_collection.csv files of one kernel (with --pmc-kernel)"
                         " into HBM bytes per launch, calibrated by the copy runs")
    ap.add_argument("--pmc-kernel", default="k_dec_gemm1_a8", help="kernel name (substring) for --pmc-csv")
    ap.add_argument("--copy-calib-bytes", type=int, default=1 << 30, help="bytes of the calibration copy")
    args = ap.parse_args()
    if args.pmc_csv:
        print(json.dumps(pmc_summary(args), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the layer shards by "
              "tensor-parallel N-slices plus one all-reduce, which is not built here).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.samples < 1:
        raise SystemExit("--steps and --samples must be positive")

    import torch
    import block_scaled_fp4_histogram_amd as M

    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    tiers_cache = {}
    log(f"config {args.config}: generating inputs")
    prob = problem(args.config, tiers_cache)
    cfg = prob.cfg
    a8 = prob.tiers[0].fmt == I.FMT_MXFP4

    if args.tune:
        toks = [int(v) for v in args.tune.split(",")]
        plan = M.Plan(cfg.E, cfg.K, cfg.N, cfg.topk, cfg.limit, M.A_MXFP8 if a8 else M.A_BF16,
                      max_tokens=max([cfg.T] + toks))
        copies = LayerCopies(M, prob, plan, args.layers, dev)
        us = plan.autotune(copies.run_tiers[0], toks, args.deterministic, reps=args.tune_reps)
        names = [s if c is None else f"{s}/{c}" for s, c in M.RACE_SLOTS]
        seqs = ("decode", "general", "prefill", "prefill_narrow")
        combs = {M.COMBINE_ATOMIC: "atomic", M.COMBINE_ROUTE_BUFFER: "route_buffer"}
        rows = [{"tokens": t, "capacity": plan.capacity(t)[0],
                 "us": {n: (None if math.isnan(v) else round(v, 2)) for n, v in zip(names, u)},
                 "pinned": seqs[plan.sequence(t) - 1],
                 "combine": combs.get(plan.combine(t))} for t, u in zip(toks, us)]
        # the same race at the workload's own batch (its routing, e.g. Zipf-skewed loads)
        x = torch.from_numpy(prob.x).to(dev).view(torch.bfloat16)
        own = plan.autotune_batch(copies.run_tiers[0], x, torch.from_numpy(prob.ids).to(dev),
                                  torch.from_numpy(prob.wts).to(dev), args.deterministic, reps=args.tune_reps)
        own_row = {"tokens": cfg.T, "capacity": plan.capacity(cfg.T)[0],
                   "us": {n: (None if math.isnan(v) else round(v, 2)) for n, v in zip(names, own)},
                   "pinned": seqs[plan.sequence(cfg.T) - 1], "combine": combs.get(plan.combine(cfg.T))}
        if args.tune_file:
            plan.save_tuning(args.tune_file)
        print(json.dumps({"workload": cfg.name, "deterministic": args.deterministic, "layer_copies": args.layers,
                          "tuning": rows, "own_batch": own_row}), flush=True)
        return

    # the copies are prepared under a plan of the same geometry; experts run under any
    # plan whose K, N and w13 layout match
    prep_plan = M.Plan(cfg.E, cfg.K, cfg.N, cfg.topk, cfg.limit, M.A_MXFP8 if a8 else M.A_BF16, max_tokens=cfg.T)
    copies = LayerCopies(M, prob, prep_plan, args.layers, dev)
    head = measure(M, prob, copies, args.deterministic, args, dev)
    alg = algorithmic(prob)

    cpu = None
    if args.cpu_seconds > 0:
        valid_rows = np.flatnonzero(((prob.ids >= 0) & (prob.ids < cfg.E)).any(axis=1))
        rng = np.random.default_rng(0)
        rows = valid_rows if len(valid_rows) <= args.cpu_rows else np.sort(rng.choice(valid_rows, args.cpu_rows,
                                                                                      replace=False))
        log(f"cpu oracle on {len(rows)} rows, budget {args.cpu_seconds}s")
        tps, cores, reps, el = cpu_baseline(prob, args.cpu_seconds, rows.astype(np.int32))
        cpu = {"value": round(tps, 3), "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": f"{len(rows)} live token rows of the {cfg.name} batch x {reps} repetitions "
                         f"({el:.1f} s, float64 CPU oracle, OpenMP over rows)"}

    secondary = []
    for item in [v for v in args.secondary.split(",") if v]:
        name, _, mode = item.partition(":")
        if name not in I.CONFIGS or mode not in ("det", "atomic", ""):
            raise SystemExit(f"--secondary: bad entry {item!r}")
        p2 = problem(name, tiers_cache)
        if weight_key(p2.cfg) != copies.key:
            del copies
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            c2 = p2.cfg
            prep_plan = M.Plan(c2.E, c2.K, c2.N, c2.topk, c2.limit,
                               M.A_MXFP8 if p2.tiers[0].fmt == I.FMT_MXFP4 else M.A_BF16, max_tokens=c2.T)
            copies = LayerCopies(M, p2, prep_plan, args.layers, dev)
        secondary.append(measure(M, p2, copies, mode == "det", args, dev))

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_layer"] / 1000.0, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {k: v for k, v in head.items() if k not in ("roofline", "dtype", "tokens_per_s")},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    line["config"]["workload"] = head["workload"]
    line["config"]["ms_per_step_p10_p90"] = [round(head["us_p10"] / 1000.0, 5), round(head["us_p90"] / 1000.0, 5)]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
