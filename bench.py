#!/usr/bin/env python3
"""MoE-LoRA expert layer benchmark on one MI355X.

One step = moe_route + moe_lora_forward (training, saving what the backward needs) +
moe_lora_backward on one batch of seeded synthetic input already resident in HBM. Prints one JSON
line: tokens/s of the whole step (value), TFLOP/s of the algorithmic work, the roofline of the
dominant kernel (from per-stage HIP events recorded on the launch stream during a second timed
pass), and the CPU oracle's rate on a bounded token sample of the same layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), Qwen3-30B-A3B shape"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
GEMM_STAGES = ("fwd_gate_up", "fwd_down", "bwd_down", "bwd_gate_up")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_work(stage, cfg, cnt, b):
    """Algorithmic FLOPs and unique HBM bytes of one step's worth of a stage (a launch, or the few
    small launches a stage groups). Bytes count each tensor the stage must read or write once: the
    activations (gathered rows count their source matrix once), the weights of the experts that
    received pairs, and the stage's outputs; recomputation, padding rows and re-reads do not count."""
    s, P, m, n, r, E, k = cfg.s, cfg.s * cfg.k, cfg.m, cfg.n, cfg.r, cfg.E, cfg.k
    u = int((cnt > 0).sum())   # experts whose weights are read
    nb = (s + 255) // 256
    if stage == "fwd_gate_up":
        fl = 2 * P * m * 2 * n + 2 * P * r * 2 * n
        by = (s * m + u * m * 2 * n + P * 2 * r + 2 * u * r * n + P * 2 * n + P * n) * b
    elif stage == "fwd_down":
        fl = 2 * P * n * m + 2 * P * r * m
        by = (P * n + u * n * m + P * r + u * r * m + P * m) * b
    elif stage == "bwd_down":
        fl = 2 * P * m * n + 2 * P * r * n
        by = (s * m + u * n * m + P * r + u * n * r + P * 2 * n + P * 2 * n) * b
    elif stage == "bwd_gate_up":
        fl = 2 * P * 2 * n * m + 2 * P * 2 * r * m
        by = (P * 2 * n + u * m * 2 * n + P * 2 * r + 2 * u * m * r + P * m) * b
    elif stage == "route_logits":
        fl = 2 * s * m * E
        by = (s * m + m * E) * b + s * E * 4
    elif stage == "route_topk":
        fl, by = 0, s * E * 4 + P * 12
    elif stage == "route_hist_rank":
        fl, by = 0, P * 8 + nb * E * 4
    elif stage == "route_scan":
        fl, by = 0, nb * E * 8 + (E + 1) * 4
    elif stage == "route_scatter":
        fl, by = 0, P * 8 + nb * E * 4 + P * 12
    elif stage == "fwd_lora_t_gate_up":
        fl = 2 * P * m * 2 * r
        by = (s * m + u * m * 2 * r + P * 2 * r) * b
    elif stage == "fwd_lora_t_down":
        fl = 2 * P * n * r
        by = (P * n + u * n * r + P * r) * b
    elif stage == "fwd_combine":
        fl, by = 2 * P * m, P * m * b + s * m * b + 8 * P
    elif stage == "bwd_router":   # row-weighted T_d rows, W_r^T, ds partials -> dz
        fl = 0
        by = 2 * P * r * b + 2 * m * E * b + (n // 64) * P * 4 + 12 * P
    elif stage == "bwd_lora_u_down":
        fl = 2 * P * m * r
        by = (s * m + u * r * m + 2 * P * r) * b
    elif stage == "bwd_lora_u_gate_up":
        fl = 2 * P * 2 * n * r
        by = (P * 2 * n + 2 * u * r * n + P * 2 * r) * b
    elif stage == "bwd_unpermute":
        fl, by = P * m * 3, P * m * b + s * m * b + 8 * P + u * m * b
    elif stage == "bwd_lora_grads":
        fl = 2 * P * (m * 2 * r + 2 * n * r + n * r + m * r)
        by = (2 * s * m + P * n + P * 2 * n + P * 6 * r) * b + E * (3 * m * r + 3 * r * n) * 4
    else:
        raise KeyError(stage)
    return fl, by


def roofline(fl, by, t_s):
    """The binding roof of algorithmic work fl (FLOP) and by (bytes) at the MI355X peaks, and the
    fraction of it that a measured time t_s reaches."""
    t_mfma = fl / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = by / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        return {"bound": "hbm", "achieved": round(by / t_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(by / t_s / 1e9 / PEAK_HBM_GBS, 4)}
    return {"bound": "mfma", "achieved": round(fl / t_s / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(fl / t_s / 1e12 / PEAK_BF16_TFLOPS, 4)}


def traffic_for(stage, workload):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/traffic.json), or None when
    absent or taken on a different build of the GEMM kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    src = hashlib.sha256(open(os.path.join(ROOT, "grouped_gemm_top_amd", "csrc", "gemm.hip"), "rb").read()).hexdigest()
    try:
        entries = json.load(open(path))
    except ValueError:
        return None
    for ent in entries.get("entries", []):
        if ent.get("stage") == stage and ent.get("workload") == workload and ent.get("gemm_hip_sha256") == src:
            return ent.get("bytes_per_launch")
    return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, inp, tokens, runs=3):
    """The oracle, untuned, on the first `tokens` tokens of the same layer (route, forward and
    backward timed separately), median of `runs` runs. Its matrix products run on the BLAS thread
    pool; the rest is single-threaded numpy."""
    import statistics

    import numpy as np
    import torch

    import oracle
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    S = min(tokens, cfg.s)
    f64 = lambda t: t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    X = f64(inp["X"][:S])
    dY = f64(inp["dY"][:S])
    Wr = f64(inp["W_r"])
    bias = f64(inp["router_bias"]) if inp["router_bias"] is not None else None
    W = {k: inp[k].detach().to("cpu", torch.float32).numpy() for k in
         ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")}
    phases = {"route": [], "forward": [], "backward": []}
    for _ in range(runs):
        t0 = time.perf_counter()
        z = oracle.router_logits(X, Wr, bias)
        rt = oracle.route(z, cfg.k, cfg.E, cfg.score, cfg.renormalize)
        t1 = time.perf_counter()
        _, saved = oracle.forward(X, W, rt, cfg.alpha, cfg.r)
        t2 = time.perf_counter()
        oracle.backward(dY, X, Wr, W, rt, cfg.alpha, cfg.r, cfg.score, cfg.renormalize, True, saved)
        t3 = time.perf_counter()
        phases["route"].append(t1 - t0)
        phases["forward"].append(t2 - t1)
        phases["backward"].append(t3 - t2)
    med = {k: statistics.median(v) for k, v in phases.items()}
    total = sum(med.values())
    return {"value": round(S / total, 3), "unit": "tokens/s", "cores": int(threads or nproc),
            "kind": "oracle", "nproc": nproc, "cpu_model": _cpu_model(),
            "phase_seconds": {k: round(v, 3) for k, v in med.items()},
            "sample": f"first {S} of {cfg.s} tokens of the same layer, route + forward + backward "
                      f"(fp64 numpy), median of {runs} runs ({total:.1f} s each)"}


def crossover(args, g, layer, config, make_inputs, torch, dev):
    """Forward of one layer evaluated two ways at growing token counts s (inputs resident, HIP
    events around each variant, median of 5 after 2 warm-up runs):
      split:  the library's Split-LoRA forward (X W + c (X A) B, no m x n product formed);
      merged: moe_peft_merge (W' = W + c A B for every expert, the materialised form) followed by the
              forward on W' with no LoRA work; reported with and without the merge.
    The merge is per training step, since A and B change every step."""
    import statistics
    s_list = [512, 1024, 2048, 4096, 8192, 16384, 32768]
    base = config(args.workload)
    big = config(args.workload, s=max(s_list))
    inp = make_inputs(big, seed=0, device=dev, with_grad_output=False)
    shape0 = layer.shape_of(big)
    Wm_gu, Wm_d = torch.empty_like(inp["W_gu"]), torch.empty_like(inp["W_d"])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=5, warm=2):
        for _ in range(warm):
            fn()
        out = []
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            out.append(ev0.elapsed_time(ev1))
        return statistics.median(out)

    def merge():
        g.moe_peft_merge(shape0, inp["W_gu"], inp["W_d"], inp["A_g"], inp["B_g"], inp["A_u"],
                         inp["B_u"], inp["A_d"], inp["B_d"], Wm_gu, Wm_d)

    t_merge = timed(merge)
    dm = dict(inp, W_gu=Wm_gu, W_d=Wm_d, A_g=None, B_g=None, A_u=None, B_u=None, A_d=None, B_d=None)
    b = 2 if base.dtype == "bf16" else 4
    E, m, n, k, r = base.E, base.m, base.n, base.k, base.r
    for s in s_list:
        cfg = config(args.workload, s=s)
        X = inp["X"][:s].contiguous()
        shape = layer.shape_of(cfg)
        shape_m = layer.shape_of(cfg, flags=g.MOE_FLAG_MERGED)
        rt = layer.route(shape, X, inp["W_r"], inp["router_bias"])
        Y = torch.empty_like(X)
        ws = torch.empty(max(1, g.moe_fwd_ws_bytes(shape, 0)), dtype=torch.uint8, device=dev)
        wsm = torch.empty(max(1, g.moe_fwd_ws_bytes(shape_m, 0)), dtype=torch.uint8, device=dev)
        t_split = timed(lambda: layer.forward(shape, X, rt, inp, training=False, Y=Y, ws=ws))
        t_mfwd = timed(lambda: layer.forward(shape_m, X, rt, dm, training=False, Y=Y, ws=wsm))
        print(json.dumps({
            "workload": base.name, "s": s, "split_fwd_ms": round(t_split, 4),
            "merged_fwd_ms": round(t_mfwd, 4), "merge_ms": round(t_merge, 4),
            "merged_total_ms": round(t_merge + t_mfwd, 4),
            "split_lowrank_bytes": 3 * k * s * r * b, "merged_delta_bytes": 3 * E * m * n * b,
        }), flush=True)
        del ws, wsm, Y, rt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)  # the first ~15 steps of a process run 1-2% slower
    ap.add_argument("--workload", default="qwen3_30b_a3b")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reference-gemm", action="store_true",
                    help="run every GEMM with the plain SIMT kernels (diagnostics)")
    ap.add_argument("--recompute", action="store_true",
                    help="keep no forward intermediates: the backward recomputes them")
    ap.add_argument("--shared-expert", type=int, default=0, metavar="N",
                    help="add a shared expert of intermediate size N (a dense Split-LoRA SwiGLU "
                         "expert on every token, added into Y and dX) to every step")
    ap.add_argument("--crossover", action="store_true",
                    help="only time the forward with Split LoRA against the materialised PEFT form "
                         "(merge W + cAB, then plain expert GEMMs) over a sweep of token counts, "
                         "print one JSON line per token count and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (scales "
                         "the HBM byte counters of a profiler against a known size) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB x 3")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the layer is benchmarked on a single MI355X; sharding it over several GPUs is not "
              "implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import grouped_gemm_top_amd as g
    from grouped_gemm_top_amd import accounting, layer
    from synth import config, make_inputs

    g.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.crossover:
        crossover(args, g, layer, config, make_inputs, torch, dev)
        return
    cfg = config(args.workload)
    log(f"[bench] workload {cfg.name}: s={cfg.s} m={cfg.m} n={cfg.n} E={cfg.E} k={cfg.k} r={cfg.r} "
        f"{cfg.dtype} {cfg.score}")
    inp = make_inputs(cfg, seed=0, device=dev, with_grad_output=True)
    flags = g.MOE_FLAG_REFERENCE_GEMM if args.reference_gemm else 0
    if args.recompute:
        flags |= g.MOE_FLAG_RECOMPUTE
    shape = layer.shape_of(cfg, flags=flags)
    X, Wr, bias, dY = inp["X"], inp["W_r"], inp["router_bias"], inp["dY"]
    rt = layer.alloc_route(shape, dev)
    saved = None if args.recompute else torch.empty(g.moe_fwd_saved_bytes(shape), dtype=torch.uint8,
                                                    device=dev)
    fws = (torch.empty(max(1, g.moe_fwd_ws_bytes(shape, 0)), dtype=torch.uint8, device=dev)
           if args.recompute else None)
    bws = torch.empty(g.moe_bwd_ws_bytes(shape), dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    grads = layer.alloc_grads(shape, dev)

    sh = None
    if args.shared_expert:  # one expert's weights (expert 0 of a draw with its own seed and shapes)
        sh_cfg = config(args.workload, n=args.shared_expert, E=8, k=1)
        sh_inp = make_inputs(sh_cfg, seed=1, device=dev, with_grad_output=False)
        sh_shape = layer.shape_of(sh_cfg, flags=flags)
        sh = {
            "cfg": sh_cfg, "shape": sh_shape,
            "W": {k: sh_inp[k][0].contiguous() for k in ("W_gu", "W_d", "A_g", "B_g", "A_u", "B_u", "A_d", "B_d")},
            "saved": None if args.recompute else torch.empty(max(1, g.moe_shared_saved_bytes(sh_shape)),
                                                             dtype=torch.uint8, device=dev),
            "fws": torch.empty(max(1, g.moe_shared_fwd_ws_bytes(sh_shape, not args.recompute)),
                               dtype=torch.uint8, device=dev),
            "bws": torch.empty(max(1, g.moe_shared_bwd_ws_bytes(sh_shape)), dtype=torch.uint8, device=dev),
            "grads": layer.shared_grads(sh_shape, dev),
        }
        log(f"[bench] shared expert: n={args.shared_expert}")

    def step():
        layer.route(shape, X, Wr, bias, bufs=rt)
        layer.forward(shape, X, rt, inp, training=not args.recompute, Y=Y, saved=saved, ws=fws)
        if sh:
            layer.shared_forward(sh["shape"], X, sh["W"], Y, training=not args.recompute, saved=sh["saved"],
                                 ws=sh["fws"])
        layer.backward(shape, dY, X, Wr, rt, inp, saved, dX=dX, grads=grads, ws=bws)
        if sh:
            layer.shared_backward(sh["shape"], dY, X, sh["W"], sh["saved"], dX, grads=sh["grads"], ws=sh["bws"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step")

    # per-step distribution: each step bracketed by its own events (reported beside the mean above)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    dist = {"p10": round(float(np.percentile(per, 10)), 4), "p50": round(float(np.percentile(per, 50)), 4),
            "p90": round(float(np.percentile(per, 90)), 4)}
    log(f"[bench] per-step ms: p10 {dist['p10']} p50 {dist['p50']} p90 {dist['p90']}")

    # second pass: per-stage HIP events on the launch stream
    g.moe_timing_enable(True)
    g.moe_timing_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages = g.moe_timing_read()
    g.moe_timing_enable(False)
    avg = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in stages.items()}
    per_step = {k: v[0] / args.steps for k, v in stages.items() if v[1]}
    for k, v in sorted(per_step.items(), key=lambda kv: -kv[1]):
        log(f"[bench]   {k:24s} {v * 1e3:9.1f} us/step")

    flops = accounting.gemm_flops(cfg.s, cfg.m, cfg.n, cfg.E, cfg.k, cfg.r, backward=True)
    total_flops = flops["total"]
    if sh:  # the shared expert: the expert arithmetic of the layer with one expert per token, no router
        sf = accounting.gemm_flops(cfg.s, cfg.m, args.shared_expert, 1, 1, cfg.r, backward=True)
        total_flops += sf["fwd_gemm"] + sf["bwd_gemm"]
    tflops = total_flops / (ms * 1e-3) / 1e12
    cnt = np.diff(rt["expert_off"].cpu().numpy())
    b = 2 if cfg.dtype == "bf16" else 4
    # per-stage roofline: algorithmic work of one step's worth of the stage against its measured
    # time per step; the layer against the sum of the stage roofs
    stages_roof = {}
    t_roof_sum = 0.0
    for st, t_us in per_step.items():
        try:
            fl, by = stage_work(st, cfg, cnt, b)
        except KeyError:
            continue
        t_s = t_us * 1e-3
        rf = roofline(fl, by, t_s)
        t_roof = max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
        t_roof_sum += t_roof
        stages_roof[st] = {"us": round(t_us * 1e3, 1), "gflop": round(fl / 1e9, 2), "mb": round(by / 1e6, 1),
                           "bound": rf["bound"], "frac": rf["frac"],
                           "mfma_frac": round(fl / t_s / 1e12 / PEAK_BF16_TFLOPS, 4) if fl else 0.0}
    dom = max(GEMM_STAGES, key=lambda st: per_step.get(st, 0.0))
    fl, by = stage_work(dom, cfg, cnt, b)
    t_s = avg[dom] * 1e-3
    roof = roofline(fl, by, t_s)
    roof["traffic"] = traffic_for(dom, cfg.name)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(avg[dom], 4)
    roof["mfma_frac"] = round(fl / t_s / 1e12 / PEAK_BF16_TFLOPS, 4)
    layer_roof = {"ms": round(ms, 4), "roof_ms": round(t_roof_sum * 1e3, 4),
                  "frac": round(t_roof_sum * 1e3 / ms, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_tokens} tokens ...")
        cpu = cpu_baseline(cfg, inp, args.cpu_tokens)
        log(f"[bench] CPU oracle: {cpu['value']} tokens/s on {cpu['cores']} threads "
            f"({cpu['nproc']} host cores, {cpu['cpu_model']}); phases {cpu['phase_seconds']}")

    out = {
        "metric": METRIC,
        "value": round(cfg.s / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_dist": dist,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "s": cfg.s, "m": cfg.m, "n": cfg.n, "E": cfg.E,
                   "k": cfg.k, "r": cfg.r, "alpha": cfg.alpha, "router": cfg.score,
                   "step": "route+forward+backward" + (" (backward recomputes the forward)"
                                                        if args.recompute else "")
                           + (f" + shared expert n={args.shared_expert}" if sh else ""),
                   "gemm": "reference-simt" if args.reference_gemm else "mfma"},
        "tflops": round(tflops, 2),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "stage_roofline": stages_roof,
        "layer_roofline": layer_roof,
        "cpu_baseline": cpu,
        "stage_us_per_step": {k: round(v * 1e3, 1) for k, v in per_step.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
