#!/usr/bin/env python3
"""MoE layer forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mixtral_bf16]
                    [--gating topk_softmax|softmax_topk|softmax_topk_scaled]
                    [--fill token|priority]

One step is one moe_forward call (router, permutation, both grouped GEMMs,
combine) over one batch of T tokens already resident in HBM. The headline
value is T / (wall time per step), timed over exactly K steps bracketed by
torch.cuda.synchronize(). A second pass runs the same kernels stage by stage
(moe_route, moe_permute, moe_expert_gate_up, moe_expert_down,
moe_unpermute_combine) with HIP events between the launches on the launch
stream, and a 512 MiB buffer read before each step so the HBM-bound stages
do not read from cache (a read leaves no dirty lines to be written back
during the timed kernels); it gives each stage's duration and the roofline
figures. The CPU oracle is timed on a bounded sample of the same workload.
--gating / --fill select a gate rule and a capacity fill order (Batch
Priority Routing); the step is then moe_forward_ex, and the permute stage
includes the priority sort. --routing expert_choice times
moe_forward_expert_choice instead (each expert takes C = capacity tokens);
its stages are route (scores and selection), gather, ffn and combine.
--pass backward times moe_backward (gradients of <dy, y> for x and all
weights, with the forward recomputed inside) instead of the forward, or
moe_backward_expert_choice with --routing expert_choice.
Two reference modes print their own JSON line instead: --library-gemm times the
vendor GEMM library on dense GEMMs of the workload's FFN shapes, --copy-probe
runs plain device copies (the calibration of the HBM byte counters).
Prints one JSON line on stdout (progress goes to stderr).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + % bf16 MFMA peak (grouped FFN), Mixtral-shape, 1 GPU"
PEAK = {"bf16_tflops": 2500.0, "f32_tflops": 157.3, "hbm_gbs": 8000.0}
# The gate/up kernel's source: its file and the headers it includes (a change to any of them can
# change the kernel, and counters taken before it no longer describe it).
DOMINANT_KERNEL_SRC = [os.path.join(ROOT, "sparse_mixture_experts_09_amd", "csrc", n)
                       for n in ("ffn_bf16.hip", "ffn_sched.h", "moe_common.h", "moe_kernels.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(paths):
    """SHA-256 over the files in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from rocprofv3 counters, if
    they were taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_digest(DOMINANT_KERNEL_SRC):
        return None
    return t.get("bytes_per_launch")


def clock_during(moe, run, steps, ms_per_step):
    """The core (shader) clock while `run()` executes `steps` times: clock
    probes (one wavefront each, waiting 1 ms of the device's constant-rate
    wall clock and counting core cycles meanwhile) run back to back on a
    second stream beside the loop, for about 80% of its length so that every
    probe overlaps it. Returns MHz statistics over the probes."""
    import torch
    khz = moe.moe_wall_clock_khz()
    n = max(1, int(0.8 * steps * ms_per_step))
    out = torch.zeros((n, 2), dtype=torch.int64, device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()   # default priority, like every stream here
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    for i in range(n):
        moe.moe_clock_probe(out[i], khz, stream=side)
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    cyc = out[:, 0].double()
    wall = out[:, 1].double()
    mhz = (cyc / wall * khz / 1e3).cpu().tolist()
    return {"mean_mhz": float(cyc.sum() / wall.sum() * khz / 1e3), "min_mhz": min(mhz), "max_mhz": max(mhz),
            "probes": n, "wall_clock_khz": khz,
            "source": "core-cycle counter over 1 ms wall-clock windows, probes on a second stream beside "
                      f"{steps} more moe_forward steps"}


def blas_threads():
    """Threads of the BLAS library numpy calls (the oracle's matmuls run there)."""
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])


def cpu_baseline(w, a, target_s, gating="topk_softmax", bpr=False):
    """The oracle, as it is, on the first S tokens of the workload."""
    from oracle import moe_oracle as orc

    def run(S):
        t = time.perf_counter()
        orc.forward(a["x"][:S], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                    gating=gating, bpr=bpr)
        return time.perf_counter() - t

    # grow the sample (x4) until it takes about target_s or covers the whole batch;
    # each run includes the oracle's fixed cost of widening the weights to float64
    S = min(w.T, 128)
    t = run(S)
    log(f"cpu oracle: {S} tokens in {t:.2f} s")
    while S < w.T and t < target_s / 2:
        S = min(w.T, 4 * S)
        t = run(S)
        log(f"cpu oracle: {S} tokens in {t:.2f} s")
    threads = blas_threads()
    drop = "dropless, so routing and outputs equal the full layer's for these tokens" if w.cf == 0 else \
        f"capacity recomputed for {S} tokens"
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {w.T} tokens of {w.name} ({drop}); whole layer forward in float64 "
                      f"numpy (BLAS matmul), {t:.1f} s"}


def cpu_baseline_backward(w, a, target_s, ec, gating="topk_softmax", bpr=False):
    """The oracle's backward pass, as it is, on the first S tokens of the workload (routing and
    capacity recomputed for them), gradients of <dy, y> for x and every weight."""
    import numpy as np

    from oracle import moe_oracle as orc

    def run(S):
        dy = np.random.default_rng(0).standard_normal((S, w.d))
        t = time.perf_counter()
        if ec:
            orc.expert_choice_backward(a["x"][:S], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], dy, w.k,
                                       w.cf, w.dtype)
        else:
            orc.backward(a["x"][:S], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], dy, w.k, w.cf, w.dtype,
                         gating=gating, bpr=bpr)
        return time.perf_counter() - t

    # grow the sample (x4) until it takes about target_s or covers the whole batch; each run
    # includes the oracle's fixed cost of widening the weights and their gradients to float64
    S = min(w.T, 64)
    t = run(S)
    log(f"cpu oracle backward: {S} tokens in {t:.2f} s")
    while S < w.T and t < target_s / 2:
        S = min(w.T, 4 * S)
        t = run(S)
        log(f"cpu oracle backward: {S} tokens in {t:.2f} s")
    rule = "expert choice" if ec else f"{gating}, {'priority' if bpr else 'token'} fill"
    return {"value": S / t, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"backward ({rule}) on the first {S} of {w.T} tokens of {w.name}, routing and capacity "
                      f"recomputed for them; float64 numpy (BLAS matmul), {t:.1f} s"}


def library_gemm(args, w, mi, torch):
    """torch.matmul on the dense shapes of the layer's two GEMMs: the T k token rows (x repeated k
    times) against one expert's [W_gate; W_up], and h = SiLU(x W_gate^T) * (x W_up^T) of those rows
    against its W_down, both with the weight as stored (K-major rows, as the grouped kernels read
    it). The same flops as the grouped GEMMs of a dropless batch, with no routing: a reference
    for what the vendor library reaches on these shapes, not part of the hot path."""
    a = mi.generate(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = a["x"].to("cuda")
    wg, wu, wd = (a[n][0].to("cuda") for n in ("w_gate", "w_up", "w_down"))
    a1 = x.repeat(w.k, 1).contiguous()
    b1 = torch.cat([wg, wu]).contiguous()
    h = (torch.nn.functional.silu((a1 @ wg.t()).float()) * (a1 @ wu.t()).float()).to(dt)
    out = {}
    for name, lhs, rhs in (("gate_up", a1, b1), ("down", h, wd)):
        for _ in range(args.warmup):
            torch.matmul(lhs, rhs.t())
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(args.steps):
            torch.matmul(lhs, rhs.t())
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / args.steps * 1e3
        flops = 2.0 * lhs.shape[0] * lhs.shape[1] * rhs.shape[0]
        out[name] = {"m": lhs.shape[0], "n": rhs.shape[0], "k": lhs.shape[1], "us": round(us, 1),
                     "tflops": round(flops / us / 1e6, 1)}
    return {"library_gemm": out, "workload": w.name, "dtype": w.dtype, "steps": args.steps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--gating", default="topk_softmax", choices=["topk_softmax", "softmax_topk", "softmax_topk_scaled"])
    ap.add_argument("--fill", default="token", choices=["token", "priority"])
    ap.add_argument("--routing", default="token_choice", choices=["token_choice", "expert_choice"])
    ap.add_argument("--pass", dest="which", default="forward", choices=["forward", "backward"])
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run K device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time torch.matmul (the vendor GEMM library) on dense GEMMs of the workload's FFN "
                         "shapes (T k rows, one expert's weights), as a reference for the grouped kernels")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (sharding over GPUs is "
              "a design note, not code). Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": args.steps}), flush=True)
        return

    import moe_inputs as mi
    if args.library_gemm:
        print(json.dumps(library_gemm(args, mi.WORKLOADS[args.workload], mi, torch)), flush=True)
        return
    from sparse_mixture_experts_09_amd import moe

    if not os.path.exists(moe.LIB_PATH):
        from sparse_mixture_experts_09_amd.build import build
        build()
    w = mi.WORKLOADS[args.workload]
    T, d, E, k, F, cf = w.T, w.d, w.E, w.k, w.F, w.cf
    s = 2 if w.dtype == "bf16" else 4
    K, W = args.steps, args.warmup
    log(f"generating {w.name} ...")
    a = mi.generate(w)
    g = {n: v.cuda() for n, v in a.items() if v is not None and n != "token_ids"}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.which == "backward":
        print(json.dumps(bench_backward(args, w, a, g, moe, stream)), flush=True)
        return
    if args.routing == "expert_choice":
        print(json.dumps(bench_expert_choice(args, w, a, g, moe, stream)), flush=True)
        return

    # ---- headline: K x moe_forward ----
    y = torch.empty_like(g["x"])
    ws = torch.empty(moe.moe_workspace_bytes(T, d, E, k, cf, F, g["x"].dtype), dtype=torch.uint8, device="cuda")

    gating, fill = args.gating, args.fill
    bpr = fill == "priority"

    def forward():
        moe.moe_forward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], k, cf, y=y, ws=ws,
                        gating=gating, fill_order=fill)

    for _ in range(W):
        forward()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        forward()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    gpu_ms_step = e0.elapsed_time(e1) / K
    log(f"moe_forward: {ms_step:.3f} ms/step wall, {gpu_ms_step:.3f} ms/step events")
    # the same step captured once in a HIP graph and replayed K times (launch gaps removed); the
    # replay must reproduce the eager output bit for bit
    graph = None
    try:
        y_eager = y.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            forward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_):
            forward()
        torch.cuda.synchronize()
        y.zero_()
        g_.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(y, y_eager))
        t0 = time.perf_counter()
        for _ in range(K):
            g_.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / K
        graph = {"ms_per_step": g_ms, "tokens_per_s": T / (g_ms * 1e-3), "equals_eager": same}
        log(f"moe_forward as a replayed HIP graph: {g_ms:.3f} ms/step (output equal to eager: {same})")
        del g_
    except Exception as exc:   # capture unsupported here: report, keep the eager figures
        graph = {"error": repr(exc)[:200]}
    # the core clock during the same loop, measured in K more steps (outside the timed region)
    clock = clock_during(moe, forward, K, ms_step)
    log(f"core clock during moe_forward: mean {clock['mean_mhz']:.0f} MHz (min {clock['min_mhz']:.0f}, "
        f"max {clock['max_mhz']:.0f}, {clock['probes']} probes)")

    # ---- stage pass: same kernels, events between launches ----
    R_max = moe.moe_rows_max(T, E, k, cf)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    perm = {"expert_counts": torch.empty(E, dtype=torch.int32, device="cuda"),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device="cuda"),
            "slot_row": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "row_slot": torch.empty(R_max, dtype=torch.int32, device="cuda"),
            "x_perm": torch.empty((R_max, d), dtype=g["x"].dtype, device="cuda"),
            "ws": torch.empty(max(moe.moe_permute_priority_workspace_bytes(T, E) if bpr else
                                  moe.moe_permute_workspace_bytes(T, E), 16), dtype=torch.uint8, device="cuda")}
    h = torch.empty((R_max, F), dtype=g["x"].dtype, device="cuda")
    o = torch.empty((R_max, d), dtype=g["x"].dtype, device="cuda")
    y2 = torch.empty_like(g["x"])
    flush = None if args.no_flush else torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    names = ["route", "permute", "gate_up", "down", "combine"]
    samples = {n: [] for n in names}
    for it in range(W + K):
        if flush is not None:
            flush.sum()   # reads 512 MiB: evicts the caches without leaving dirty lines
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(stream)
        moe.moe_route(g["x"], g["w_router"], k, topk_idx=idx, topk_gate=gate, stream=stream, gating=gating)
        ev[1].record(stream)
        moe.moe_permute(g["x"], idx, E, cf, out=perm, stream=stream, score=gate if bpr else None, score_stride=k)
        ev[2].record(stream)
        moe.moe_expert_gate_up(perm["x_perm"], perm["expert_offsets"], g["w_gate"], g["w_up"], T, k, cf, h=h,
                               stream=stream)
        ev[3].record(stream)
        moe.moe_expert_down(h, perm["expert_offsets"], g["w_down"], T, k, cf, out_perm=o, stream=stream)
        ev[4].record(stream)
        moe.moe_unpermute_combine(o, perm["slot_row"], gate, E, cf, y=y2, stream=stream)
        ev[5].record(stream)
        if it >= W:
            samples["_ev"] = samples.get("_ev", []) + [ev]
    torch.cuda.synchronize()
    for ev in samples.pop("_ev"):
        for i, n in enumerate(names):
            samples[n].append(ev[i].elapsed_time(ev[i + 1]))
    st_ms = {n: float(np.mean(v)) for n, v in samples.items()}
    same_as_forward = bool(torch.equal(y, y2))

    offsets = perm["expert_offsets"].cpu().numpy().astype(np.int64)
    slot_row = perm["slot_row"].cpu().numpy()
    kept = np.diff(offsets)
    R = int(offsets[-1])
    active = int((kept > 0).sum())
    T_read = int((slot_row >= 0).any(axis=1).sum())
    alg = {
        "route": dict(bytes=T * d * s + E * d * s + T * k * 8, flops=2 * T * d * E),
        "permute": dict(bytes=T_read * d * s + R * d * s + 4 * (2 * T * k + R + 2 * E), flops=0),
        "gate_up": dict(bytes=active * 2 * F * d * s + R * d * s + R * F * s, flops=4 * d * F * R),
        "down": dict(bytes=active * d * F * s + R * F * s + R * d * s, flops=2 * d * F * R),
        "combine": dict(bytes=R * d * s + T * k * 8 + T * d * s, flops=2 * R * d),
    }
    peak_mm = PEAK["bf16_tflops"] if w.dtype == "bf16" else PEAK["f32_tflops"]
    stages = {}
    for n in names:
        t = st_ms[n] * 1e-3
        stages[n] = {"us": st_ms[n] * 1e3, "GB/s": alg[n]["bytes"] / t / 1e9,
                     "TFLOP/s": alg[n]["flops"] / t / 1e12,
                     "hbm_frac": alg[n]["bytes"] / t / 1e9 / PEAK["hbm_gbs"]}
        log(f"  {n:8s} {st_ms[n] * 1e3:9.1f} us  {stages[n]['GB/s']:8.0f} GB/s  {stages[n]['TFLOP/s']:8.1f} TFLOP/s")
    # ---- what a plain memory-bound torch kernel reaches on the same byte counts, timed the same
    # way (flushed caches, events around one launch): a device copy moving each stage's algorithmic
    # bytes, half read and half written. It shows what a kernel of that size reaches here, launch
    # included.
    half = {n: alg[n]["bytes"] // 2 for n in ("route", "permute", "combine")}
    ref_src = torch.empty(max(half.values()) + 64, dtype=torch.uint8, device="cuda")
    ref_dst = torch.empty_like(ref_src)
    ref_ops = {n: (2 * half[n], (lambda m: lambda: ref_dst[:m].copy_(ref_src[:m]))(half[n])) for n in half}
    ref_samples = {n: [] for n in ref_ops}
    for it in range(W + K):
        for n, (_, op) in ref_ops.items():
            if flush is not None:
                flush.sum()
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e_a.record(stream)
            op()
            e_b.record(stream)
            if it >= W:
                ref_samples[n].append((e_a, e_b))
    torch.cuda.synchronize()
    hbm_ref = {}
    for n, (nbytes, _) in ref_ops.items():
        if ref_samples[n]:
            us = float(np.mean([a_.elapsed_time(b_) for a_, b_ in ref_samples[n]])) * 1e3
            hbm_ref[n] = {"us": us, "bytes": nbytes, "GB/s": nbytes / us / 1e3, "stage_us": st_ms[n] * 1e3}
    del ref_src, ref_dst
    if hbm_ref:
        log("  plain torch kernels on the same bytes: " + ", ".join(
            f"{n} {v['us']:.1f} us ({v['GB/s']:.0f} GB/s)" for n, v in hbm_ref.items()))
    ffn_t = (st_ms["gate_up"] + st_ms["down"]) * 1e-3
    ffn_frac = (alg["gate_up"]["flops"] + alg["down"]["flops"]) / ffn_t / 1e12 / peak_mm
    hbm_t = (st_ms["route"] + st_ms["permute"] + st_ms["combine"]) * 1e-3
    hbm_frac = (alg["route"]["bytes"] + alg["permute"]["bytes"] + alg["combine"]["bytes"]) / hbm_t / 1e9 / PEAK["hbm_gbs"]
    gu_t = st_ms["gate_up"] * 1e-3
    if w.dtype == "bf16" and min(moe.moe_capacity(T, E, k, cf), R_max) <= 64:
        # at most 64 rows per expert: the weight-streaming kernel, bound by HBM
        achieved = alg["gate_up"]["bytes"] / gu_t / 1e9
        roofline = {"bound": "hbm", "kernel": "ffn_bf16_skinny_kernel<true,1,3,2> (gate/up weight stream + SwiGLU)",
                    "achieved": achieved, "peak": PEAK["hbm_gbs"], "unit": "GB/s",
                    "frac": achieved / PEAK["hbm_gbs"], "traffic": load_traffic(w.name),
                    "alg_bytes_per_launch": alg["gate_up"]["bytes"], "avg_launch_us": st_ms["gate_up"] * 1e3}
    else:
        achieved = alg["gate_up"]["flops"] / gu_t / 1e12
        roofline = {"bound": "mfma", "kernel": "ffn_bf16_w4_kernel<128,true,false> (grouped gate/up GEMM + SwiGLU epilogue)",
                    "achieved": achieved, "peak": peak_mm, "unit": "TFLOP/s", "frac": achieved / peak_mm,
                    "traffic": load_traffic(w.name), "alg_flops_per_launch": alg["gate_up"]["flops"],
                    "avg_launch_us": st_ms["gate_up"] * 1e3}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w, a, args.cpu_seconds, gating, bpr)

    out = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d": d, "E": E, "k": k, "F": F, "cf": cf, "kept_rows": R,
                   "gating": gating, "fill": fill, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ffn_mfma_frac": ffn_frac,
        "route_permute_combine_hbm_frac": hbm_frac,
        "hbm_stage_reference": {
            "method": "torch device copy of each stage's algorithmic bytes (half read, half written), flushed "
                      "caches, events around one launch, as the stages",
            "stages": hbm_ref,
            "hbm_frac": (sum(v["bytes"] for v in hbm_ref.values()) / (sum(v["us"] for v in hbm_ref.values()) * 1e-6)
                         / 1e9 / PEAK["hbm_gbs"]) if hbm_ref else None},
        "layer_tflops": (alg["route"]["flops"] + alg["gate_up"]["flops"] + alg["down"]["flops"]) / (ms_step * 1e-3) / 1e12,
        "gpu_ms_per_step_events": gpu_ms_step,
        "graph_replay": graph,
        "core_clock": clock,
        "stages": stages,
        "stage_path_equals_forward": same_as_forward,
    }
    print(json.dumps(out), flush=True)


def bench_backward(args, w, a, g, moe, stream):
    """Backward pass: K timed moe_backward (or, with --routing expert_choice,
    moe_backward_expert_choice) steps, the forward recomputed inside."""
    import numpy as np
    import torch

    T, d, E, k, F, cf = w.T, w.d, w.E, w.k, w.F, w.cf
    K, W = args.steps, args.warmup
    dy = torch.from_numpy(np.random.default_rng(0).standard_normal((T, d)).astype(np.float32)).to(g["x"].dtype).cuda()
    ec = args.routing == "expert_choice"
    gating, fill = args.gating, args.fill
    if ec:
        n = moe._size_query("moe_backward_expert_choice_workspace_bytes", T, d, E, k, cf, F, moe._dt(g["x"]))
    else:
        n = moe._size_query("moe_backward_workspace_bytes", T, d, E, k, cf, F, moe._dt(g["x"]))
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")

    def step():
        if ec:
            moe.moe_backward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], dy, k, cf,
                                           ws=ws)
        else:
            moe.moe_backward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], dy, k, cf, ws=ws,
                             gating=gating, fill_order=fill)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    if ec:
        R = E * moe.moe_capacity(T, E, k, cf)
    else:
        idx, gate, _ = moe.moe_route(g["x"], g["w_router"], k, gating=gating)
        perm = moe.moe_permute(g["x"], idx, E, cf, score=gate if fill == "priority" else None, score_stride=k)
        R = int(perm["expert_offsets"][-1].item())
    flops = 18 * d * F * R + 4 * T * d * E
    peak = PEAK["bf16_tflops"]
    achieved = flops / (ms_step * 1e-3) / 1e12
    name = "moe_backward_expert_choice" if ec else "moe_backward"
    log(f"{name}: {ms_step:.3f} ms/step, {achieved:.0f} TFLOP/s over the layer ({R} rows), workspace {n / 2**30:.2f} GiB")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle's backward ...")
        cpu = cpu_baseline_backward(w, a, args.cpu_seconds, ec, gating, fill == "priority")
    return {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "T": T, "d": d, "E": E, "k": k, "F": F, "cf": cf,
                   "routing": args.routing, "gating": None if ec else gating, "fill": None if ec else fill,
                   "kept_rows": R, "workspace_bytes": n,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "whole backward (recompute + data and weight gradient GEMMs)",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "alg_flops_per_launch": flops, "avg_launch_us": ms_step * 1e3},
        "cpu_baseline": cpu,
    }


def bench_expert_choice(args, w, a, g, moe, stream):
    """Expert-choice layer: K timed moe_forward_expert_choice steps, then a stage pass."""
    import numpy as np
    import torch

    T, d, E, k, F, cf = w.T, w.d, w.E, w.k, w.F, w.cf
    s = 2 if w.dtype == "bf16" else 4
    K, W = args.steps, args.warmup
    C = moe.moe_capacity(T, E, k, cf)
    R = E * C
    y = torch.empty_like(g["x"])
    ws = torch.empty(max(moe._size_query("moe_forward_expert_choice_workspace_bytes", T, d, E, k, cf, F,
                                             moe._dt(g["x"])), 16), dtype=torch.uint8, device="cuda")

    def forward():
        moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], k, cf, y=y, ws=ws)

    for _ in range(W):
        forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        forward()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    log(f"moe_forward_expert_choice: {ms_step:.3f} ms/step (C = {C}, {R} rows)")

    names = ["route", "gather", "ffn", "combine"]
    flush = None if args.no_flush else torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    samples = {n: [] for n in names}
    evs = []
    y2 = torch.empty_like(g["x"])
    for it in range(W + K):
        if flush is not None:
            flush.sum()   # reads 512 MiB: evicts the caches without leaving dirty lines
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        r = moe.moe_route_expert_choice(g["x"], g["w_router"], k, cf, stream=stream)
        ev[1].record(stream)
        xp = moe.moe_gather_rows(g["x"], r["expert_tokens"], R, stream=stream)
        ev[2].record(stream)
        _, o = moe.moe_grouped_ffn_rows(xp, r["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"], R, stream=stream)
        ev[3].record(stream)
        moe.moe_combine_expert_choice(o, r["slot"], r["scores"], k, cf, y=y2, stream=stream)
        ev[4].record(stream)
        if it >= W:
            evs.append(ev)
    torch.cuda.synchronize()
    for ev in evs:
        for i, n in enumerate(names):
            samples[n].append(ev[i].elapsed_time(ev[i + 1]))
    st_ms = {n: float(np.mean(v)) for n, v in samples.items()}
    active = E
    alg = {
        "route": dict(bytes=T * d * s + E * d * s + T * E * 4 * 3 + R * 4 + T * E * 4, flops=2 * T * d * E),
        "gather": dict(bytes=2 * R * d * s + R * 4, flops=0),
        "ffn": dict(bytes=active * 3 * F * d * s + 2 * R * d * s + 2 * R * F * s, flops=6 * d * F * R),
        "combine": dict(bytes=R * d * s + T * E * 8 + T * d * s, flops=2 * R * d),
    }
    stages = {}
    for n in names:
        t = st_ms[n] * 1e-3
        stages[n] = {"us": st_ms[n] * 1e3, "GB/s": alg[n]["bytes"] / t / 1e9, "TFLOP/s": alg[n]["flops"] / t / 1e12,
                     "hbm_frac": alg[n]["bytes"] / t / 1e9 / PEAK["hbm_gbs"]}
        log(f"  {n:8s} {st_ms[n] * 1e3:9.1f} us  {stages[n]['GB/s']:8.0f} GB/s  {stages[n]['TFLOP/s']:8.1f} TFLOP/s")
    peak_mm = PEAK["bf16_tflops"] if w.dtype == "bf16" else PEAK["f32_tflops"]
    achieved = alg["ffn"]["flops"] / (st_ms["ffn"] * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        from oracle import moe_oracle as orc
        t0 = time.perf_counter()
        S = min(T, 1024)
        orc.expert_choice_forward(a["x"][:S], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], k, cf, w.dtype)
        t = time.perf_counter() - t0
        cpu = {"value": S / t, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"expert-choice layer on the first {S} of {T} tokens (selection recomputed for them), {t:.1f} s"}
    return {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "routing": "expert_choice", "T": T, "d": d, "E": E, "k": k, "F": F, "cf": cf,
                   "tokens_per_expert": C, "rows": R, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "grouped SwiGLU FFN over the selected rows (both GEMMs)",
                     "achieved": achieved, "peak": peak_mm, "unit": "TFLOP/s", "frac": achieved / peak_mm,
                     "traffic": None, "alg_flops_per_launch": alg["ffn"]["flops"], "avg_launch_us": st_ms["ffn"] * 1e3},
        "cpu_baseline": cpu,
        "stages": stages,
        "stage_path_equals_forward": bool(torch.equal(y, y2)),
    }


if __name__ == "__main__":
    main()
