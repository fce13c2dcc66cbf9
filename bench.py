"""Benchmark of the fused MatMul -> slice-reduce -> epilogue block on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload gpt2_mlp]

A step is one call of the whole block (all P slice GEMMs, the fixed-order slice
reduction, bias + Philox dropout + residual) on one batch of seeded synthetic input
already resident in HBM.  Default workload: the GPT-2 8.3B MLP down-projection block,
M=8192, K=12288 split in P=16 slices, N=3072 (bf16 in, fp32 accumulate and out).

The timed plan is the autotuned one (mmar_autotune after the warm-up; --no-autotune
keeps the default persistent plan; the --only modes below always use the default plan).

One JSON line on stdout: throughput in TFLOP/s (2*M*N*K per step), the roofline of the
dominant kernel (the persistent fused tile kernel: its mean launch duration from two HIP
events around the timed launches, on the stream it runs on), the hidden fraction 1 - (T_fused - T_gemm_alone) / T_re_alone
(both on the persistent schedule),
and the oracle's CPU throughput on a bounded sample of the same workload.  Comparison
legs: the sequential schedule (same kernels, no overlap), the two-stream schedule, and
the unfused path (one kernel per operation, mask materialized); their ratios to the
fused time are the one-GPU analogues of the pages' block-level speedups.  Also timed:
the balanced schedule, the block with a bf16 output,
the producer MatMul in front of the block (H = GeLU(X0 . W1 + b1), bf16; the same flop
count), the whole MLP (producer then block), the QKV projection in front of the GPT-2
attention block (bias, no activation), and the data-parallel side (gradient
average of P = 8 replicas + Adam step over BERT-large's 335M parameters, HBM-bound),
beside PyTorch's mean + fused AdamW.  Then the other three block workloads, each with its
own tuned plan (fused time, roofline fraction, the epilogue's exposed cost and hipBLASLt's
plain GEMM of the same shape; --no-other-workloads skips them).

The default warm-up (50 steps, about 30 ms) takes the GPU past the clock transient of
its first launches; the timed steps then run at the sustained clock.

--only fused     time only the fused block (for rocprofv3 runs); --tile 256x128 / 256x192
                 runs the persistent schedule on that tile shape
--only streams   time only the two-stream schedule (for a kernel-trace timeline of its
                 chunk pipeline)
--only producer  time only the producer MatMuls (the GeLU layer of the workload's MLP and
                 the GPT-2 QKV projection), for their kernel traces
--only copy      one plain 1 GiB device copy, the calibration point for HBM counters
--only vendor    time only hipBLASLt's plain bf16 GEMM at the block's shape (torch.matmul),
                 the vendor yardstick, for its kernel trace
--only tune      autotune the four block workloads and print the plans chosen (with
                 MMAR_PLAN_CACHE set, the cache file also records each plan's margin)
--only hbm       time only the HBM-bound kernels (the reduce+epilogue over the workload's
                 P materialized partials, the epilogue alone, the reduce + Adam step), for
                 their kernel traces and byte counters
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "fused GEMM+reduce+epilogue TFLOP/s, % bf16 MFMA peak, % epilogue hidden"


def _paired(torch, fa, fb, pairs):
    """Runs fa, fb alternately (ABAB...) ``pairs`` times, each launch between HIP events on
    the current stream, so both see the same clock and cache state.  Returns the medians
    of a and b and the median and interquartile range of the per-pair differences a - b
    (ms)."""
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(pairs)]
    for e in ev:
        e[0].record(s); fa(); e[1].record(s)
        e[2].record(s); fb(); e[3].record(s)
    torch.cuda.synchronize()
    ta = sorted(e[0].elapsed_time(e[1]) for e in ev)
    tb = sorted(e[2].elapsed_time(e[3]) for e in ev)
    d = sorted(e[0].elapsed_time(e[1]) - e[2].elapsed_time(e[3]) for e in ev)
    q = lambda v, f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]
    return q(ta, 0.5), q(tb, 0.5), q(d, 0.5), q(d, 0.75) - q(d, 0.25)


def _ev_batch(torch, fn, reps, batch=10):
    """Median over ``reps`` batches of the mean per-call time (ms) of ``batch`` calls launched
    back to back between two HIP events: the host work of a call (library heuristics,
    argument checks) overlaps the GPU work of the previous ones, as in a model's forward
    pass."""
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(batch):
            fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / batch)
    times.sort()
    return times[len(times) // 2]


def _ev_batches_ab(torch, fa, fb, reps, warm, batch=10):
    """Medians (ms per call) of ``fa`` and ``fb`` timed as alternating batches of ``batch``
    back-to-back calls (A, B, A, B, ...), after ``warm`` untimed calls of each: both see the
    same clock and thermal state, and the vendor library's GEMM, whose duration settles
    only after about a hundred launches, is timed at its steady state."""
    for _ in range(warm):
        fa()
    for _ in range(warm):
        fb()
    s = torch.cuda.current_stream()
    ta, tb = [], []
    for _ in range(reps):
        for fn, out in ((fa, ta), (fb, tb)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(batch):
                fn()
            e1.record(s)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) / batch)
    ta.sort()
    tb.sort()
    return ta[len(ta) // 2], tb[len(tb) // 2]


def _ev_time(torch, fn, reps, before=None, stats=False):
    """Median and mean of per-call durations (ms), HIP events on the current stream.
    ``before`` runs (untimed) ahead of every call; ``stats`` adds min and p90."""
    s = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    med, mean = times[len(times) // 2], sum(times) / len(times)
    if stats:
        return med, mean, times[0], times[min(len(times) - 1, int(0.9 * (len(times) - 1) + 0.5))]
    return med, mean


TILE_KERNEL_SOURCES = ("tile_kernel.hip", "device_common.h", "mmar_internal.h")


def _code_only(text):
    """C++ source without its comments and blank lines (no string literal in these
    sources holds a comment marker)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.split("\n"))
    return "\n".join(ln for ln in lines if ln)


def tile_kernel_sha():
    """sha256 over the code of the sources that define the fused tile kernel, comments and
    blank lines left out (its counters are valid only for this exact code)."""
    h = hashlib.sha256()
    for name in TILE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "chunked_matmul_reduce_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def _traffic(kernel_sha):
    """HBM bytes per launch from the committed counter summary, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic_tile_kernel_fused_gpt2_mlp.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("tile_kernel_sources_sha256") != kernel_sha:
        return None
    return d.get("traffic_bytes_per_launch")


def _cpu_baseline(inp, w, budget_s):
    import contextlib
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
    rows_done, t_total = 0, 0.0
    block = 1024
    with ctx:
        while rows_done < w.M and t_total < budget_s:
            rows = np.arange(rows_done, min(w.M, rows_done + block))
            t0 = time.perf_counter()
            oracle.run_inputs(inp, rows=rows)
            t_total += time.perf_counter() - t0
            rows_done += rows.size
    flops = 2.0 * rows_done * w.N * w.K
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{rows_done - 1} of M={w.M} (all N={w.N}, K={w.K}, P={w.P}): "
                      f"{rows_done / w.M:.0%} of the workload, fp64 numpy/OpenBLAS, "
                      f"{t_total:.1f} s"}


def _other_workloads(torch, np, mmar, names, steps, warmup):
    """The other block workloads, each with its own tuned plan: the fused call's mean launch
    duration from two HIP events around ``steps`` back-to-back launches (as for the
    headline), the epilogue's exposed cost from 100 alternating fused / GEMM-alone launches
    against the epilogue alone, and hipBLASLt's plain GEMM of the same shape."""
    from workload import WORKLOADS, make_inputs
    out_all = {}
    for name in names:
        w = WORKLOADS[name]
        inp = make_inputs(w)
        d = {k: torch.from_numpy(inp[k].view(np.int16)).to("cuda").view(torch.bfloat16)
             for k in ("X", "W", "bias", "residual")}
        del inp
        X, W, bias, res = d["X"], d["W"], d["bias"], d["residual"]
        P, p, seed = w.P, w.p_drop, w.seed
        out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        T = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def fused():
            mmar.fused(X, W, bias, res, P, p, seed, out=out)
        for _ in range(warmup):
            fused()
        torch.cuda.synchronize()
        mmar.autotune(w.M, w.N, w.K, P)
        plan = mmar.get_plan(w.M, w.N, w.K, P)
        for _ in range(10):
            fused()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(steps):
            fused()
        e1.record(s)
        torch.cuda.synchronize()
        t_f = e0.elapsed_time(e1) / steps
        pers = lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "persistent", chunk=plan["chunk"]
                                     if plan["schedule"] == 3 else (0, 0), w_mode="direct",
                                     tile=plan["tile"], out=out)
        _, _, pr_d, pr_iqr = _paired(torch, pers, lambda: mmar.gemm_only(X, W, P, out=T), 100)
        mmar.gemm_only(X, W, P, out=T)
        t_epi = _ev_time(torch, lambda: mmar.reduce_epilogue_only(T[None], bias, res, p, seed,
                                                                  out=out), 20)[0]
        Cv = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        t_v, t_fb = _ev_batches_ab(torch, lambda: torch.matmul(X, W, out=Cv), fused, 10, warm=100)
        ach = w.flops / (t_f * 1e-3) / 1e12
        out_all[name] = {
            "shape": {"M": w.M, "K": w.K, "N": w.N, "P": P},
            "plan": {"schedule": {1: "sequential", 2: "streams", 3: "persistent",
                                  4: "balanced", 5: "split"}[plan["schedule"]],
                     "chunk": list(plan["chunk"]),
                     "w_mode": {0: "direct", 1: "pretranspose"}[plan["w_mode"]],
                     "tile": {0: "256x128", 1: "256x192"}[plan["tile"]]},
            "fused_us": round(t_f * 1e3, 2), "TFLOP/s": round(ach, 2),
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "paired_fused_minus_gemm_us": round(pr_d * 1e3, 2), "paired_iqr_us": round(pr_iqr * 1e3, 2),
            "epi_alone_us": round(t_epi * 1e3, 2),
            "hidden_fraction_epilogue": round(min(1.0, max(0.0, 1.0 - pr_d / t_epi)), 4),
            "vendor_gemm_bf16_us": round(t_v * 1e3, 2),
            "fused_over_vendor_time": round(t_fb / t_v, 3)}
        del d, X, W, bias, res, out, T, Cv
        torch.cuda.empty_cache()
    return out_all


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gpt2_mlp")
    ap.add_argument("--only", choices=["all", "fused", "streams", "producer", "copy", "vendor",
                                       "tune", "hbm"],
                    default="all")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the summary of the other block workloads")
    ap.add_argument("--no-autotune", action="store_true",
                    help="time the default plan instead of the autotuned one")
    ap.add_argument("--tile", choices=["auto", "256x128", "256x192"], default="auto",
                    help="with --only fused: run the persistent schedule on this tile shape")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the P ranks are folded onto one device as K-slices)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_matmul_reduce_amd as mmar
    from workload import (ADAM_WORKLOADS, WORKLOADS, make_inputs, make_producer_inputs,
                          make_qkv_inputs)

    torch.cuda.set_device(0)
    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n}))
        return

    if args.only == "tune":
        plans = {}
        for name in ("gpt2_attn", "gpt2_mlp", "bert_mlp", "gpt3_mlp"):
            wl = WORKLOADS[name]
            mmar.autotune(wl.M, wl.N, wl.K, wl.P)
            plans[name] = mmar.get_plan(wl.M, wl.N, wl.K, wl.P)
        print(json.dumps({"only": "tune", "plans": plans}), flush=True)
        return

    w = WORKLOADS[args.workload]
    if args.only == "producer":
        res = {"only": "producer", "steps": args.steps}
        for name, (mk, keys, act) in {"gelu": (make_producer_inputs(w), ("X0", "W1", "b1"), "gelu_tanh"),
                                      "qkv": (make_qkv_inputs(WORKLOADS["gpt2_attn"]),
                                              ("X0", "Wqkv", "bqkv"), "none")}.items():
            pd = [torch.from_numpy(mk[k].view(np.int16)).to("cuda").view(torch.bfloat16) for k in keys]
            H = torch.empty((pd[0].shape[0], pd[1].shape[1]), dtype=torch.bfloat16, device="cuda")
            for _ in range(args.warmup):
                mmar.linear(pd[0], pd[1], pd[2], act, out=H)
            torch.cuda.synchronize()
            med, mean = _ev_time(torch, lambda: mmar.linear(pd[0], pd[1], pd[2], act, out=H), args.steps)
            fl = 2.0 * pd[0].shape[0] * pd[0].shape[1] * pd[1].shape[1]
            res[name] = {"shape": [pd[0].shape[0], pd[0].shape[1], pd[1].shape[1]], "median_us": round(med * 1e3, 2),
                         "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 2)}
            del pd, H
            torch.cuda.empty_cache()
        print(json.dumps(res), flush=True)
        return
    inp = make_inputs(w)
    d = {k: torch.from_numpy(inp[k].view(np.int16)).to("cuda").view(torch.bfloat16)
         for k in ("X", "W", "bias", "residual")}
    X, W, bias, res = d["X"], d["W"], d["bias"], d["residual"]
    P, p, seed = w.P, float(inp["p_drop"]), w.seed
    out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

    def fused():
        mmar.fused(X, W, bias, res, P, p, seed, out=out)

    if args.only == "fused" and args.tile != "auto":
        def fused():
            mmar.fused_ex(X, W, bias, res, P, p, seed, "persistent", w_mode="direct", tile=args.tile,
                          out=out)

    if args.only == "hbm":
        # the HBM-bound kernels alone, for their kernel traces and byte counters: the
        # reduce+epilogue over the P materialized slice partials of the workload, the
        # epilogue alone over a materialized T (P = 1), and the data-parallel reduce + Adam
        # step over BERT-large's parameters
        parts = torch.empty((P, w.M, w.N), dtype=torch.float32, device="cuda")
        mmar.gemm_partials(X, W, P, out=parts)
        T = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        mmar.gemm_only(X, W, P, out=T)
        res_hbm = {"only": "hbm", "workload": w.name, "steps": args.steps}
        legs = {"reduce_epilogue": (lambda: mmar.reduce_epilogue_only(parts, bias, res, p, seed, out=out),
                                    (4 * P + 6) * w.M * w.N + 2 * w.N),
                "epilogue": (lambda: mmar.reduce_epilogue_only(T[None], bias, res, p, seed, out=out),
                             10 * w.M * w.N + 2 * w.N)}
        aw = ADAM_WORKLOADS["bert_large_adam"]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(aw.seed)
        ag = torch.randn((aw.P, aw.n), generator=gen, device="cuda").mul_(1e-2)
        ap_ = torch.randn(aw.n, generator=gen, device="cuda").mul_(0.02)
        am = torch.randn(aw.n, generator=gen, device="cuda").mul_(1e-3)
        av = am.mul(2).square()
        apb = torch.empty(aw.n, dtype=torch.bfloat16, device="cuda")
        legs["adam"] = (lambda: mmar.adam_step(ag, ap_, am, av, aw.step, aw.lr, aw.beta1, aw.beta2,
                                               aw.eps, aw.weight_decay, param_bf16=apb), aw.bytes)
        for name, (fn, nbytes) in legs.items():
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            med = _ev_time(torch, fn, args.steps)[0]
            res_hbm[name] = {"median_us": round(med * 1e3, 2), "bytes": int(nbytes),
                             "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1),
                             "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        print(json.dumps(res_hbm), flush=True)
        return

    if args.only == "vendor":
        Cv = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        for _ in range(args.warmup):
            torch.matmul(X, W, out=Cv)
        torch.cuda.synchronize()
        med = _ev_batch(torch, lambda: torch.matmul(X, W, out=Cv), max(1, args.steps // 10))
        print(json.dumps({"only": "vendor", "workload": w.name, "steps": args.steps,
                          "median_us": round(med * 1e3, 2),
                          "TFLOP/s": round(w.flops / (med * 1e-3) / 1e12, 2)}), flush=True)
        return

    if args.only == "streams":
        def streams():
            mmar.fused_ex(X, W, bias, res, P, p, seed, "streams", out=out)
        for _ in range(args.warmup):
            streams()
        torch.cuda.synchronize()
        med, mean = _ev_time(torch, streams, args.steps)
        print(json.dumps({"schedule": "streams", "workload": w.name, "steps": args.steps,
                          "median_us": round(med * 1e3, 2), "mean_us": round(mean * 1e3, 2)}),
              flush=True)
        return

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    if args.only == "all" and not args.no_autotune:
        # the tuned plan (persistent chunk shapes, weight layouts and, where the tile count
        # leaves a partial last round, the balanced schedule), timed at the settled clock
        # after the warm-up; then a few calls of the chosen plan before the timed region
        mmar.autotune(w.M, w.N, w.K, P)
        for _ in range(10):
            fused()
        torch.cuda.synchronize()
    plan = mmar.get_plan(w.M, w.N, w.K, P)
    stream = torch.cuda.current_stream()
    # two HIP events around the K back-to-back launches on the launch stream: the mean
    # launch duration includes any gap between launches (none: the queue stays full), and
    # no event record sits between two launches (each one costs the GPU about 10 us idle)
    e_first = torch.cuda.Event(enable_timing=True)
    e_last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_first.record(stream)
    for _ in range(args.steps):
        fused()
    e_last.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = e_first.elapsed_time(e_last) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e12

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.desc}", "M": w.M, "K": w.K, "N": w.N, "P": P,
                   "p_drop": p, "seed": seed, "out_dtype": "fp32", "accumulate": "fp32",
                   "plan": {"schedule": {1: "sequential", 2: "streams", 3: "persistent",
                                         4: "balanced", 5: "split"}[plan["schedule"]],
                            "chunk": list(plan["chunk"]), "ring": plan["ring"],
                            "w_mode": {0: "direct", 1: "pretranspose"}[plan["w_mode"]],
                            "tile": {0: "256x128", 1: "256x192"}[plan["tile"]]}},
    }
    ksha = tile_kernel_sha()
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                          "traffic": _traffic(ksha),
                          "kernel": ("mmar::tile_kernel<kModeFused, 64, *> (persistent; with a "
                                     "pre-transposed W the step also runs the transpose kernel)"
                                     if plan["schedule"] == 3 else
                                     "mmar::tile_kernel<kModeFused, 64, *> over the head block, then "
                                     "the tail's one-slice partials and reduce+epilogue kernels "
                                     "(balanced schedule; achieved is over the whole step)"),
                          "per_launch": f"2*M*N*K = {w.flops} flop"}
    result["pct_bf16_peak"] = round(100 * value / PEAK_BF16_TFLOPS, 2)

    if args.only == "all":
        reps = max(10, args.steps)
        t_fused, _, t_fused_min, t_fused_p90 = _ev_time(torch, fused, reps, stats=True)
        # cold caches: write 1 GiB (more than the 8 x 4 MB L2 and the 256 MB MALL) before
        # every call
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        t_cold = _ev_time(torch, fused, max(10, reps // 4), before=lambda: flush.fill_(1.0))[0]
        del flush
        T = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        t_gemm = _ev_time(torch, lambda: mmar.gemm_only(X, W, P, out=T), reps)[0]
        # the epilogue's exposed cost: fused and GEMM-only (the same persistent kernel on the
        # plan's tile, storing T instead of applying the epilogue) alternated launch by launch
        pers = lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "persistent", chunk=plan["chunk"]
                                     if plan["schedule"] == 3 else (0, 0), w_mode="direct",
                                     tile=plan["tile"], out=out)
        pr_f, pr_g, pr_d, pr_iqr = _paired(torch, pers, lambda: mmar.gemm_only(X, W, P, out=T),
                                           max(100, args.steps))
        parts = torch.empty((P, w.M, w.N), dtype=torch.float32, device="cuda")
        t_parts = _ev_time(torch, lambda: mmar.gemm_partials(X, W, P, out=parts), reps)[0]
        t_re = _ev_time(torch, lambda: mmar.reduce_epilogue_only(parts, bias, res, p, seed, out=out),
                        reps)[0]
        t_epi = _ev_time(torch, lambda: mmar.reduce_epilogue_only(T[None], bias, res, p, seed, out=out),
                         reps)[0]
        t_seq = _ev_time(torch, lambda: mmar.sequential(X, W, bias, res, P, p, seed, out=out), reps)[0]
        t_str = _ev_time(torch, lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "streams", out=out),
                         reps)[0]
        mask = torch.empty((w.M, w.N), dtype=torch.uint8, device="cuda")
        t_unf = _ev_time(torch, lambda: mmar.unfused(X, W, bias, res, P, p, seed, out=out, mask=mask),
                         reps)[0]
        del mask
        t_dir = _ev_time(torch, lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "persistent",
                                                      w_mode="direct", out=out), reps)[0]
        t_pre = _ev_time(torch, lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "persistent",
                                                      w_mode="pretranspose", out=out), reps)[0]
        t_bal = _ev_time(torch, lambda: mmar.fused_ex(X, W, bias, res, P, p, seed, "balanced",
                                                      w_mode="direct", out=out), reps)[0]
        Wt = mmar.transpose_weight(W)
        t_tr = _ev_time(torch, lambda: mmar.transpose_weight(W, out=Wt), reps)[0]
        t_nt = _ev_time(torch, lambda: mmar.fused_nt(X, Wt, bias, res, P, p, seed, out=out), reps)[0]
        del Wt
        # the same block with its output rounded once more, to bf16 (half the output bytes)
        outb = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        t_bf16 = _ev_time(torch, lambda: mmar.fused_bf16(X, W, bias, res, P, p, seed, out=outb),
                          reps)[0]
        del outb
        # vendor yardstick: hipBLASLt's plain bf16 GEMM at the block's shape through
        # torch.matmul (bf16 out, no slices, no reduction order, no epilogue: strictly less
        # work than the block)
        Cv = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        t_vendor, t_fused_batch = _ev_batches_ab(torch, lambda: torch.matmul(X, W, out=Cv),
                                                 fused, max(10, reps // 5), warm=150)
        del Cv
        del parts
        # one rank's share on its own, at its real shape: the GEMM of one K-slice (P = 1,
        # K / P deep) with its fp32 output (the partials kernel), what each of P
        # tensor-parallel GPUs would run before the exchange
        ks = w.K // P
        Xr, Wr = X[:, :ks].contiguous(), W[:ks].contiguous()
        # the per-rank kernel is the partials mode with one slice: S_p = X_p W_p, fp32
        T1 = T.view(1, w.M, w.N)
        # back to back in batches of 10 launches (the kernel's own time; a single call
        # after a synchronization also pays the launch latency, 8-10 us at this size)
        t_rank = _ev_batch(torch, lambda: mmar.gemm_partials(Xr, Wr, 1, out=T1), reps)
        t_rank_single = _ev_time(torch, lambda: mmar.gemm_partials(Xr, Wr, 1, out=T1), reps)[0]
        del Xr, Wr, T, T1
        torch.cuda.empty_cache()
        # the producer MatMul in front of the block (H = GeLU(X0 . W1 + b1), bf16) and the
        # whole MLP (producer then block), on the producer's seeded inputs
        pin = make_producer_inputs(w)
        pd = {k: torch.from_numpy(pin[k].view(np.int16)).to("cuda").view(torch.bfloat16)
              for k in ("X0", "W1", "b1")}
        Hbuf = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")
        t_prod = _ev_time(torch, lambda: mmar.gelu_linear(pd["X0"], pd["W1"], pd["b1"], out=Hbuf),
                          reps)[0]
        t_mlp = _ev_time(torch, lambda: mmar.mlp(pd["X0"], pd["W1"], pd["b1"], W, bias, res, P, p,
                                                 seed, out=out, hidden=Hbuf), reps)[0]
        # the same MLP in one call, H handed to the block in row chunks (producer of chunk
        # c + 1 on this stream beside the block of chunk c on the library's second stream)
        t_mlp_ch = {}
        for cm in (w.M // 8, w.M // 4, w.M // 2):
            if cm % 32 == 0 and cm > 0:
                t_mlp_ch[cm] = _ev_time(torch, lambda: mmar.mlp_chunked(
                    pd["X0"], pd["W1"], pd["b1"], W, bias, res, P, p, seed, chunk_m=cm, out=out,
                    hidden=Hbuf), reps)[0]
        del pd, Hbuf
        torch.cuda.empty_cache()
        # the QKV projection in front of the GPT-2 attention block (bias, no activation):
        # [8192, 3072] x [3072, 9216], whichever block workload is timed
        qw = WORKLOADS["gpt2_attn"]
        qin = make_qkv_inputs(qw)
        qd = {k: torch.from_numpy(qin[k].view(np.int16)).to("cuda").view(torch.bfloat16)
              for k in ("X0", "Wqkv", "bqkv")}
        Qbuf = torch.empty((qw.M, 3 * qw.K), dtype=torch.bfloat16, device="cuda")
        t_qkv = _ev_time(torch, lambda: mmar.linear(qd["X0"], qd["Wqkv"], qd["bqkv"], "none",
                                                    out=Qbuf), reps)[0]
        qkv_flops = 2 * qw.M * qw.N * 3 * qw.K
        del qd, Qbuf
        torch.cuda.empty_cache()
        # the data-parallel side: gradient average + Adam step over BERT-large's parameters
        # (seeded on the device; HBM-bound, (4P + 26) bytes per parameter)
        aw = ADAM_WORKLOADS["bert_large_adam"]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(aw.seed)
        ag = torch.randn((aw.P, aw.n), generator=gen, device="cuda").mul_(1e-2)
        ap = torch.randn(aw.n, generator=gen, device="cuda").mul_(0.02)
        am = torch.randn(aw.n, generator=gen, device="cuda").mul_(1e-3)
        av = torch.randn(aw.n, generator=gen, device="cuda").mul_(1e-3).square_().add_(
            am.mul(2).square())
        apb = torch.empty(aw.n, dtype=torch.bfloat16, device="cuda")
        t_adam = _ev_time(torch, lambda: mmar.adam_step(ag, ap, am, av, aw.step, aw.lr, aw.beta1,
                                                        aw.beta2, aw.eps, aw.weight_decay,
                                                        param_bf16=apb), 20)[0]
        t_adam_torch = None
        try:   # PyTorch's own path for comparison: mean of the replicas, then fused AdamW
            tp = torch.nn.Parameter(ap.clone())
            topt = torch.optim.AdamW([tp], lr=aw.lr, betas=(aw.beta1, aw.beta2), eps=aw.eps,
                                     weight_decay=aw.weight_decay, fused=True)

            def torch_step():
                tp.grad = ag.mean(dim=0)
                topt.step()
            t_adam_torch = _ev_time(torch, torch_step, 20)[0]
            del tp, topt
        except (RuntimeError, TypeError, ValueError):
            t_adam_torch = None
        del ag, ap, am, av, apb
        torch.cuda.empty_cache()
        re_bytes = (4 * P + 6) * w.M * w.N + 2 * w.N
        epi_bytes = 10 * w.M * w.N + 2 * w.N
        result["times_us"] = {k: round(v * 1e3, 2) for k, v in
                              {"fused": t_fused, "gemm_alone": t_gemm, "partials_gemm": t_parts,
                               "re_alone": t_re, "epi_alone": t_epi, "sequential": t_seq,
                               "streams": t_str, "unfused": t_unf, "persistent_w_direct": t_dir,
                               "persistent_w_pretranspose": t_pre, "balanced": t_bal,
                               "w_transpose": t_tr,
                               "persistent_w_given_transposed": t_nt,
                               "fused_bf16_out": t_bf16}.items()}
        result["fused_us_stats"] = {"median": round(t_fused * 1e3, 2), "min": round(t_fused_min * 1e3, 2),
                                    "p90": round(t_fused_p90 * 1e3, 2),
                                    "median_cold_caches": round(t_cold * 1e3, 2)}
        # Hidden fractions, from the paired protocol: d = median over pairs of
        # (T_fused - T_gemm_alone) on the persistent kernel with the plan's tile (IQR beside
        # it).  T_re_alone reduces P materialized partials, which the persistent schedule
        # never writes: it removes the partial traffic rather than hiding it, so
        # `hidden_fraction` is near 1 by construction; `hidden_fraction_epilogue` (against
        # the epilogue alone over a materialized T) is the meaningful one.  Values are
        # clamped to [0, 1] and `*_raw` keeps the unclamped figure.
        def _frac(x):
            return round(min(1.0, max(0.0, x)), 4)
        result["paired_fused_minus_gemm"] = {"median_us": round(pr_d * 1e3, 2),
                                             "iqr_us": round(pr_iqr * 1e3, 2),
                                             "fused_us": round(pr_f * 1e3, 2),
                                             "gemm_alone_us": round(pr_g * 1e3, 2),
                                             "pairs": max(100, args.steps)}
        result["hidden_fraction"] = _frac(1.0 - pr_d / t_re)
        result["hidden_fraction_epilogue"] = _frac(1.0 - pr_d / t_epi)
        result["hidden_fraction_epilogue_raw"] = round(1.0 - pr_d / t_epi, 4)
        result["vendor_gemm_bf16"] = {"us": round(t_vendor * 1e3, 2),
                                      "TFLOP/s": round(flops / (t_vendor * 1e-3) / 1e12, 2),
                                      "what": f"torch.matmul [{w.M},{w.K}] x [{w.K},{w.N}] bf16 -> bf16 "
                                              "(hipBLASLt), no epilogue; after 150 untimed "
                                              "launches of each, batches of 10 launches back to "
                                              "back alternating with batches of the fused block",
                                      "fused_same_protocol_us": round(t_fused_batch * 1e3, 2),
                                      "fused_over_vendor_time": round(t_fused_batch / t_vendor, 3)}
        result["speedup_vs_sequential"] = round(t_seq / t_fused, 3)
        result["speedup_streams_vs_sequential"] = round(t_seq / t_str, 3)
        result["speedup_vs_unfused"] = round(t_unf / t_fused, 3)
        rank_flops = 2.0 * w.M * w.N * (w.K // P)
        result["per_rank_gemm"] = {"us": round(t_rank * 1e3, 2),
                                   "TFLOP/s": round(rank_flops / (t_rank * 1e-3) / 1e12, 2),
                                   "out_GBps": round(4.0 * w.M * w.N / (t_rank * 1e-3) / 1e9, 1),
                                   "us_single_call": round(t_rank_single * 1e3, 2),
                                   "timing": "median of batches of 10 launches back to back; "
                                             "us_single_call: one launch after a synchronization",
                                   "shape": f"[{w.M},{w.K // P}] x [{w.K // P},{w.N}] -> fp32, one slice"}
        result["producer_gelu"] = {"us": round(t_prod * 1e3, 2),
                                   "TFLOP/s": round(flops / (t_prod * 1e-3) / 1e12, 2),
                                   "shape": f"[{w.M},{w.N}] x [{w.N},{w.K}] -> bf16 [{w.M},{w.K}]"}
        result["mlp"] = {"us": round(t_mlp * 1e3, 2),
                         "TFLOP/s": round(2 * flops / (t_mlp * 1e-3) / 1e12, 2),
                         "what": "producer (GeLU layer) then the block, two calls in sequence"}
        result["mlp_chunked"] = {str(cm): {"us": round(t * 1e3, 2),
                                           "TFLOP/s": round(2 * flops / (t * 1e-3) / 1e12, 2)}
                                 for cm, t in t_mlp_ch.items()}
        result["mlp_chunked"]["what"] = ("mmar_mlp with row chunks of chunk_m rows: the producer of "
                                         "chunk c+1 beside the block of chunk c on a second stream")
        result["producer_qkv"] = {"us": round(t_qkv * 1e3, 2),
                                  "TFLOP/s": round(qkv_flops / (t_qkv * 1e-3) / 1e12, 2),
                                  "shape": f"[{qw.M},{qw.N}] x [{qw.N},{3 * qw.K}] -> bf16 "
                                           f"[{qw.M},{3 * qw.K}], bias, no activation"}
        adam_gbs = aw.bytes / (t_adam * 1e-3) / 1e9
        result["adam"] = {"workload": aw.desc, "us": round(t_adam * 1e3, 1),
                          "GB/s": round(adam_gbs, 1), "frac_hbm": round(adam_gbs / PEAK_HBM_GBS, 4),
                          "torch_mean_plus_fused_adamw_us":
                              None if t_adam_torch is None else round(t_adam_torch * 1e3, 1)}
        result["re_alone_GBps"] = round(re_bytes / (t_re * 1e-3) / 1e9, 1)
        result["epi_alone_GBps"] = round(epi_bytes / (t_epi * 1e-3) / 1e9, 1)

    if args.only == "all" and not args.no_other_workloads:
        del X, W, bias, res, out, d
        torch.cuda.empty_cache()
        others = [n for n in ("gpt2_attn", "gpt2_mlp", "bert_mlp", "gpt3_mlp") if n != w.name]
        result["other_workloads"] = _other_workloads(torch, np, mmar, others, 20, 20)
    if not args.no_cpu_baseline and args.only == "all":
        result["cpu_baseline"] = _cpu_baseline(inp, w, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
