#!/usr/bin/env python3
"""Benchmark of the routed 4-bit MoE expert FFN forward on one MI355X.

One step = one full forward (route/sort/tile, gate|up + GeGLU, down +
weighted unsort, combine) over one batch of synthetic inputs that are already
resident in HBM.  Several full copies of every input are rotated step by step
so that the 256 MB Infinity Cache cannot serve a step from the previous one.

Prints ONE JSON line:
  value         whole-forward assignments/s over the timed steps (host clock,
                synchronised on both sides), no per-kernel events in that loop;
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                divided by its mean duration, from HIP events recorded on the
                library's stream in a second, instrumented loop;
  cpu_baseline  the CPU oracle on this host's cores, on a bounded sample of the
                same workload, with a parity check of the GPU output against it.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "expert-FFN assignments/s and TFLOP/s (or HBM GB/s) vs roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
BM_BIG, BM_SMALL = 64, 16      # tile heights the forward routes with


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(p):
    """Per-launch algorithmic bytes and flops of each kernel: what the method
    must move and compute for the rows that kernel owns (experts of <= 16
    rows go to the skinny kernels, larger ones to the wide kernels), not what a
    kernel happens to re-read."""
    import numpy as np
    E, H, I, T, k = p.E, p.H, p.I, p.T, p.k
    A = T * k
    G_h, G_i = H // p.gs, I // p.gs
    cb = p.bits / 8                                           # code bytes per weight
    gu_expert = int(2 * I * H * cb) + 2 * (2 * I * G_h * 2)   # codes + scales + biases
    d_expert = int(H * I * cb) + 2 * (H * G_i * 2)
    ids = p.topk_ids.ravel()
    counts = np.bincount(ids, minlength=E)
    # experts of <= 16 rows run as one skinny tile, larger ones in wide
    # tiles; batches of <= 16 tokens run every expert on the skinny path
    skinny_max = A if T <= BM_SMALL else BM_SMALL
    bm_big = 32 if p.bits == 8 else BM_BIG  # the forward's wide tile height
    skinny_rows = np.where(counts <= skinny_max, counts, 0)
    wide_rows = counts - skinny_rows
    in_skinny = np.isin(ids, np.nonzero((counts > 0) & (counts <= skinny_max))[0])
    tok = np.arange(A) // k
    tok_s = np.unique(tok[in_skinny]).size
    tok_w = np.unique(tok[~in_skinny]).size
    rs, rw = int(skinny_rows.sum()), int(wide_rows.sum())
    es, ew = int(np.count_nonzero(skinny_rows)), int(np.count_nonzero(wide_rows))
    work = {
        "moe_route_sort_tiles": dict(bytes=A * 12 + (2 * E + 1) * 4 + T * H * 4 + T * G_h * 4,
                                     flops=0),
        "moe_gateup_skinny": dict(bytes=es * gu_expert + tok_s * H * 2 + rs * I * 2,
                                  flops=rs * 4 * H * I),
        "moe_gateup_wide": dict(bytes=ew * gu_expert + tok_w * H * 2 + rw * I * 2,
                                flops=rw * 4 * H * I),
        "moe_down_skinny": dict(bytes=es * d_expert + rs * I * 2 + rs * H * 4, flops=rs * 2 * H * I),
        "moe_down_wide": dict(bytes=ew * d_expert + rw * I * 2 + rw * H * 4, flops=rw * 2 * H * I),
        "moe_combine": dict(bytes=A * H * 4 + T * H * 2 + A * 4, flops=A * H),
    }

    touched = int(np.count_nonzero(counts))
    fwd = dict(bytes=touched * (gu_expert + d_expert) + T * H * 2 + A * 8 + T * H * 2,
               flops=A * 6 * H * I)
    # tile heights of the forward's tiling (wide tiles near-equal per expert)
    hist = {"skinny 1-4": 0, "skinny 5-8": 0, "skinny 9-16": 0,
            "wide 17-32": 0, "wide 33-48": 0, "wide 49-64": 0}
    for c in counts.tolist():
        if c == 0:
            continue
        if c <= skinny_max:
            for r0 in range(0, c, BM_SMALL):
                r = min(BM_SMALL, c - r0)
                hist["skinny 1-4" if r <= 4 else "skinny 5-8" if r <= 8 else "skinny 9-16"] += 1
            continue
        n = -(-c // bm_big)
        for j in range(n):
            r = c // n + (1 if j < c % n else 0)
            hist["wide 17-32" if r <= 32 else "wide 33-48" if r <= 48 else "wide 49-64"] += 1
    split = dict(skinny_rows=rs, wide_rows=rw, experts_with_skinny_tile=es,
                 wide_tiles=int(np.sum((wide_rows + bm_big - 1) // bm_big)), tile_rows=hist)
    return work, fwd, split


def bound_of(w):
    t_hbm = w["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = w["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    return "hbm" if t_hbm >= t_mfma else "mfma"


def roofline_entry(w, seconds):
    b = bound_of(w)
    if b == "hbm":
        ach = w["bytes"] / seconds / 1e9
        return dict(bound="hbm", achieved=round(ach, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    ach = w["flops"] / seconds / 1e12
    return dict(bound="mfma", achieved=round(ach, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(ach / BF16_PEAK_TFLOPS, 4))


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if a summary for
    this kernel, workload and kernel source is committed under profiles/."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        from bit_gathered_quantized_amd.build import source_digest
        if rec.get("source_digest") != source_digest():
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_leg(p, gpu_out, seconds_budget: float):
    """The oracle (as it stands) on this host's cores, on a bounded sample of
    the same workload; the same run checks the GPU output."""
    import numpy as np

    import oracle

    if p.T <= 16:
        tokens = np.arange(p.T, dtype=np.int32)
        sample = f"full batch: {p.T} tokens x top-{p.k} = {p.T * p.k} assignments"
    else:
        rng = np.random.default_rng(123)
        n = 48
        tokens = np.sort(rng.choice(p.T, size=n, replace=False)).astype(np.int32)
        sample = f"{n} random tokens of {p.T} (x top-{p.k} = {n * p.k} assignments)"
    times = []
    ref = None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        r = oracle.ffn_tokens(p, tokens, want_h=False, want_y=False)
        times.append(time.perf_counter() - t0)
        if ref is None:
            ref = r["out"]
        if len(times) >= 2 and time.perf_counter() - t_start >= seconds_budget:
            break
        if len(times) >= 50:
            break
    med = statistics.median(times)
    n_asg = tokens.size * p.k
    one_thread = None
    if p.T <= 64:  # the small configurations: also one core
        cores = oracle.num_threads()
        oracle.set_num_threads(1)
        t1 = []
        t_start = time.perf_counter()
        while len(t1) < 20 and (len(t1) < 2 or time.perf_counter() - t_start < seconds_budget / 2):
            t0 = time.perf_counter()
            oracle.ffn_tokens(p, tokens, want_h=False, want_y=False)
            t1.append(time.perf_counter() - t0)
        oracle.set_num_threads(cores)
        one_thread = round(n_asg / statistics.median(t1), 3)
    got = gpu_out[tokens]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    allow = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(got), np.abs(ref)), 1e-38))) - 8)
    excess = float(np.max(np.abs(got - ref) - allow)) / rms
    base = dict(value=round(n_asg / med, 3), unit="assignments/s", cores=oracle.num_threads(),
                kind="oracle", sample=f"{sample}; median of {len(times)} runs",
                seconds_per_run=round(med, 4), host_cpu=host_cpu(),
                affinity=len(os.sched_getaffinity(0)))
    if one_thread is not None:
        base["one_thread_value"] = one_thread
    parity = dict(tokens=int(tokens.size), bf16_excess_over_rms=round(excess, 6), bar=2e-2,
                  ok=bool(excess <= 2e-2))
    return base, parity


def timed_loop(fn, steps):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def extra_legs(args, p, sets, prob, ws, out, stream):
    """The same workload through the device router, the SwiGLU epilogue and
    HIP-graph replays of the forward (host clock, same input rotation)."""
    import numpy as np
    import torch

    import bit_gathered_quantized_amd as bgq

    A = p.T * p.k
    steps = max(20, min(args.steps, 200))
    res = {}
    # device router at the workload's shape
    rng = np.random.default_rng(7)
    logits = torch.from_numpy(rng.standard_normal((p.T, p.E)).astype(np.float32)).cuda()
    ids = torch.empty((p.T, p.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    for _ in range(3):
        bgq.router_topk(logits, p.k, ids, wts, stream=stream)
    sec = timed_loop(lambda i: bgq.router_topk(logits, p.k, ids, wts, stream=stream), steps)
    res["router_topk"] = dict(us_per_call=round(sec * 1e6, 2), tokens_per_s=round(p.T / sec, 1),
                              shape=[p.T, p.E, p.k])
    # SwiGLU epilogue instead of GeGLU
    for i in range(3):
        bgq.expert_ffn_forward(*sets[i % len(sets)], swiglu=True, out=out, workspace=ws,
                               stream=stream)
    sec = timed_loop(lambda i: bgq.expert_ffn_forward(*sets[i % len(sets)], swiglu=True, out=out,
                                                      workspace=ws, stream=stream), steps)
    res["swiglu_forward"] = dict(ms_per_step=round(sec * 1e3, 5),
                                 assignments_per_s=round(A / sec, 1))
    # the pre-sorted entry, given each copy's expert-sorted order
    flat = p.topk_ids.ravel()
    keys = np.where((flat >= 0) & (flat < p.E), flat, p.E)
    order = torch.from_numpy(np.argsort(keys, kind="stable").astype(np.int32)).cuda()
    for i in range(3):
        bgq.expert_ffn_forward(*sets[i % len(sets)], out=out, workspace=ws, stream=stream,
                               sorted_order=order)
    sec = timed_loop(lambda i: bgq.expert_ffn_forward(*sets[i % len(sets)], out=out, workspace=ws,
                                                      stream=stream, sorted_order=order), steps)
    res["presorted_forward"] = dict(ms_per_step=round(sec * 1e3, 5),
                                    assignments_per_s=round(A / sec, 1))
    # the whole forward as one HIP graph per input copy
    graphs = []
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for st in sets:
            bgq.expert_ffn_forward(*st, out=out, workspace=ws, stream=cs)
        torch.cuda.synchronize()
        for st in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                bgq.expert_ffn_forward(*st, out=out, workspace=ws, stream=cs)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    sec = timed_loop(lambda i: graphs[i % len(graphs)].replay(), steps)
    res["graph_forward"] = dict(ms_per_step=round(sec * 1e3, 5),
                                assignments_per_s=round(A / sec, 1))
    if args.bits == 4 and args.group_size == 64 and not args.intermediate:
        res["other_geometries"] = geometry_legs(args, p, steps, stream)
    return res


def geometry_legs(args, p, steps, stream):
    """The same tokens and routing with weights of the other geometries: 8-bit
    codes, and 4-bit codes in groups of 32 and 128 columns (I rounded up to a
    multiple of 128 there).  Two copies of the weights are rotated."""
    import numpy as np
    import torch

    import bit_gathered_quantized_amd as bgq
    import moe_synth as ms

    c = ms.CONFIGS[args.workload]
    A = p.T * p.k
    res = {}
    for bits, gs in ((8, 64), (4, 32), (4, 128)):
        I = -(-p.I // gs) * gs
        q = ms.make_problem(p.E, p.H, I, p.T, p.k, seed=0, router=c["router"], gs=gs, bits=bits,
                            name=args.workload)
        assert np.array_equal(q.topk_ids, p.topk_ids)

        def t(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()
        sets = []
        for _ in range(2):
            sets.append([t(q.x, np.int16).view(torch.bfloat16), t(q.topk_ids, np.int32),
                         t(q.topk_weights, np.float32), t(q.w_gateup, np.int32), t(q.s_gateup, np.int16),
                         t(q.b_gateup, np.int16), t(q.w_down, np.int32), t(q.s_down, np.int16),
                         t(q.b_down, np.int16)])
        prob = bgq.problem(q.T, q.k, q.E, q.H, q.I, 0, group_size=gs, bits=bits)
        ws = torch.empty(bgq.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
        out = torch.empty((q.T, q.H), dtype=torch.bfloat16, device="cuda")

        def step(i):
            bgq.expert_ffn_forward(*sets[i % 2], out=out, workspace=ws, stream=stream)
        for i in range(3):
            step(i)
        sec = timed_loop(step, steps)
        res[f"bits{bits}_gs{gs}"] = dict(I=I, ms_per_step=round(sec * 1e3, 5),
                                         assignments_per_s=round(A / sec, 1))
        del sets, ws, out
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill16k",
                    choices=["tiny", "decode", "prefill4k", "prefill8k", "prefill16k"])
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the router, SwiGLU, pre-sorted, graph and geometry legs")
    ap.add_argument("--no-legs", action="store_true",
                    help="time only --workload (not the other workloads as well)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the forward, copy MIB MiB device-to-device 5 times "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--group-size", type=int, default=64, choices=[32, 64, 128],
                    help="quantisation group size of the synthetic weights")
    ap.add_argument("--bits", type=int, default=4, choices=[4, 8],
                    help="code width of the synthetic weights")
    ap.add_argument("--intermediate", type=int, default=0, metavar="I",
                    help="override the workload's intermediate size (e.g. 768 at group "
                         "size 128, which does not divide 704)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the expert FFN here runs on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_gathered_quantized_amd as bgq
    import moe_synth as ms

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bgq.lib()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 5}}),
              flush=True)
        return

    result, ctx = measure_workload(args, args.workload, args.steps, args.warmup, args.group_size,
                                   args.bits, args.intermediate, args.cpu_seconds,
                                   not args.no_cpu_baseline)
    p, sets, prob, ws, out, stream = ctx
    result = {
        "metric": METRIC,
        "value": result.pop("value"),
        "unit": "assignments/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        **result,
    }
    result["extras"] = None if args.no_extras else extra_legs(args, p, sets, prob, ws, out, stream)
    del sets, ws, out
    # the other workloads on the same GPU, each with its own roofline, parity
    # and CPU baseline (the headline is the largest one)
    legs = {}
    if not args.no_legs and not result["config"].get("custom"):
        for name, steps in LEG_STEPS.items():
            if name == args.workload:
                continue
            if name in NOT_RUN:
                legs[name] = dict(measured=False, reason=NOT_RUN[name])
                continue
            leg, _ = measure_workload(args, name, steps, max(5, steps // 10), ms.GROUP_SIZE, 4, 0,
                                      args.cpu_seconds / 2, not args.no_cpu_baseline)
            legs[name] = leg
    result["workloads"] = legs
    print(json.dumps(result), flush=True)


# Timed steps of the other workloads carried in the same JSON line.
LEG_STEPS = {"decode": 200, "prefill4k": 50, "prefill8k": 30}
# Workloads kept off the GPU, with the reason.
NOT_RUN = {"prefill8k": "a GPU memory fault on this workload in an earlier build of the kernels; "
                        "its cause has not been shown, so the workload is kept off the GPU"}


def measure_workload(args, name, steps, warmup, gs, bits, inter, cpu_seconds, want_cpu):
    """One workload: timed forward, per-kernel events, roofline of the dominant
    kernel, the whole forward's fraction of its roofline, and (want_cpu) the
    oracle's rate on a bounded sample with a parity check of the GPU output.
    Returns (result fields, (problem, input sets, problem struct, workspace,
    out, stream))."""
    import numpy as np
    import torch

    import bit_gathered_quantized_amd as bgq
    import moe_synth as ms

    c = ms.CONFIGS[name]
    I = inter or c["I"]
    custom = gs != ms.GROUP_SIZE or I != c["I"] or bits != 4
    if custom:
        p = ms.make_problem(c["E"], c["H"], I, c["T"], c["k"], seed=0, router=c["router"],
                            gs=gs, bits=bits, name=name)
    else:
        p = ms.make_config(name, seed=0)
    A = p.T * p.k
    counts = np.bincount(p.topk_ids.ravel(), minlength=p.E)
    touched = int(np.count_nonzero(counts))
    log(f"workload {name}: E={p.E} H={p.H} I={p.I} T={p.T} k={p.k} A={A} "
        f"gs={p.gs} touched={touched}")

    dev = torch.device("cuda", 0)

    def upload():
        def t(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
        return [t(p.x, np.int16).view(torch.bfloat16), t(p.topk_ids, np.int32),
                t(p.topk_weights, np.float32), t(p.w_gateup, np.int32), t(p.s_gateup, np.int16),
                t(p.b_gateup, np.int16), t(p.w_down, np.int32), t(p.s_down, np.int16),
                t(p.b_down, np.int16)]

    sets = [upload() for _ in range(max(1, args.copies))]
    prob = bgq.problem(p.T, p.k, p.E, p.H, p.I, 0, group_size=p.gs, bits=p.bits)
    ws = torch.empty(bgq.workspace_bytes(prob), dtype=torch.uint8, device=dev)
    out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        bgq.expert_ffn_forward(*sets[i % len(sets)], out=out, workspace=ws, stream=stream,
                               events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed loop: whole forward, host clock
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / steps * 1e3
    log(f"timed loop: {steps} steps, {ms_per_step * 1e3:.1f} us/step")

    # instrumented loop: per-kernel durations from events on the same stream
    kernels = bgq.KERNELS
    n_ev = min(steps, 100)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(bgq.N_EVENTS)]
           for _ in range(n_ev)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(n_ev):
        step(i, events=[e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    kern_us = {s: [] for s in kernels}
    fwd_us = []
    for row in evs:
        for j, s in enumerate(kernels):
            kern_us[s].append(row[2 * j].elapsed_time(row[2 * j + 1]) * 1e3)
        fwd_us.append(row[0].elapsed_time(row[-1]) * 1e3)
    mean_us = {s: statistics.fmean(v) for s, v in kern_us.items()}

    work, fwd_work, split = algorithmic_work(p)
    # at most 16 tokens the library launches no wide kernel: their event pair
    # brackets nothing
    not_launched = {"moe_gateup_wide", "moe_down_wide"} if p.T <= BM_SMALL else set()
    dominant = max((s for s in kernels if s not in not_launched), key=lambda s: mean_us[s])
    roof = roofline_entry(work[dominant], mean_us[dominant] * 1e-6)
    roof["kernel"] = dominant
    # counter summaries are committed for the named workloads only
    roof["traffic"] = None if custom else load_traffic(dominant, name)

    fwd_s = statistics.median(fwd_us) * 1e-6
    fwd_roof = roofline_entry(fwd_work, ms_per_step * 1e-3)
    forward = dict(
        event_us_median=round(statistics.median(fwd_us), 2),
        event_us_p10=round(float(np.percentile(fwd_us, 10)), 2),
        event_us_p90=round(float(np.percentile(fwd_us, 90)), 2),
        tflops=round(fwd_work["flops"] / fwd_s / 1e12, 2),
        hbm_gbs=round(fwd_work["bytes"] / fwd_s / 1e9, 1),
        algorithmic_bytes=int(fwd_work["bytes"]),
        algorithmic_flops=int(fwd_work["flops"]),
        bound=bound_of(fwd_work),
        frac=roofline_entry(fwd_work, fwd_s)["frac"],
        wall_frac=fwd_roof["frac"],
    )
    # the whole forward beside the dominant kernel: the fraction of its own
    # roofline (bytes or flops of the forward over the timed loop's time)
    roof["forward_frac"] = fwd_roof["frac"]
    roof["forward_bound"] = fwd_roof["bound"]
    kstats = {}
    for s in kernels:
        w = work[s]
        if s in not_launched:
            kstats[s] = dict(launched=False)
            continue
        entry = dict(mean_us=round(mean_us[s], 2))
        if (w["bytes"] or w["flops"]) and mean_us[s] > 0:
            e = roofline_entry(w, mean_us[s] * 1e-6)
            entry.update(bound=e["bound"], achieved=e["achieved"], unit=e["unit"], frac=e["frac"])
        kstats[s] = entry

    result = {
        "value": round(A / (ms_per_step * 1e-3), 1),
        "ms_per_step": round(ms_per_step, 5),
        "steps": steps,
        "config": {"workload": name, "E": p.E, "H": p.H, "I": p.I, "T": p.T,
                   "k": p.k, "assignments": A, "group_size": p.gs, "bits": p.bits,
                   "router": ms.CONFIGS[name]["router"], "seed": 0,
                   "touched_experts": touched, "input_copies": len(sets), **split,
                   **({"custom": True} if custom else {})},
        "roofline": roof,
        "forward": forward,
        "kernels": kstats,
    }
    if want_cpu:
        gpu_out = out.float().cpu().numpy().astype(np.float64)
        base, parity = cpu_baseline_leg(p, gpu_out, cpu_seconds)
        result["cpu_baseline"] = base
        result["parity"] = parity
    else:
        result["cpu_baseline"] = None
    return result, (p, sets, prob, ws, out, stream)


if __name__ == "__main__":
    main()
