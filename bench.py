#!/usr/bin/env python3
"""Benchmark of the Nystrom attention hot path on one MI355X.

One step = one full call of the library (landmarks, A and its
pseudo-inverse, B V, W, output with the convolution) on one batch of
synthetic input already resident in HBM.  Steps rotate over several input
replicas whose total exceeds the 256 MB Infinity Cache, so each step reads
its Q, K, V from HBM rather than from the previous step's cache lines.

Prints ONE JSON line.  `value` is tokens/s = B * n / step time on the
headline workload (bf16, B=4 H=12 n=4096 d=64 m=64, the n = 4096 config of
the target).  `roofline` rates the kernel that takes the most time per step
(per-kernel durations from the hipEvent pair the library attaches to each
of its launches, stamped with the kernel's own start and end, over the same
number of steps); `cpu_baseline` times the float64 oracle on the host cores.
--gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Nyström-attention tokens/s (B·n/s) on 1 MI355X; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
MALL_BYTES = 256 << 20


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="workload index 1..5 (default 3)")
    ap.add_argument("--also", default="2,4,5", help="other workloads to time briefly ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probs", action="store_true", help="skip timing the attention-weights call")
    ap.add_argument("--no-module", action="store_true", help="skip timing the self-attention module call")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="no GPU work: 'commands W DIR' prints the rocprofv3 runs; 'trace W DIR OUT' "
                         "and 'traffic W DIR OUT' turn their CSV output into text summaries")
    return ap.parse_args()


def source_sha() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "efficient_transformer_attention_segment_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Compulsory HBM bytes per launch of each kernel, from the per-head
    figures: reads of the [n, d] tensors it must consume, writes of the
    [n, d] output, plus the small per-head operands (landmarks, A, W, mask,
    conv weights).  Implementation scratch (B V partials, bf16 copies) is
    not counted."""
    e = 2 if w.dtype == "bf16" else 4
    BH, n, d, m = w.B * w.H, w.n, w.d, w.m
    nd = n * d * e
    small = 4 * (2 * m * d + m * m)              # Qt, Kt, A (float32) per head
    mask = w.B * n if w.mask is not None else 0
    per = {
        "k_landmark": BH * (2 * nd + small),
        "k_pinv_bv": BH * (2 * nd + 4 * m * d * 2 + 4 * m * m * 2) + mask,   # K, V, Qt, A, Z, B V
        "k_mw": BH * 4 * (m * m + 2 * m * d),                                 # Z, B V -> W
        "k_out": BH * (3 * nd + 4 * 2 * m * d) + w.H * 65 * 4,               # Q, V -> O; Kt, W
        "k_out_stream": BH * (3 * nd + 2 * 2 * m * d) + w.H * 65 * 4,        # Q, V -> O; Kt, W^T (bf16)
        "k_exact": BH * 4 * nd,
    }
    path = BH * 4 * nd + mask + w.H * 65 * 4                                  # Q, K, V in, O out
    return per, path


def algorithmic_flops(w):
    BH, n, d, m = w.B * w.H, w.n, w.d, w.m
    return BH * (8 * n * m * d + 4 * m * m * d + 8 * w.n_iter * m ** 3 + 130 * n * d)


def read_traffic(kernel: str, wname: str, sha: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE,
    WRITE_SIZE), scaled by the copy-kernel calibration factor; None unless
    the summary was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{wname}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_trace_avg(kernel: str, wname: str, sha: str):
    """The rocprofv3 average duration (us) of `kernel` in
    profiles/kernel_trace_<workload>.txt, or None unless that summary was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{wname}.txt")
    if not os.path.exists(path):
        return None
    lines = open(path).read().splitlines()
    if f"source_sha: {sha}" not in lines:
        return None
    for line in lines:
        cells = [c.strip() for c in line.split("|")]
        if len(cells) >= 3 and _short(cells[0]) == kernel:
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def make_replicas(w, x, count, torch):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to(a):
        return torch.from_numpy(a).to(dev).to(tdt)

    q0, k0, v0 = to(x["q"]), to(x["k"]), to(x["v"])
    reps = []
    for i in range(count):
        q, k, v = (q0, k0, v0) if i == 0 else (q0.clone(), k0.clone(), v0.clone())
        reps.append((q, k, v, torch.empty_like(q0)))
    mask = torch.from_numpy(x["key_mask"]).to(dev) if x["key_mask"] is not None else None
    conv = torch.from_numpy(x["conv_w"]).to(dev)
    return reps, mask, conv


def copy_bandwidth(torch, mb=1024, reps=10):
    """Attainable HBM bandwidth of a plain device copy (read + write bytes
    per second), timed with events on the current stream."""
    n = (mb << 20) // 4
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbs


def time_workload(w, steps, warmup, torch, nys):
    from efficient_transformer_attention_segment_amd.workloads import make_inputs
    x = make_inputs(w)
    e = 2 if w.dtype == "bf16" else 4
    per_rep = 4 * w.B * w.H * w.n * w.d * e
    count = max(2, min(16, math.ceil(2 * MALL_BYTES / per_rep)))
    reps, mask, conv = make_replicas(w, x, count, torch)
    fn = nys.nystrom_attention_bf16 if w.dtype == "bf16" else nys.nystrom_attention

    def step(i):
        q, k, v, o = reps[i % count]
        fn(q, k, v, mask, conv, m=w.m, n_iter=w.n_iter, init_option=w.init_option, out=o)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the same steps with one event at every step boundary on the stream the
    # library launches on (torch's current stream): the step-time spread
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    st = sorted(1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    pct = lambda f: st[min(len(st) - 1, int(round(f * (len(st) - 1))))]
    spread = {"p10": round(pct(0.1), 2), "p50": round(pct(0.5), 2), "p90": round(pct(0.9), 2)}
    # and again with the library's kernel timing on: each launch carries a
    # hipEvent pair that the runtime stamps with the kernel's own start and
    # end on that stream
    nys.profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = nys.profile_collect()
    nys.profile_enable(False)
    # warm: one input set for every step, so Q, K, V stay in the Infinity
    # Cache (reported beside the cold figure, never as the value)
    for _ in range(warmup):
        step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(0)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms, prof, count, x, spread, warm_ms


def time_probs(w, x, steps, warmup, torch, nys):
    """The same workload through nystrom_attention_probs (the output plus the
    attention weights F A^+, [B,H,n,m]): step time and the k_probs launch
    against its compulsory bytes (Q in, weights out, Kt and Z per head)."""
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v"))
    mask = torch.from_numpy(x["key_mask"]).to(dev) if x["key_mask"] is not None else None
    conv = torch.from_numpy(x["conv_w"]).to(dev)
    out = torch.empty_like(q)
    probs = torch.empty((w.B, w.H, w.n, w.m), dtype=tdt, device=dev)

    def step():
        nys.attention_with_probs(q, k, v, mask, conv, m=w.m, n_iter=w.n_iter, init_option=w.init_option,
                                 out=out, probs=probs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    nys.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = nys.profile_collect()
    nys.profile_enable(False)
    e = 2 if w.dtype == "bf16" else 4
    BH, M = w.B * w.H, 32 * ((w.m + 31) // 32)
    nbytes = BH * (w.n * w.d * e + w.n * w.m * e + 2 * 2 * M * w.d + 4 * M * M)
    tot, cnt = prof["k_probs"]
    us = 1e3 * tot / cnt
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"call": "nystrom_attention_probs", "ms_per_step": round(ms, 5), "kernel": "k_probs",
            "kernel_avg_us": round(us, 2), "algorithmic_bytes_per_launch": nbytes,
            "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}


def time_module(w, steps, warmup, torch, nys, core_ms):
    """The self-attention module at the workload's shape (hidden = H d): the
    stacked q/k/v projection (the library's GEMM, k_qkv) and the attention
    reading its output in place; the projection kernel is timed with the
    library's kernel-stamped events."""
    from efficient_transformer_attention_segment_amd.workloads import make_module_inputs
    hidden = w.H * w.d
    inp = make_module_inputs(w.B, w.n, hidden, w.H, w.d, seed=2000 + w.index, dtype=w.dtype,
                             lengths=None if w.mask is None else [w.mask[1]] * w.B)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x, wq, bq = (torch.from_numpy(inp[k]).to(dev).to(tdt) for k in ("x", "w_qkv", "b_qkv"))
    cw = torch.from_numpy(inp["conv_w"]).to(dev)
    km = torch.from_numpy(inp["key_mask"]).to(dev) if inp["key_mask"] is not None else None
    qkv = torch.empty((w.B, w.n, 3, w.H, w.d), dtype=tdt, device=dev)
    out = torch.empty((w.B, w.n, hidden), dtype=tdt, device=dev)

    def step():
        nys.self_attention(x, wq, bq, w.H, km, cw, m=w.m, n_iter=w.n_iter, init_option=w.init_option, qkv=qkv,
                           out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    nys.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = nys.profile_collect()
    nys.profile_enable(False)
    flops = 2 * w.B * w.n * hidden * 3 * w.H * w.d
    tot, cnt = prof.get("k_qkv", (0.0, 1))
    gemm_us = 1e3 * tot / cnt
    return {"call": "nystrom_self_attention", "hidden": hidden, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.tokens / (ms / 1e3), 1), "attention_only_ms": round(core_ms, 5),
            "projection_kernel": "k_qkv", "projection_us": round(gemm_us, 2), "projection_flops": flops,
            "projection_tflops": round(flops / (gemm_us * 1e-6) / 1e12, 1) if gemm_us > 0 else None,
            "projection_mfma_frac": round(flops / (gemm_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4)
            if gemm_us > 0 else None,
            "kernels_us": {kk: round(1e3 * t / c, 2) for kk, (t, c) in prof.items()},
            "note": "inputs resident"}


def time_backward(w, x, steps, warmup, torch, nys):
    """The backward pass (nystrom_attention_backward: the forward stages
    recomputed, then dq, dk, dv, dconv_w) on the workload: step time and
    per-kernel times."""
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v"))
    dout = torch.randn(q.shape, device=dev).to(tdt)
    mask = torch.from_numpy(x["key_mask"]).to(dev) if x["key_mask"] is not None else None
    conv = torch.from_numpy(x["conv_w"]).to(dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dw = torch.empty(conv.shape, dtype=torch.float32, device=dev)

    def step():
        nys.attention_backward(q, k, v, dout, mask, conv, m=w.m, n_iter=w.n_iter, init_option=w.init_option,
                               dq=dq, dk=dk, dv=dv, dconv_w=dw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    nys.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = nys.profile_collect()
    nys.profile_enable(False)
    return {"call": "nystrom_attention_backward", "ms_per_step": round(ms, 5),
            "tokens_per_s": round(w.tokens / (ms / 1e3), 1),
            "kernels_us": {kk: round(1e3 * t / c, 2) for kk, (t, c) in prof.items()}}


def cpu_baseline(w, x, budget_s):
    import numpy as np
    from oracle import nystrom_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.nystrom_attention(x["q"], x["k"], x["v"], x["key_mask"], x["conv_w"], w.m, w.n_iter,
                            w.init_option)
        times.append(time.perf_counter() - t0)
        if len(times) >= 30 or time.perf_counter() - t_start > budget_s:
            break
    med = float(np.median(times))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {"value": w.tokens / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full float64 oracle calls of {w.name} (median {med:.2f} s each)",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": model, "blas_threads": int(threads)}


def copy_probe(mb, torch):
    n = (mb << 20) // 4
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}))


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    """'void nys::k_out<unsigned short, 64>(nys::OutArgs)' -> 'k_out'."""
    head = name.split("(")[0].split("<")[0]
    return head.replace("void ", "").split("::")[-1].strip()


# rocprofv3 runs behind the summaries in profiles/ (run from /tmp with
# TMPDIR=/tmp; {R} = repository root, {O} = output directory, {W} = workload
# index).  Counter passes each take one counter, on a short bench run.
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {O}/trace -o trace -- "
             "python3 {R}/bench.py --workload {W} --steps 20 --warmup 5 --also '' --no-cpu-baseline --no-probs "
             "--no-module --no-backward",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {O}/fetch -o fetch -- "
             "python3 {R}/bench.py --workload {W} --steps 5 --warmup 2 --also '' --no-cpu-baseline --no-probs "
             "--no-module --no-backward",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {O}/write -o write -- "
             "python3 {R}/bench.py --workload {W} --steps 5 --warmup 2 --also '' --no-cpu-baseline --no-probs "
             "--no-module --no-backward",
    "trace_all": "rocprofv3 --kernel-trace --stats --output-format csv -d {O}/trace_all -o trace_all -- "
                 "python3 {R}/bench.py --workload {W} --steps 10 --warmup 3 --also '' --no-cpu-baseline",
    "sq": "rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_INSTS_LDS "
          "SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA --output-format csv -d {O}/sq -o sq -- "
          "python3 {R}/bench.py --workload {W} --steps 5 --warmup 2 --also '' --no-cpu-baseline --no-probs "
          "--no-module --no-backward",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {O}/copy_fetch -o copy_fetch -- "
                  "python3 {R}/bench.py --copy-probe-mb 256",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {O}/copy_write -o copy_write -- "
                  "python3 {R}/bench.py --copy-probe-mb 256",
}
COPY_PROBE_MB = 256


def summarize(argv):
    """Text summaries of rocprofv3 output for profiles/.

    commands W O          print the rocprofv3 command lines for workload W
    trace W O OUTDIR      kernel_trace_<workload>.txt: rocprofv3 per-kernel
                          statistics beside the bench's own event timings
    trace_all W O OUTDIR  kernel_trace_all_<workload>.txt: the same for the
                          bench with the weights, module and backward calls
    traffic W O OUTDIR    traffic_<kernel>_<workload>.txt for every library
                          kernel: FETCH_SIZE / WRITE_SIZE per launch, scaled
                          by a plain copy of known size
    counters W O OUTDIR   counters_<workload>.txt: per kernel the SQ counters
                          of one pass (matrix-core busy fraction against the
                          kernel's rocprof duration on all 1024 SIMDs at
                          2.4 GHz, wave wait fractions, LDS bank conflict
                          cycles per LDS instruction)
    """
    from efficient_transformer_attention_segment_amd.workloads import WORKLOADS
    kind, widx, odir = argv[0], int(argv[1]), argv[2]
    w = WORKLOADS[widx]
    cmds = {k: v.format(R="<repo>", O=odir, W=widx) for k, v in PROFILE_COMMANDS.items()}
    if kind == "commands":
        for k, v in PROFILE_COMMANDS.items():
            print(v.format(R=ROOT, O=odir, W=widx))
        return
    outdir = argv[3]
    sha = source_sha()
    if kind in ("trace", "trace_all"):
        stats = _csv_rows(os.path.join(odir, kind, f"{kind}_kernel_stats.csv"))
        bench_line = None   # the same bench command, run without the profiler
        plain = os.path.join(odir, "plain_bench.json")
        if os.path.exists(plain):
            with open(plain) as f:
                for line in f:
                    if line.startswith("{"):
                        bench_line = json.loads(line)
        lines = [f"# Kernel durations, {w.name}",
                 f"# command (from /tmp, TMPDIR=/tmp): {cmds[kind]}",
                 f"# summary: python3 bench.py --summarize {kind} {widx} {odir} {outdir}",
                 f"source_sha: {sha}", "",
                 f"# bench column: {cmds['trace'].split(' -- ', 1)[1]} run alone (no profiler), "
                 "kernel-stamped hipEvents",
                 "kernel | calls | rocprof avg_us | min_us | max_us | % of GPU time | bench hipEvent avg_us",
                 "---|---|---|---|---|---|---"]
        if kind == "trace_all":
            bench_line = None
            lines = lines[:5] + ["kernel | calls | rocprof avg_us | min_us | max_us | % of GPU time", "---|---|---|---|---|---"]
        bk = (bench_line or {}).get("kernels", {})
        for r in stats:
            k = _short(r["Name"])
            ev = bk.get(k, {}).get("avg_us")
            row = (f"{r['Name'][:80]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}")
            lines.append(row if kind == "trace_all" else row + f" | {'' if ev is None else f'{ev:.2f}'}")
        if bench_line:
            lines += ["", f"bench without the profiler: ms_per_step {bench_line['ms_per_step']}, "
                          f"step_us {bench_line.get('step_us')}, value {bench_line['value']} tokens/s"]
        path = os.path.join(outdir, f"kernel_trace_{'all_' if kind == 'trace_all' else ''}{w.name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)
        return
    if kind == "traffic":
        copy_bytes = COPY_PROBE_MB << 20

        def per_kernel(path):
            acc = {}
            for r in _csv_rows(path):
                acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
            return acc

        def copy_kib(path):
            return max(float(r["Counter_Value"]) for r in _csv_rows(path) if "copy" in r["Kernel_Name"].lower())

        f_fac = copy_bytes / 1024.0 / copy_kib(os.path.join(odir, "copy_fetch", "copy_fetch_counter_collection.csv"))
        w_fac = copy_bytes / 1024.0 / copy_kib(os.path.join(odir, "copy_write", "copy_write_counter_collection.csv"))
        fk = per_kernel(os.path.join(odir, "fetch", "fetch_counter_collection.csv"))
        wk = per_kernel(os.path.join(odir, "write", "write_counter_collection.csv"))
        per_bytes, _ = algorithmic_bytes(w)
        for k in sorted(fk):
            if not k.startswith("k_"):
                continue
            fkib = sum(fk[k]) / len(fk[k])
            wkib = sum(wk.get(k, [0.0])) / max(1, len(wk.get(k, [])))
            hbm = (fkib * f_fac + wkib * w_fac) * 1024.0
            lines = [f"# HBM traffic per launch of {k}, {w.name}",
                     f"# commands (from /tmp, TMPDIR=/tmp):",
                     *[f"#   {cmds[c]}" for c in ("fetch", "write", "copy_fetch", "copy_write")],
                     f"# summary: python3 bench.py --summarize traffic {widx} {odir} {outdir}",
                     f"# factors: a {COPY_PROBE_MB} MiB device copy reads {COPY_PROBE_MB} MiB and writes "
                     f"{COPY_PROBE_MB} MiB; FETCH_SIZE / WRITE_SIZE read for it give the scale factors below",
                     f"workload: {w.name}", f"kernel: {k}", f"source_sha: {sha}",
                     f"dispatches: {len(fk[k])}",
                     f"fetch_kib_per_launch: {fkib:.1f}", f"write_kib_per_launch: {wkib:.1f}",
                     f"copy_fetch_factor: {f_fac:.3f}", f"copy_write_factor: {w_fac:.3f}",
                     f"hbm_bytes_per_launch: {hbm:.0f}",
                     f"algorithmic_bytes_per_launch: {per_bytes.get(k, 'n/a')}"]
            path = os.path.join(outdir, f"traffic_{k}_{w.name}.txt")
            with open(path, "w") as f:
                f.write("\n".join(lines) + "\n")
            print(path)
        return
    if kind == "counters":
        rows = _csv_rows(os.path.join(odir, "sq", "sq_counter_collection.csv"))
        acc = {}
        for r in rows:
            k = _short(r["Kernel_Name"])
            if not k.startswith("k_"):
                continue
            d = acc.setdefault(k, {})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        trace = {}
        tpath = os.path.join(odir, "trace", "trace_kernel_stats.csv")
        if os.path.exists(tpath):
            for r in _csv_rows(tpath):
                trace[_short(r["Name"])] = float(r["AverageNs"]) / 1e3
        lines = [f"# SQ counters per launch, {w.name}",
                 f"# command (from /tmp, TMPDIR=/tmp): {cmds['sq']}",
                 f"# durations: {cmds['trace']}",
                 f"# summary: python3 bench.py --summarize counters {widx} {odir} {outdir}",
                 f"source_sha: {sha}", "",
                 "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x rocprof avg duration x 2.4 GHz);",
                 "# wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES; wait_inst = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;",
                 "# lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS (cycles per LDS instruction)",
                 "kernel | launches | rocprof avg_us | SQ_INSTS_MFMA | mfma_busy | wait | wait_inst | "
                 "SQ_INSTS_LDS | lds_conflict",
                 "---|---|---|---|---|---|---|---|---"]
        for k in sorted(acc):
            d = {c: sum(v) / len(v) for c, v in acc[k].items()}
            n = len(next(iter(acc[k].values())))
            us = trace.get(k)
            busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            mb = busy / (1024 * us * 1e-6 * 2.4e9) if us else None
            wc = d.get("SQ_WAVE_CYCLES", 0.0) or 1.0
            li = d.get("SQ_INSTS_LDS", 0.0)
            lines.append(f"{k} | {n} | {'' if us is None else f'{us:.2f}'} | {d.get('SQ_INSTS_MFMA', 0):.0f} | "
                         f"{'' if mb is None else f'{mb:.3f}'} | {d.get('SQ_WAIT_ANY', 0) / wc:.3f} | "
                         f"{d.get('SQ_WAIT_INST_ANY', 0) / wc:.3f} | {li:.0f} | "
                         f"{(d.get('SQ_LDS_BANK_CONFLICT', 0) / li) if li else 0:.3f}")
        path = os.path.join(outdir, f"counters_{w.name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)
        return
    raise SystemExit(f"unknown summary kind {kind!r}")


def main():
    args = parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU path is not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb, torch)
        return
    import efficient_transformer_attention_segment_amd as nys
    from efficient_transformer_attention_segment_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    ms, prof, reps, x, spread, warm_ms = time_workload(w, args.steps, args.warmup, torch, nys)
    value = w.tokens / (ms / 1e3)
    per_bytes, path_bytes = algorithmic_bytes(w)
    sha = source_sha()
    kern = {k: {"avg_us": 1e3 * tot / cnt, "launches_per_step": cnt / args.steps}
            for k, (tot, cnt) in prof.items()}
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    dom_us = kern[dom]["avg_us"]
    achieved = per_bytes.get(dom, 0) / (dom_us * 1e-6) / 1e9
    flops = algorithmic_flops(w)
    path = {"bytes": path_bytes, "hbm_frac": round(path_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4),
            "roofline_us": round(1e6 * max(path_bytes / (HBM_PEAK_GBS * 1e9),
                                           flops / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)), 2)}
    rp_us = read_trace_avg(dom, w.name, sha)
    rp_ach = per_bytes.get(dom, 0) / (rp_us * 1e-6) / 1e9 if rp_us else None
    # frac: the dominant kernel (live kernel-stamped events); call_frac: the
    # whole call's roofline time over its measured time, the measure the
    # 50 % target is stated in
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(dom, w.name, sha), "kernel": dom,
                "kernel_avg_us": round(dom_us, 2),
                "algorithmic_bytes_per_launch": per_bytes.get(dom, 0),
                "rocprof_avg_us": rp_us,
                "frac_rocprof": round(rp_ach / HBM_PEAK_GBS, 4) if rp_ach else None,
                "call_frac": round(path["roofline_us"] / (ms * 1e3), 4),
                "call_roofline_us": path["roofline_us"]}
    also = []
    for s in [s for s in args.also.split(",") if s.strip()]:
        wi = WORKLOADS[int(s)]
        if wi.index == w.index:
            continue
        msi, profi, _, _, _, _ = time_workload(wi, max(5, args.steps // 5), max(2, args.warmup // 2), torch, nys)
        pb, pathb = algorithmic_bytes(wi)
        fl = algorithmic_flops(wi)
        rl_us = 1e6 * max(pathb / (HBM_PEAK_GBS * 1e9), fl / (MFMA_PEAK_TFLOPS[wi.dtype] * 1e12))
        also.append({"workload": wi.name, "dtype": wi.dtype, "ms_per_step": round(msi, 4),
                     "tokens_per_s": round(wi.tokens / (msi / 1e3), 1),
                     "path_hbm_frac": round(pathb / (msi * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "path_roofline_us": round(rl_us, 2),
                     "call_frac": round(rl_us / (msi * 1e3), 4),
                     "kernels_us": {k: round(1e3 * t / c, 2) for k, (t, c) in profi.items()}})
    weights = None if args.no_probs else time_probs(w, x, max(5, args.steps // 5), max(2, args.warmup // 2),
                                                    torch, nys)
    # the projection GEMM keeps the matrix cores busy and reaches its steady
    # rate only after tens of milliseconds of such work (measured: 87 us per
    # GEMM after 30 calls, 70 us after 200), so the module gets 200 untimed
    # warm-up calls and 50 timed ones (about 30 ms in all)
    module = None if args.no_module else time_module(w, max(50, args.steps), max(200, args.warmup * 20), torch,
                                                     nys, ms)
    backward = None
    if not args.no_backward:
        backward = time_backward(w, x, max(5, args.steps // 5), max(2, args.warmup // 2), torch, nys)
    copy_gbs = copy_bandwidth(torch)
    roofline["attainable_copy_GBps"] = round(copy_gbs, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbs, 4)
    path["frac_of_copy"] = round(path_bytes / (ms * 1e-3) / 1e9 / copy_gbs, 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, x, args.cpu_seconds)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, 0.02 N(0,1) conv weights, right-padding masks)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "d": w.d, "m": w.m,
                   "n_iter": w.n_iter, "init_option": w.init_option, "conv_taps": 65,
                   "mask": (f"valid length U{{{w.mask[0]}..{w.mask[1]}}}" if w.mask else "none"),
                   "input_replicas": reps, "parallelism": "single GPU"},
        "step_us": spread,
        "warm": {"ms_per_step": round(warm_ms, 5), "tokens_per_s": round(w.tokens / (warm_ms / 1e3), 1),
                 "note": "one input set for every step (cache-resident); the value above rotates "
                         "input replicas larger than the Infinity Cache"},
        "roofline": roofline, "path": path, "kernels": {k: {kk: round(vv, 3) for kk, vv in v.items()}
                                                         for k, v in kern.items()},
        "cpu_baseline": cpu, "also": also, "attention_weights": weights, "module": module, "backward": backward,
        "source_sha": sha,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
