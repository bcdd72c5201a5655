#!/usr/bin/env python3
"""Benchmark of the weight-only quantized GEMM on one MI355X.

Headline (the printed `value`): decode GEMV HBM bandwidth at M=1 over the
W4A16 decode workload -- K=2048, group 64, bf16 activations and output,
N in {2048, 3072, 13312} plus the tied-vocab projection N=131072.  One step
is one GEMV per shape; `value` = algorithmic bytes of a step / step time.

Secondary sections on the same JSON line:
  sweep    every (M, N) of the decode workload, M in {1, 2, 4, 8};
  prefill  W4A16 M=512, K=2048, N in {3072, 13312, 131072}, g in {64, 128},
           fp16 bias: TFLOP/s against the dense bf16 matrix-core peak (the
           aggregate over the M=512 shapes); the same shapes at M=2048 beside it;
  moe      grouped W4A16 MoE, 2048 tokens, hidden 2048, inter 1408,
           64 experts, top-6;
  w8       W8A16 at K=3584, N in {3584, 18944}, M from 1 to 4096, per-channel
           and group-128 scales;
  w4_forms W4A16 N=13312, K=2048 at M in {1, 512} for each scale form
           (groupwise with zeros, scale-only, per channel);
  w8a8     int8 x int8 GEMM at K=3584, N in {3584, 18944}, M from 1 to 4096,
           per-token x per-channel scales (TOP/s against the int8 peak);
  embed    int4 embedding lookups from the tied 131072 x 2048 table;
  quantize the load-side groupwise int4 quantizer on bf16 weights
           [N, 2048], N in {13312, 131072}, group 64 (GB/s against HBM);
  roofline the decode kernel of the N=131072 GEMV: algorithmic bytes per
           launch / its mean launch time (HIP events on the launch stream);
  cpu_baseline  the CPU oracle (its fp32-accumulating GEMM) on bounded
           samples: whole decode steps on every host thread (`value`), one
           thread, and one prefill, W8A16 and MoE shape each, with the host's
           CPU model, sockets and the thread count the oracle actually ran.

`python bench.py --trace-summary <kernel_trace.csv>` prints per-dispatch
statistics (median, p10, p90) of a rocprofv3 kernel trace of this script.

The compute-bound legs (prefill, MoE, W8A16, the int4 scale forms, W8A8 and
the dense-GEMM ceiling) are timed at the chip's sustained clock: each shape
first runs back to back, untimed, for 40 ms, then at least 20 ms of calls are
timed.  A short burst instead lands in the power controller's transient
(`--launch-series` prints it per launch): the first few ms run fast, the next
10-20 ms up to 25 % slower, then the kernel time settles.

Inputs are seeded synthetic data generated on the host and copied to HBM
before timing.  Memory-bound shapes rotate over enough identical weight
copies (>= 1 GiB per shape) that no launch finds its weights in the 256 MB
Infinity Cache or in L2.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix cores, TOP/s
ROTATE_BYTES = 1 << 30
STEADY_WARM_MS, STEADY_MIN_MS = 40.0, 20.0   # compute-bound legs: warm-up, timed span

DECODE_K, DECODE_G = 2048, 64
DECODE_N = [2048, 3072, 13312, 131072]
SWEEP = [(m, n) for m in (1, 2, 4, 8) for n in (2048, 3072, 13312)] + [(1, 131072)]
PREFILL = [(512, n, g) for g in (64, 128) for n in (3072, 13312, 131072)]
PREFILL_2048 = [(2048, n, g) for g in (64, 128) for n in (3072, 13312, 131072)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w4_bytes(m, n, k, g, bias=False):
    """Algorithmic bytes of one W4A16 GEMM: packed codes, bf16 scales and
    zeros, activations, output (and bias)."""
    return n * k // 2 + 2 * 2 * n * (k // g) + 2 * m * k + 2 * m * n + (2 * n if bias else 0)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ["weight_only_quantized_w8a16_amd/csrc/decode.hip",
                  "weight_only_quantized_w8a16_amd/csrc/qg_common.hpp"]


PREFILL_SOURCES = ["weight_only_quantized_w8a16_amd/csrc/prefill.hip",
                   "weight_only_quantized_w8a16_amd/csrc/tile_big.hpp",
                   "weight_only_quantized_w8a16_amd/csrc/tile_gemm.hpp",
                   "weight_only_quantized_w8a16_amd/csrc/qg_common.hpp"]
PREFILL_TRAFFIC_SHAPE = (512, 131072, 64)


def load_traffic(name="traffic_decode_w4_m1_n131072.json", sources=None):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter
    runs, if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest(sources or DECODE_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


class Weights:
    """`copies` identical device copies of one tiled W4 weight set."""

    def __init__(self, torch, qg, si, n, k, g, tag, copies, bias=False):
        packed, s, z, b = si.w4_weights(n, k, g, si.seed_of(tag, "w", n, k, g),
                                        bias_dtype=si.FP16 if bias else si.NONE)
        dev = "cuda"
        base = qg.repack_w4(torch.from_numpy(packed).to(dev))
        sc = torch.from_numpy(s.view("int16")).view(torch.bfloat16).to(dev)
        ze = torch.from_numpy(z.view("int16")).view(torch.bfloat16).to(dev)
        self.bias = torch.from_numpy(b.view("int16")).view(torch.float16).to(dev) if bias else None
        self.sets = [(base, sc, ze)]
        for _ in range(copies - 1):
            self.sets.append((base.clone(), sc.clone(), ze.clone()))
        self.n, self.k, self.g = n, k, g

    def __getitem__(self, i):
        return self.sets[i % len(self.sets)]


def copies_for(nbytes):
    return max(2, math.ceil(ROTATE_BYTES / nbytes))


def gpu_lead(torch, ms=20.0):
    """Queue a GPU-side wait so the host can enqueue ahead of the device:
    the timed kernels then run back to back, without host gaps."""
    try:
        torch.cuda._sleep(int(ms * 1e-3 * 2.1e9))
    except Exception:   # pragma: no cover - torch without _sleep
        pass


KERNEL_LEGS = ("decode", "prefill", "copy", "decode_small", "w8", "w8a8", "moe")


def launch_series(args, torch, qg, si):
    """Per-launch durations of `--steps` back-to-back calls (HIP events
    between calls, after a 6 ms GPU-side wait) of the M=512 N=131072 g=64
    W4A16 GEMM and of the 2048-token MoE: how the kernel time follows the
    chip's clock from the first launch of a burst to the sustained state."""
    dev = "cuda"
    stream = torch.cuda.current_stream()

    def series(fn, count):
        for i in range(3):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
        torch.cuda.synchronize()
        gpu_lead(torch, 6.0)
        ev[0].record(stream)
        for i in range(count):
            fn(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return [round(ev[i].elapsed_time(ev[i + 1]) * 1e3, 1) for i in range(count)]

    def summary(name, us):
        srt = sorted(us)
        rec = {"leg": name, "launches": len(us), "us": us,
               "first8_mean": round(sum(us[:8]) / 8, 1),
               "launch9_20_mean": round(sum(us[8:20]) / 12, 1),
               "last40_mean": round(sum(us[-40:]) / 40, 1),
               "median": srt[len(srt) // 2],
               "elapsed_ms_at_launch": [round(sum(us[:i]) / 1e3, 2) for i in (8, 20, len(us) - 40)]}
        print(json.dumps(rec), flush=True)

    count = max(60, args.steps)
    m, n, g = 512, 131072, 64
    A = torch.from_numpy(si.activations(m, 2048, si.seed_of("cfg3", "a", m, 2048))
                         .view("int16")).view(torch.bfloat16).to(dev)
    w = Weights(torch, qg, si, n, 2048, g, "cfg3", 2, bias=True)
    C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def call(i):
        B, S, Z = w[i]
        qg.gemm_w4a16(A, B, S, Z, w.bias, g, out=C)
    summary("prefill W4A16 M=512 N=131072 K=2048 g64, fp16 bias", series(call, count))
    del w, C
    T, H, I, E, TK, G = 2048, 2048, 1408, 64, 6, 64
    p = si.moe_problem(T, H, I, E, TK, G, tag="cfg4")

    def up16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    x, lg = up16(p.x), torch.from_numpy(p.logits).to(dev)
    w1 = torch.stack([qg.repack_w4(torch.from_numpy(p.w1[e]).to(dev)) for e in range(E)])
    w2 = torch.stack([qg.repack_w4(torch.from_numpy(p.w2[e]).to(dev)) for e in range(E)])
    s1, z1, s2, z2 = (up16(a) for a in (p.s1, p.z1, p.s2, p.z2))
    ws = torch.empty(qg.moe_workspace_size(T, H, I, E, TK), dtype=torch.uint8, device=dev)
    summary("MoE T=2048 H=2048 I=1408 E=64 top-6 g64",
            series(lambda i: qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, TK, G, workspace=ws), count))


def kernel_only(args, torch, qg, si):
    """Only the chosen legs, each `--steps` times, for rocprofv3 counter runs:
    decode -- the N=131072 M=1 GEMV; prefill -- the M=512 N=131072 g=64 GEMM
    (fp16 bias); copy -- a plain copy kernel over 512 MiB three times (torch's
    elementwise negation: reads 512 MiB, writes 512 MiB, in full cache lines),
    calibrating FETCH_SIZE / WRITE_SIZE; decode_small -- the M=1 GEMVs at
    N=2048, 3072, 13312; w8 -- W8A16 K=3584 N=18944 at M=1 and M=4096; w8a8 --
    W8A8 K=3584 N=18944 at M=1 and M=4096; moe -- the 2048-token MoE."""
    dev = "cuda"
    legs = args.kernel_only.split(",")
    bad = [x for x in legs if x not in KERNEL_LEGS]
    if bad:
        raise SystemExit(f"unknown --kernel-only legs {bad}; choose from {KERNEL_LEGS}")

    def act(m, k, tag, dt=torch.bfloat16, code=None):
        bits = si.activations(m, k, si.seed_of(tag, "a", m, k), code if code else si.BF16)
        return torch.from_numpy(bits.view("int16")).view(dt).to(dev)
    if "decode" in legs:
        n = 131072
        w = Weights(torch, qg, si, n, DECODE_K, DECODE_G, "cfg1",
                    copies_for(w4_bytes(1, n, DECODE_K, DECODE_G)))
        A = act(1, DECODE_K, "cfg1")
        C = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
        for i in range(args.steps):
            B, S, Z = w[i]
            qg.gemm_w4a16(A, B, S, Z, None, DECODE_G, out=C)
        del w, C
    if "prefill" in legs:
        pm, pn, pg = PREFILL_TRAFFIC_SHAPE
        wp = Weights(torch, qg, si, pn, 2048, pg, "cfg3", 2, bias=True)
        Ap = act(pm, 2048, "cfg3")
        Cp = torch.empty((pm, pn), dtype=torch.bfloat16, device=dev)
        for i in range(args.steps):
            B, S, Z = wp[i]
            qg.gemm_w4a16(Ap, B, S, Z, wp.bias, pg, out=Cp)
        del wp, Cp
    if "decode_small" in legs:
        A = act(1, DECODE_K, "cfg1")
        for n in DECODE_N[:3]:
            w = Weights(torch, qg, si, n, DECODE_K, DECODE_G, "cfg1",
                        copies_for(w4_bytes(1, n, DECODE_K, DECODE_G)))
            C = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
            for i in range(args.steps):
                B, S, Z = w[i]
                qg.gemm_w4a16(A, B, S, Z, None, DECODE_G, out=C)
            del w, C
    if "w8" in legs:
        k8, n = 3584, 18944
        codes, sc, _ = si.w8_weights(n, k8, -1, si.seed_of("cfg2", "w", n, k8, -1))
        B = qg.repack_w8(torch.from_numpy(codes).to(dev))
        S = torch.from_numpy(sc.view("int16")).view(torch.float16).to(dev)
        sets = [(B, S)] + [(B.clone(), S.clone()) for _ in range(copies_for(n * k8) - 1)]
        for m in (1, 4096):
            A = act(m, k8, "cfg2", torch.float16, si.FP16)
            C = torch.empty((m, n), dtype=torch.float16, device=dev)
            for i in range(args.steps):
                B_, S_ = sets[i % len(sets)]
                qg.gemm_w8a16(A, B_, S_, None, -1, out=C)
        del sets, B
    if "w8a8" in legs:
        ka, n = 3584, 18944
        for m in (1, 4096):
            pa = si.w8a8_problem(m, n, ka, True, True, tag="w8a8-bench")
            A, B = torch.from_numpy(pa.A).to(dev), torch.from_numpy(pa.B).to(dev)
            row, col = torch.from_numpy(pa.alpha_row).to(dev), torch.from_numpy(pa.alpha_col).to(dev)
            C = torch.empty((m, n), dtype=torch.float16, device=dev)
            need = qg.w8a8_workspace_size(m, n, ka)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            for i in range(args.steps):
                qg.gemm_w8a8(A, B, row, col, out=C, workspace=ws)
    if "moe" in legs:
        T, H, I, E, TK, G = 2048, 2048, 1408, 64, 6, 64
        p = si.moe_problem(T, H, I, E, TK, G, tag="cfg4")

        def up16(a):
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        w1 = torch.stack([qg.repack_w4(torch.from_numpy(p.w1[e]).to(dev)) for e in range(E)])
        w2 = torch.stack([qg.repack_w4(torch.from_numpy(p.w2[e]).to(dev)) for e in range(E)])
        s1, z1, s2, z2 = (up16(a) for a in (p.s1, p.z1, p.s2, p.z2))
        x, lg = up16(p.x), torch.from_numpy(p.logits).to(dev)
        ws = torch.empty(qg.moe_workspace_size(T, H, I, E, TK), dtype=torch.uint8, device=dev)
        for i in range(args.steps):
            qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, TK, G, workspace=ws)
    if "copy" in legs:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"kernel-only: legs {legs}, {args.steps} calls each")


def counter_summary(path):
    """Per-kernel means of every counter in a rocprofv3 counter collection
    (`rocprofv3 --pmc ... --output-format csv`, run_counter_collection.csv),
    for the library's kernels and the calibration copy, as a markdown table."""
    import csv
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if "qg::" not in name and "neg_kernel" not in name and "AUnaryFunctor" not in name:
                continue
            key = (name, int(row.get("Grid_Size", row.get("Grid_Size_X", 0)) or 0))
            d = vals.setdefault(key, {})
            d.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    counters = sorted({c for d in vals.values() for c in d})
    out = ["| kernel | grid threads | dispatches | " + " | ".join(counters) + " |",
           "|---|---:|---:|" + "---:|" * len(counters)]
    for (name, grid), d in sorted(vals.items()):
        n = max(len(v) for v in d.values())
        cells = [f"{sum(d[c]) / len(d[c]):,.0f}" if c in d else "" for c in counters]
        short = name if len(name) <= 100 else name[:97] + "..."
        out.append(f"| `{short}` | {grid} | {n} | " + " | ".join(cells) + " |")
    return "\n".join(out)


def trace_summary(path, top=60):
    """Per-dispatch statistics from a rocprofv3 kernel trace (CSV from
    `rocprofv3 --kernel-trace --output-format csv`): for each library kernel
    and launch shape (grid and workgroup size) the dispatch count and the
    median, 10th and 90th percentile, mean, min and max duration in us, as a
    markdown table, sorted by total time."""
    import csv
    import statistics
    groups = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if not name.lstrip("void ").startswith("qg::"):
                continue
            key = (name, int(row["Grid_Size_X"]), int(row["Workgroup_Size_X"]))
            us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append(us)

    def pct(xs, q):
        xs = sorted(xs)
        i = q * (len(xs) - 1)
        lo = int(math.floor(i))
        hi = min(lo + 1, len(xs) - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    out = ["| dispatches | median us | p10 us | p90 us | mean us | min us | max us | grid threads | wg | kernel |",
           "|---:|---:|---:|---:|---:|---:|---:|---:|---:|---|"]
    for (name, grid, wg), xs in rows:
        short = name if len(name) <= 110 else name[:107] + "..."
        out.append(f"| {len(xs)} | {statistics.median(xs):.2f} | {pct(xs, 0.1):.2f} | {pct(xs, 0.9):.2f} | "
                   f"{statistics.fmean(xs):.2f} | {min(xs):.2f} | {max(xs):.2f} | {grid} | {wg} | `{short}` |")
    return "\n".join(out)


def host_cpu():
    """Model name, sockets and logical CPUs of this host (from /proc/cpuinfo)
    and the CPUs this process may run on."""
    model, sockets, logical = "unknown", set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model == "unknown":
                    model = v
                elif k == "physical id":
                    sockets.add(v)
                elif k == "processor":
                    logical += 1
    except OSError:
        pass
    return {"model": model, "sockets": max(1, len(sockets)), "logical_cpus": logical,
            "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(args, si, step_bytes):
    """The oracle (oracle/qref.c, as written) on bounded samples of the
    workloads, on this host's cores.  The timed GEMMs are the oracle's
    fp32-accumulating variant; the thread count is set inside the oracle
    library (omp_set_num_threads) and `cores` is the team size a parallel
    region of it actually got."""
    import oracle
    oracle.lib()
    host = host_cpu()
    nthr = host["affinity_cpus"]
    oracle.set_threads(nthr)
    team = oracle.team_size()

    def rate(fn, min_s):
        fn()
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return n, dt

    # headline: whole M=1 decode steps (every N), GB/s of algorithmic bytes
    probs = []
    for n in DECODE_N:
        packed, sc, ze, _ = si.w4_weights(n, DECODE_K, DECODE_G,
                                          si.seed_of("cfg1", "w", n, DECODE_K, DECODE_G))
        probs.append((packed, sc, ze))
    A1 = si.activations(1, DECODE_K, si.seed_of("cfg1", "a", 1, DECODE_K))
    def step():
        for (packed, sc, ze) in probs:
            oracle.gemm_w4_f32acc(A1, packed, sc, ze, DECODE_G)
    passes, dt = rate(step, args.cpu_seconds)
    cpu = {"value": round(passes * step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": team,
           "kind": "oracle",
           "sample": f"{passes} full M=1 decode steps (N={DECODE_N}, K=2048, g=64) in {dt:.1f} s, "
                     f"fp32-accumulating oracle GEMM, {team} OpenMP threads",
           "host": host}

    # one thread: the two smallest decode GEMVs, and the tiny config
    oracle.set_threads(1)
    team1 = oracle.team_size()
    small = [(2048, probs[0]), (3072, probs[1])]
    b_small = sum(w4_bytes(1, n, DECODE_K, DECODE_G) for n, _ in small)
    passes1, dt1 = rate(lambda: [oracle.gemm_w4_f32acc(A1, *pp, DECODE_G) for _, pp in small], 3.0)
    p0 = si.w4_problem(4, 128, 256, 64, tag="cfg0")
    n0, dt0 = rate(lambda: oracle.gemm_w4_f32acc(p0.A, p0.packed, p0.scale, p0.zero, 64), 0.5)
    cpu["single_thread"] = {"value": round(passes1 * b_small / dt1 / 1e9, 4), "unit": "GB/s",
                            "cores": team1,
                            "sample": f"M=1 GEMVs N in {{2048, 3072}}, K=2048, g=64, {dt1:.1f} s"}
    cpu["tiny_single_thread"] = {"value": round(n0 * 2 * 4 * 128 * 256 / dt0 / 1e9, 4),
                                 "unit": "GFLOP/s", "cores": team1,
                                 "sample": "W4A16 M=4, K=256, N=128, g=64 (the tiny config)"}
    oracle.set_threads(nthr)

    # beside the GPU's other sections, on all threads
    p3 = si.w4_problem(512, 3072, 2048, 64, tag="cfg3", bias_dtype=si.FP16)
    n3, dt3 = rate(lambda: oracle.gemm_w4_f32acc(p3.A, p3.packed, p3.scale, p3.zero, 64, si.BF16,
                                            p3.bias, si.FP16), 1.0)
    p2 = si.w8_problem(128, 3584, 3584, -1, tag="cfg2")
    n2, dt2 = rate(lambda: oracle.gemm_w8_f32acc(p2.A, p2.codes, p2.scale, -1, si.FP16), 1.0)
    pm = si.moe_problem(2048, 2048, 1408, 64, 6, 64, tag="cfg4")
    import numpy as np
    toks = np.arange(16)
    t0 = time.perf_counter()
    oracle.moe(pm.x, pm.logits, pm.w1, pm.s1, pm.z1, pm.w2, pm.s2, pm.z2, 6, 64, tokens=toks)
    dtm = time.perf_counter() - t0
    moe_flop = 2.0 * len(toks) * 6 * (2 * 1408 * 2048 + 2048 * 1408)
    cpu["configs"] = {
        "prefill_M512_N3072_g64": {"value": round(n3 * 2.0 * 512 * 3072 * 2048 / dt3 / 1e9, 2),
                                   "unit": "GFLOP/s", "cores": team,
                                   "sample": f"{n3} GEMMs in {dt3:.1f} s, fp32 accumulation"},
        "w8a16_M128_N3584_K3584": {"value": round(n2 * 2.0 * 128 * 3584 * 3584 / dt2 / 1e9, 2),
                                   "unit": "GFLOP/s", "cores": team,
                                   "sample": f"{n2} GEMMs in {dt2:.1f} s, fp32 accumulation"},
        "moe_T2048_16_tokens": {"value": round(moe_flop / dtm / 1e9, 2), "unit": "GFLOP/s",
                                "cores": team,
                                "sample": f"16 of the 2048 tokens (routing of all) in {dtm:.1f} s, "
                                          "fp64 oracle, expert weights dequantized once"},
    }
    return cpu


def run(args):
    import torch

    import synth_inputs as si
    import weight_only_quantized_w8a16_amd as qg

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (HIP device)")
    torch.cuda.init()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({props.gcnArchName}), CUs {props.multi_processor_count}")
    if args.kernel_only:
        kernel_only(args, torch, qg, si)
        return
    if args.launch_series:
        launch_series(args, torch, qg, si)
        return

    # ---- decode workload ------------------------------------------------------
    t0 = time.time()
    decode_w = {}
    for n in DECODE_N:
        b = w4_bytes(1, n, DECODE_K, DECODE_G)
        decode_w[n] = Weights(torch, qg, si, n, DECODE_K, DECODE_G, "cfg1", copies_for(b))
    acts = {m: torch.from_numpy(si.activations(m, DECODE_K, si.seed_of("cfg1", "a", m, DECODE_K))
                                .view("int16")).view(torch.bfloat16).to(dev) for m in (1, 2, 4, 8)}
    outs = {(m, n): torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for (m, n) in SWEEP + [(1, n) for n in DECODE_N]}
    torch.cuda.synchronize()
    log(f"decode inputs ready in {time.time() - t0:.1f}s "
        f"({sum(len(w.sets) for w in decode_w.values())} weight copies)")

    def gemv(m, n, i):
        B, S, Z = decode_w[n][i]
        qg.gemm_w4a16(acts[m], B, S, Z, None, DECODE_G, out=outs[(m, n)])

    # warmup
    for i in range(args.warmup):
        for n in DECODE_N:
            gemv(1, n, i)
    torch.cuda.synchronize()

    # Timed region: K steps, each one GEMV per shape, back to back on torch's
    # current stream (the stream the library launches on), bracketed by two
    # HIP events.  A GPU-side wait queued first lets the host run ahead, so
    # the region holds no host gaps.
    stream = torch.cuda.current_stream()
    K = args.steps

    def timed(fn, reps, calls_per_rep=1, warm=0):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # the lead outlasts the host's enqueue time (generously 0.2 ms a call,
        # at most 300 ms); `warm` untimed calls run right before the start
        # event, so the timed calls find the clocks already up.
        gpu_lead(torch, min(300.0, 2.0 + 0.2 * (reps + warm) * calls_per_rep))
        for i in range(warm):
            fn(i)
        a.record(stream)
        for i in range(reps):
            fn(warm + i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def steady(fn, reps, calls_per_rep=1):
        """Mean ms per call of `fn` at the chip's sustained clock.  Under
        back-to-back compute-bound launches the power controller first lets
        the clock run high (a few ms), then pulls it well below its sustained
        level and lets it recover over the next 10-20 ms (the launch series of
        `--launch-series`); so `fn` first runs untimed for STEADY_WARM_MS,
        then at least `reps` calls spanning STEADY_MIN_MS are timed."""
        est = timed(fn, 3, calls_per_rep) / 3
        warm = min(1000, math.ceil(STEADY_WARM_MS / est))
        reps = max(reps, min(500, math.ceil(STEADY_MIN_MS / est)))
        return timed(fn, reps, calls_per_rep, warm=warm) / reps

    def step(i):
        for n in DECODE_N:
            gemv(1, n, args.warmup + i)

    h0 = time.perf_counter()
    # The W warm-up steps run again in-stream right before the start event
    # (the GPU is busy with them while the host enqueues the timed steps).
    region_ms = timed(step, K, len(DECODE_N), warm=args.warmup)
    host_s = time.perf_counter() - h0
    step_bytes = sum(w4_bytes(1, n, DECODE_K, DECODE_G) for n in DECODE_N)
    ms_per_step = region_ms / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # Per shape: the same launches, one shape at a time, back to back; the
    # mean launch time is the region over the launch count.
    per_shape, launch_ms = {}, {}
    for n in DECODE_N:
        ms = timed(lambda i, n=n: gemv(1, n, 3 * i + 1), K) / K
        b = w4_bytes(1, n, DECODE_K, DECODE_G)
        launch_ms[n] = ms
        per_shape[str(n)] = {"us": round(ms * 1e3, 2),
                             "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                             "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
    log(f"decode M=1 step: {ms_per_step * 1e3:.1f} us on the device clock "
        f"({host_s / K * 1e6:.0f} us host incl. the lead), {value:.0f} GB/s; "
        f"per shape {per_shape}")

    lm_ms = launch_ms[131072]
    lm_bytes = w4_bytes(1, 131072, DECODE_K, DECODE_G)
    achieved = lm_bytes / (lm_ms * 1e-3) / 1e9
    traffic = load_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "k_decode_w4_stream (M=1, N=131072, K=2048, g=64)",
                "bytes_per_launch": lm_bytes, "mean_launch_us": round(lm_ms * 1e3, 2)}

    # ---- full decode sweep (M = 1, 2, 4, 8) -----------------------------------
    sweep = {}
    if not args.quick:
        reps = max(10, K // 2)
        for (m, n) in SWEEP:
            ms = timed(lambda i, m=m, n=n: gemv(m, n, 7 * i + m), reps) / reps
            b = w4_bytes(m, n, DECODE_K, DECODE_G)
            sweep[f"M{m}_N{n}"] = {"us": round(ms * 1e3, 2),
                                   "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                   "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
        log(f"decode sweep: {sweep}")
    del decode_w
    torch.cuda.empty_cache()

    # ---- prefill M=512 ------------------------------------------------------------
    prefill = None
    if not args.no_prefill:
        acts_p = {m: torch.from_numpy(si.activations(m, 2048, si.seed_of("cfg3", "a", m, 2048))
                                      .view("int16")).view(torch.bfloat16).to(dev) for m in (512, 2048)}
        shapes = {}
        tot_flop, tot_ms = 0.0, 0.0
        for (m, n, g) in PREFILL + ([] if args.quick else PREFILL_2048):
            A = acts_p[m]
            w = Weights(torch, qg, si, n, 2048, g, "cfg3", 2, bias=True)
            C = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            for i in range(3):
                B, S, Z = w[i]
                qg.gemm_w4a16(A, B, S, Z, w.bias, g, out=C)
            reps = max(10, K // 2) if m == 512 else max(5, K // 10)

            def call(i, w=w, C=C, g=g, A=A):
                B, S, Z = w[i]
                qg.gemm_w4a16(A, B, S, Z, w.bias, g, out=C)
            ms = steady(call, reps)
            flop = 2.0 * m * n * 2048
            if m == 512:
                tot_flop += flop
                tot_ms += ms
            key = f"N{n}_g{g}" if m == 512 else f"M{m}_N{n}_g{g}"
            shapes[key] = {"us": round(ms * 1e3, 1),
                           "TFLOPS": round(flop / (ms * 1e-3) / 1e12, 1),
                           "frac": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 3)}
            del w, C
        tf = tot_flop / (tot_ms * 1e-3) / 1e12
        pm, pn, pg = PREFILL_TRAFFIC_SHAPE
        prefill = {"metric": "prefill TFLOPS at M=512 (W4A16, K=2048, fp16 bias); M=2048 shapes "
                             "reported beside it",
                   "value": round(tf, 1), "unit": "TFLOP/s",
                   "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                "traffic": load_traffic("traffic_prefill_w4_m512_n131072.json",
                                                        PREFILL_SOURCES),
                                "traffic_kernel": f"k_prefill_dma (M={pm}, N={pn}, K=2048, g={pg})",
                                "bytes_per_launch": w4_bytes(pm, pn, 2048, pg, bias=True)},
                   "shapes": shapes}
        log(f"prefill: {prefill}")
        torch.cuda.empty_cache()

    # ---- MoE ------------------------------------------------------------------------
    moe = None
    if not args.no_moe:
        T, H, I, E, TK, G = 2048, 2048, 1408, 64, 6, 64
        p = si.moe_problem(T, H, I, E, TK, G, tag="cfg4")

        def up16(a):
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

        x = up16(p.x)
        lg = torch.from_numpy(p.logits).to(dev)
        w1 = torch.stack([qg.repack_w4(torch.from_numpy(p.w1[e]).to(dev)) for e in range(E)])
        w2 = torch.stack([qg.repack_w4(torch.from_numpy(p.w2[e]).to(dev)) for e in range(E)])
        s1, z1, s2, z2 = (up16(a) for a in (p.s1, p.z1, p.s2, p.z2))
        ws = torch.empty(qg.moe_workspace_size(T, H, I, E, TK), dtype=torch.uint8, device=dev)
        for _ in range(3):
            qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, TK, G, workspace=ws)
        reps = max(5, K // 5)
        ms = steady(lambda i: qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, TK, G, workspace=ws),
                    reps, 5)
        flop = 2.0 * T * TK * (2 * I * H + H * I)
        wbytes = E * (w4_bytes(0, 2 * I, H, G) + w4_bytes(0, H, I, G))
        moe = {"config": "T=2048 H=2048 I=1408 E=64 top-6 g=64", "us": round(ms * 1e3, 1),
               "TFLOPS": round(flop / (ms * 1e-3) / 1e12, 1),
               "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1)}
        log(f"moe: {moe}")
        del w1, w2, ws
        torch.cuda.empty_cache()

    # ---- W8A16 (int8 weights, fp16 activations), K = 3584 ----------------------------
    w8 = None
    if not args.no_w8:
        k8 = 3584
        w8shapes = {}
        for group in (-1, 128):
            for n in (3584, 18944):
                codes, sc, _ = si.w8_weights(n, k8, group, si.seed_of("cfg2", "w", n, k8, group))
                base = qg.repack_w8(torch.from_numpy(codes).to(dev))
                S = torch.from_numpy(sc.view("int16")).view(torch.float16).to(dev)
                wb = n * k8 + 2 * S.numel()
                copies = copies_for(wb)
                sets = [(base, S)] + [(base.clone(), S.clone()) for _ in range(copies - 1)]
                ms_list = (1, 16, 128, 1024, 4096) if group == -1 else (1, 16, 1024)
                for m in ms_list:
                    A = torch.from_numpy(si.activations(m, k8, si.seed_of("cfg2", "a", m, k8),
                                                        si.FP16).view("int16")).view(torch.float16).to(dev)
                    C = torch.empty((m, n), dtype=torch.float16, device=dev)
                    reps = max(10, K // 5)

                    def call(i, A=A, C=C, sets=sets, group=group):
                        B, S_ = sets[i % len(sets)]
                        qg.gemm_w8a16(A, B, S_, None, group, out=C)
                    for i in range(3):
                        call(i)
                    ms = steady(call, reps)
                    b = wb + 2 * m * k8 + 2 * m * n
                    flop = 2.0 * m * n * k8
                    w8shapes[f"g{group}_M{m}_N{n}"] = {
                        "us": round(ms * 1e3, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                        "TFLOPS": round(flop / (ms * 1e-3) / 1e12, 1),
                        "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                        "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 3)}
                    del A, C
                del sets, base
                torch.cuda.empty_cache()
        w8 = {"config": "W8A16, K=3584, N in {3584, 18944}, fp16 A/C, int8 codes; per-channel "
                        "scales (g-1) and group-128 scales (g128); GB/s against 8 TB/s for "
                        "small M, TFLOP/s against the 2.5 PFLOP/s fp16 peak for large M",
              "shapes": w8shapes}
        log(f"w8: {w8}")

    # ---- int4 scale forms: groupwise with zeros, scale-only, per channel ----------
    forms = None
    if not args.no_w8:
        fk, fn = 2048, 13312
        fshapes = {}
        for label, group, zeros in (("g64_zeros", 64, True), ("g64_scale_only", 64, False),
                                    ("per_channel_zeros", -1, True),
                                    ("per_channel_scale_only", -1, False)):
            packed, sc, ze, _ = si.w4_weights(fn, fk, group, si.seed_of("forms", "w", fn, fk, group))
            base = qg.repack_w4(torch.from_numpy(packed).to(dev))
            S = torch.from_numpy(sc.view("int16")).view(torch.bfloat16).to(dev)
            Z = torch.from_numpy(ze.view("int16")).view(torch.bfloat16).to(dev) if zeros else None
            wb = fn * fk // 2 + 2 * S.numel() * (2 if zeros else 1)
            copies = copies_for(wb)
            sets = [(base, S, Z)] + [(base.clone(), S.clone(), None if Z is None else Z.clone())
                                     for _ in range(copies - 1)]
            for m in (1, 512):
                A = torch.from_numpy(si.activations(m, fk, si.seed_of("forms", "a", m, fk))
                                     .view("int16")).view(torch.bfloat16).to(dev)
                C = torch.empty((m, fn), dtype=torch.bfloat16, device=dev)
                reps = max(10, K // 5)

                def call(i, A=A, C=C, sets=sets, group=group):
                    B, S_, Z_ = sets[i % len(sets)]
                    qg.gemm_w4a16(A, B, S_, Z_, None, group, out=C)
                for i in range(3):
                    call(i)
                ms = steady(call, reps)
                b = wb + 2 * m * fk + 2 * m * fn
                fshapes[f"{label}_M{m}"] = {"us": round(ms * 1e3, 2),
                                            "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                            "TFLOPS": round(2.0 * m * fn * fk / (ms * 1e-3) / 1e12, 1)}
                del A, C
            del sets, base
        forms = {"config": "W4A16 N=13312 K=2048 bf16, M in {1, 512}: groupwise g64 with zeros / "
                           "scale-only, per-channel with zeros / scale-only",
                 "shapes": fshapes}
        log(f"w4 forms: {forms}")
        torch.cuda.empty_cache()

    # ---- W8A8 (int8 x int8, per-token x per-channel scales), K = 3584 ------------------
    w8a8 = None
    if not args.no_w8a8:
        ka = 3584
        ashapes = {}
        for n in (3584, 18944):
            p0 = si.w8a8_problem(1, n, ka, True, True, tag="w8a8-bench")
            base = torch.from_numpy(p0.B).to(dev)
            col = torch.from_numpy(p0.alpha_col).to(dev)
            wb = n * ka + 4 * n
            copies = copies_for(wb)
            sets = [(base, col)] + [(base.clone(), col.clone()) for _ in range(copies - 1)]
            for m in (1, 16, 128, 1024, 4096):
                pa = si.w8a8_problem(m, n, ka, True, True, tag="w8a8-bench")
                A = torch.from_numpy(pa.A).to(dev)
                row = torch.from_numpy(pa.alpha_row).to(dev)
                C = torch.empty((m, n), dtype=torch.float16, device=dev)
                need = qg.w8a8_workspace_size(m, n, ka)
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
                reps = max(10, K // 5)

                def call(i, A=A, C=C, sets=sets, row=row, ws=ws):
                    B, col_ = sets[i % len(sets)]
                    qg.gemm_w8a8(A, B, row, col_, out=C, workspace=ws)
                for i in range(3):
                    call(i)
                ms = steady(call, reps)
                b = wb + m * ka + 4 * m + 2 * m * n
                ops = 2.0 * m * n * ka
                ashapes[f"M{m}_N{n}"] = {
                    "us": round(ms * 1e3, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                    "TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
                    "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                    "frac_mfma_i8": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 3),
                    "split_k_ws_bytes": need}
                del A, C, ws
            del sets, base
            torch.cuda.empty_cache()
        w8a8 = {"config": "W8A8 int8 x int8, K=3584, N in {3584, 18944}, per-token x "
                          "per-channel fp32 scales, fp16 C; GB/s against 8 TB/s for small M, "
                          "TOP/s against the 5.0 POP/s dense int8 peak for large M",
                "shapes": ashapes}
        log(f"w8a8: {w8a8}")

    # ---- embedding lookup from the tied vocab table ------------------------------------
    emb = None
    if not args.no_w8a8:
        vocab, hid, eg = 131072, 2048, 64
        packed, sc, ze, _ = si.w4_weights(vocab, hid, eg, si.seed_of("cfg1", "w", vocab, hid, eg))
        table = qg.repack_w4(torch.from_numpy(packed).to(dev))
        S = torch.from_numpy(sc.view("int16")).view(torch.bfloat16).to(dev)
        Z = torch.from_numpy(ze.view("int16")).view(torch.bfloat16).to(dev)
        eshapes = {}
        for T in (1, 64, 2048):
            gen = torch.Generator().manual_seed(T)
            ids = [torch.randint(0, vocab, (T,), generator=gen, dtype=torch.int32).to(dev)
                   for _ in range(8)]
            reps = max(10, K // 5)
            for i in range(3):
                qg.embed_w4(ids[i % 8], table, S, Z, eg)
            ms = timed(lambda i: qg.embed_w4(ids[i % 8], table, S, Z, eg), reps, warm=reps) / reps
            b = T * (hid // 2 + 4 * (hid // eg) + 4 + 2 * hid)
            eshapes[f"T{T}"] = {"us": round(ms * 1e3, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                "bytes": b}
        emb = {"config": "int4 embedding lookup from the tied 131072 x 2048 table (tiled, g64, "
                         "bf16 out), T random token ids", "shapes": eshapes}
        del table, S, Z
        log(f"embed: {emb}")

    # ---- load-side quantizer ------------------------------------------------------
    quant = None
    if not args.no_quant:
        qk, qgp = 2048, 64
        qshapes, best = {}, None
        for n in (13312, 131072):
            gen = torch.Generator(device=dev)
            gen.manual_seed(n)
            nbytes = n * qk * 2
            copies = max(1, min(16, math.ceil(ROTATE_BYTES / nbytes)))
            Ws = [(torch.randn(n, qk, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
                  for _ in range(copies)]
            for i in range(2):
                qg.quantize_w4(Ws[i % copies], qgp)
            reps = max(10, K // 5)
            ms = timed(lambda i: qg.quantize_w4(Ws[i % copies], qgp), reps, warm=reps) / reps
            b = nbytes + n * qk // 2 + 2 * 2 * n * (qk // qgp)
            gbps = b / (ms * 1e-3) / 1e9
            qshapes[f"N{n}"] = {"us": round(ms * 1e3, 1), "GBps": round(gbps, 1),
                                "frac": round(gbps / HBM_PEAK_GBS, 3), "bytes": b}
            best = (n, gbps, b, ms)
            del Ws
        n, gbps, b, ms = best
        quant = {"metric": "int4 groupwise min/max quantizer: bf16 W [N, 2048] -> portable "
                           "codes + bf16 scale/zero, group 64",
                 "shapes": qshapes,
                 "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                              "traffic": None, "kernel": f"k_quantize_w4 (N={n}, K=2048, g=64)",
                              "bytes_per_launch": b, "mean_launch_us": round(ms * 1e3, 2)}}
        log(f"quantize: {quant}")
        torch.cuda.empty_cache()

    # ---- ceiling: a plain device-to-device copy (read + write) ----------------------
    ceil = None
    if not args.quick:
        nbytes = 1 << 30
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i) for i in range(3)]
        reps = 10
        ms = timed(lambda i: bufs[(i + 1) % 3].copy_(bufs[i % 3]), reps) / reps
        ceil = {"copy_GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                "note": "torch device copy of 1 GiB, read + write bytes"}
        del bufs
        # Streaming-read probe over the decode step's byte counts (rotating
        # over 1 GiB of distinct bytes so nothing is served from the
        # Infinity Cache), and an empty launch: the read floor of each GEMV.
        big = torch.empty(ROTATE_BYTES + (256 << 20), dtype=torch.uint8, device=dev)
        outp = torch.empty(int(qg.lib().qg_read_probe_blocks(1 << 30)), dtype=torch.int32, device=dev)
        probe, floor_us = {}, 0.0
        for n in [0] + DECODE_N:
            b = w4_bytes(1, n, DECODE_K, DECODE_G) // 16 * 16 if n else 0
            slots = max(1, ROTATE_BYTES // max(b, 1)) if b else 1
            reps = max(20, K // 2)

            def call(i, b=b, slots=slots):
                off = (i % slots) * b
                qg.read_probe(big[off:off + b] if b else None, b, outp)
            for i in range(3):
                call(i)
            us = timed(call, reps, warm=reps) / reps * 1e3
            key = f"N{n}" if n else "empty_launch"
            probe[key] = {"us": round(us, 2), "bytes": b,
                          "GBps": round(b / (us * 1e-6) / 1e9, 1) if b else None}
            if n:
                floor_us += us
        ceil["read_probe"] = probe
        # LDS read bandwidth per CU (qg_lds_probe: one workgroup per CU, a
        # conflict-free 16-byte read loop timed by the shader clock): what the
        # prefill tiles' fragment reads draw on.
        lds = {}
        for waves in (4, 8, 16):
            cyc = torch.zeros(props.multi_processor_count, dtype=torch.int64, device=dev)
            iters = 4096
            for _ in range(3):
                qg.lds_probe(waves, iters, cyc)
            torch.cuda.synchronize()
            lds[f"waves{waves}"] = round(iters * waves * 1024 / float(cyc.double().median()), 1)
        ceil["lds_read_bytes_per_clock_per_cu"] = lds
        # The vendor library's plain dense GEMM on the prefill and W8A16 shapes
        # (torch.mm -> hipBLASLt; no dequantization, 16-bit weights, so four or
        # two times the weight bytes): what a tuned dense GEMM of these shapes
        # reaches on this chip.
        dense = {}
        for (m, n, k, dt) in ((512, 131072, 2048, torch.bfloat16), (2048, 131072, 2048, torch.bfloat16),
                              (512, 13312, 2048, torch.bfloat16), (4096, 18944, 3584, torch.float16)):
            gen = torch.Generator(device=dev)
            gen.manual_seed(m + n)
            Ad = torch.randn(m, k, generator=gen, device=dev).to(dt)
            Wt = torch.randn(k, n, generator=gen, device=dev).to(dt)   # [K, N], contiguous
            Cd = torch.empty(m, n, dtype=dt, device=dev)
            for _ in range(3):
                torch.mm(Ad, Wt, out=Cd)
            reps = 10 if m * n < 1e9 else 5
            ms = steady(lambda i: torch.mm(Ad, Wt, out=Cd), reps)
            tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            dense[f"M{m}_N{n}_K{k}_{'bf16' if dt == torch.bfloat16 else 'fp16'}"] = {
                "us": round(ms * 1e3, 1), "TFLOPS": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 3)}
            del Ad, Wt, Cd
        ceil["dense_gemm_torch_mm"] = dense
        ceil["read_floor_step_us"] = round(floor_us, 2)
        ceil["read_floor_step_GBps"] = round(step_bytes / (floor_us * 1e-6) / 1e9, 1)
        ceil["decode_step_vs_read_floor"] = round(floor_us / (ms_per_step * 1e3), 3)
        # the headline kernel against a plain read of the same bytes
        pr = probe[f"N{DECODE_N[-1]}"]["GBps"]
        roofline["read_probe_GBps"] = pr
        roofline["frac_of_read_probe"] = round(roofline["achieved"] / pr, 3)
        del big, outp
        torch.cuda.empty_cache()
        log(f"ceiling: {ceil}")

    # ---- CPU oracle baseline -----------------------------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, si, step_bytes)
        log(f"cpu baseline: {cpu}")

    result = {
        "metric": "decode GEMV HBM GB/s (% of peak) at M=1; prefill TFLOPS (% MFMA peak) at M=512",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "config": {"workload": "W4A16 decode GEMV, M=1, K=2048, group 64, bf16 in/out, "
                               "N in {2048, 3072, 13312, 131072}",
                   "global_batch": 1, "parallelism": "none (one GPU)",
                   "weights_rotated_bytes": ROTATE_BYTES},
        "per_shape": per_shape,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "prefill": prefill,
        "moe": moe,
        "w8": w8,
        "w4_forms": forms,
        "w8a8": w8a8,
        "embed": emb,
        "quantize": quant,
        "ceiling": ceil,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-quant", action="store_true")
    ap.add_argument("--no-w8", action="store_true")
    ap.add_argument("--no-w8a8", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the M sweep and the copy ceiling")
    ap.add_argument("--kernel-only", metavar="LEGS", nargs="?", const="decode,prefill,copy",
                    help="run only the comma-separated legs (" + ",".join(KERNEL_LEGS) + "; "
                         "default decode,prefill,copy), --steps calls each, for profiler "
                         "counter runs; prints no result line")
    ap.add_argument("--launch-series", action="store_true",
                    help="print per-launch durations of --steps back-to-back prefill (M=512, "
                         "N=131072) and MoE calls, then exit")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="print per-kernel counter means of a rocprofv3 counter collection and exit")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-dispatch statistics of a rocprofv3 kernel trace and exit")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; there is no multi-GPU path to run "
              "(the GEMM shards along N without communication, so one GPU's shard is the "
              "kernel measured here). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
