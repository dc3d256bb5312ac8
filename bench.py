#!/usr/bin/env python3
"""Benchmark of the attention forward (libmi355_attn) on one MI355X.

One step = one attn_fwd call over the headline workload: bf16 B=4, H=16,
M=N=4096, D=128, non-causal (the long-sequence configuration whose MFMA
roofline target is stated; the pages' own bench shapes are bf16 long-context
tensors of this kind). Inputs are seeded synthetic N(0,1) draws rounded to
bf16, resident in HBM before timing starts; outputs are preallocated.

Prints ONE JSON line with the metric (TFLOP/s with 4*B*H*M*N*D FLOPs, halved
when causal), the roofline of the dominant kernel, the CPU oracle's rate on a
bounded sample of the same workload, and the other workloads (fp32 single
head, fp32 batch-96 non-causal / causal, the two axial passes with a
same-bytes device copy beside them, bf16 causal 8192, the Blackwell example's
two bench shapes, the headline shape in fp16, the fused axial-attention block
and its two passes, the fp32 batch and the long bf16 shape with a value head dim
of its own (Dv = 64 beside D = 128), and the backward at three bf16 shapes and the fp16 one,
10*B*H*M*N*D FLOPs) as additional measurements. Every measurement times 7
windows of its steps: the first is the reported figure, all seven give the
median and minimum per call ("repeat"). The single-head fp32 problem and the
axial passes are also timed cold, cycling through more independent buffer
sets than the Infinity Cache and L2 hold ("cold_us_per_call").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                       [--no-cpu-baseline] [--workload c4]
"""
from __future__ import annotations

import argparse
import statistics
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 / fp16 MFMA
PEAK_FP32_TFLOPS = 157.3    # fp32 (vector and MFMA)
PEAK_HBM_GBS = 8000.0       # HBM3E
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 (e4m3) MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--axial-only", action="store_true",
                    help="only time the fused axial block and its passes (for profiling)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time attn_bwd on --workload (16-bit workloads; for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times "
                         "(reference reading for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 5}))


# What the 16-bit forward kernel is built from: its source, the device header
# it includes and its hipcc flags. The counter summaries are tied to this.
TRAFFIC_KERNEL_SOURCES = ("attn_fwd_bf16.hip", "attn_device.h")


def kernel_source_hash() -> str:
    import hashlib
    from scaled_dot_product_12_amd import build as B
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_12_amd", "csrc")
    for f in TRAFFIC_KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    flags = B.COMMON + B.KERNEL_FLAGS + B.SOURCE_FLAGS.get(TRAFFIC_KERNEL_SOURCES[0], [])
    h.update(" ".join(flags).replace(ROOT, "").encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this workload or the kernels have changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# Timed windows per measurement: the first is the reported figure (exactly
# the requested steps); all of them give the median and the minimum.
REPS = 7


def time_launches(fn, steps, warmup, graph=False, spin_s=1.0, reps=REPS):
    """Average GPU time per call (ms) with HIP events on the launch stream,
    over the first timed window of `steps` calls, the wall time of that
    window, and {median_us, min_us} per call over `reps` such windows.
    graph=True captures the calls in one HIP graph first (for microsecond
    kernels whose Python launch cost would otherwise leave the GPU idle)."""
    import torch
    stream = torch.cuda.current_stream()
    # Spin the GPU up to its sustained clock before the warmup proper, so the
    # timed steps do not include the power-state ramp.
    t_end = time.perf_counter() + spin_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    fn()
        torch.cuda.synchronize()
        g.replay()  # warm the graph
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            for _ in range(steps):
                fn()
    per_call, wall = [], None
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        run()
        end.record(stream)
        torch.cuda.synchronize()
        if wall is None:
            wall = time.perf_counter() - t0
        per_call.append(start.elapsed_time(end) / steps)
    stats = {"median_us": round(statistics.median(per_call) * 1e3, 3),
             "min_us": round(min(per_call) * 1e3, 3), "windows": reps}
    return per_call[0], wall, stats


def gpu_setup(w):
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import workload_inputs
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def fn():
        attn.attn_fwd(q, k, v, is_causal=w.causal, scale=w.scale, out=(o, lse))
    return fn, (q, k, v, o, lse)


# Host threads for the CPU oracle: every core this process may use, capped
# at the 16-core share that goes with one GPU.
CPU_THREADS_CAP = 16


def cpu_baseline(w, target_s):
    """The oracle as it is, on the host cores, over a bounded row sample of
    the same workload (rows evenly spaced inside a seeded choice of heads);
    rate scaled to TFLOP/s with the same FLOP count per row (4*N_visible*D),
    so causal rows count their visible keys only."""
    import oracle
    from scaled_dot_product_12_amd.inputs import workload_inputs
    q, k, v = workload_inputs(w)
    B, H, M, D = q.shape
    N = k.shape[2]
    rng = np.random.default_rng(7)
    cores = min(oracle.host_threads(), CPU_THREADS_CAP)
    heads = [(b, h) for b in range(B) for h in range(H)]
    rng.shuffle(heads)

    def sample(n):
        n = max(1, min(n, B * H * M))
        n_heads = min(len(heads), max(1, -(-n // M)))
        per = -(-n // n_heads)
        rows = []
        for b, h in heads[:n_heads]:
            for i in np.unique(np.linspace(0, M - 1, min(per, M)).astype(int)):
                rows.append((b, h, int(i)))
        return rows[:n]

    def flops(rows):
        return sum(4.0 * (min(i + 1, N) if w.causal else N) * D for _, _, i in rows)

    # Size the sample from a short run, then re-size (at most twice) until a
    # run takes at least half the target; the last run is the one reported.
    rows = sample(max(cores * 64, 512))
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, rows, is_causal=w.causal, scale=w.scale, nthreads=cores)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or len(rows) >= B * H * M:
            break
        per_row_s = dt / len(rows)
        rows = sample(int(target_s / max(per_row_s, 1e-12)))
    n_heads = len({(b, h) for b, h, _ in rows})
    return {"value": round(flops(rows) / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} query rows of {w.describe()} ({n_heads} heads, rows evenly "
                      f"spaced in each), fp64, {dt:.1f} s wall"}


def bwd_flops(w) -> float:
    """Backward FLOPs: five products of 2*B*H*M*N*D each (QK^T, dO V^T, P^T dO,
    dS^T Q, dS K), i.e. 2.5x the forward's count; halved when causal."""
    f = 10.0 * w.B * w.H * w.M * w.N * w.D
    return f / 2 if w.causal else f


def measure_bwd(w, steps, warmup, one_pass=True):
    """Average time of one attn_bwd call on the workload's tensors, with the
    forward's O and L and a seeded dO: the one-pass path (delta kernel + fused
    kernel, work area allocated beforehand) where it applies and one_pass is
    set, else the two kernels (dQ kernel + dK/dV kernel). Returns the path
    taken too."""
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import make_dout
    fn_fwd, (q, k, v, o, lse) = gpu_setup(w)
    fn_fwd()
    g = make_dout(w.B, w.H, w.M, w.D, w.dtype, w.seed).to(q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    code = attn.MI355_ATTN_FP16 if w.dtype == "fp16" else attn.MI355_ATTN_BF16
    need = attn.attn_bwd_work_bytes(w.B, w.H, w.M, w.N, w.D, w.causal, code) if one_pass else 0
    work = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None

    def fn():
        attn.attn_bwd(q, k, v, o, lse, g, is_causal=w.causal, scale=w.scale,
                      out=(dq, dk, dv), delta=delta, one_pass=one_pass, work=work)
    ms, _, st = time_launches(fn, steps, warmup)
    path = "one pass (delta + fused kernel)" if need else "two kernels (dQ, dK/dV)"
    return ms, bwd_flops(w) / (ms * 1e-3) / 1e12, st, path


def measure(w, steps, warmup, graph):
    fn, tensors = gpu_setup(w)
    ms, wall, st = time_launches(fn, steps, warmup, graph=graph)
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
    return ms, wall, tflops, gbs, tensors, st


def same_bytes_copy_us(nbytes: int, steps: int = 200) -> float:
    """Time per call of a plain device copy (torch copy_) that reads and
    writes nbytes / 2 each, i.e. moves the same total bytes as a kernel with
    nbytes of algorithmic traffic: the practical floor for a microsecond
    launch of that size (HIP graph of `steps` calls, like the small
    workloads)."""
    import torch
    n = max(1, nbytes // 8)  # fp32 elements per direction
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms, _, _ = time_launches(lambda: dst.copy_(src), steps, 3, graph=True)
    return ms * 1e3


def same_bytes_copy_cold_us(nbytes: int, min_calls: int = 200) -> float:
    """same_bytes_copy_us with cold caches: the copies cycle through
    independent source/destination pairs totalling more than COLD_BYTES
    (HIP graph), like measure_cold does for the attention calls."""
    import torch
    n = max(1, nbytes // 8)
    nsets = max(2, -(-COLD_BYTES // (8 * n)))
    pairs = [(torch.ones(n, dtype=torch.float32, device="cuda:0"),
              torch.empty(n, dtype=torch.float32, device="cuda:0")) for _ in range(nsets)]
    state = {"i": 0}

    def fn():
        src, dst = pairs[state["i"] % nsets]
        state["i"] += 1
        dst.copy_(src)
    calls = nsets * max(1, -(-min_calls // nsets))
    ms, _, _ = time_launches(fn, calls, 3, graph=True, spin_s=0.2, reps=3)
    del pairs
    torch.cuda.empty_cache()
    return ms * 1e3


# Bytes one pass over the cold-timing buffer sets must touch: more than the
# 256 MB Infinity Cache plus the 8 x 4 MB of L2, so every call finds its
# inputs evicted.
COLD_BYTES = 320 * 10**6


def measure_cold(w, min_calls: int = 200):
    """Per-call time with cold caches: the calls cycle through independent
    input/output buffer sets (copies of the workload's tensors) whose total
    size exceeds the caches, inside one HIP graph. Returns (us, sets)."""
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import workload_inputs
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    nsets = max(2, -(-COLD_BYTES // w.algorithmic_bytes()))
    sets = []
    for _ in range(nsets):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        sets.append((q.clone(), k.clone(), v.clone(), o, lse))
    state = {"i": 0}

    def fn():
        sq, sk, sv, so, sl = sets[state["i"] % nsets]
        state["i"] += 1
        attn.attn_fwd(sq, sk, sv, is_causal=w.causal, scale=w.scale, out=(so, sl))
    calls = nsets * max(1, -(-min_calls // nsets))
    ms, _, st = time_launches(fn, calls, 3, graph=True, spin_s=0.2, reps=3)
    del sets
    torch.cuda.empty_cache()
    return ms * 1e3, nsets, st


def measure_fp8(steps: int = 30):
    """The long-sequence shape with fp8 (e4m3) inputs through attn_fwd_fp8 (V
    transposed, P rounded to fp8 for the second product, bf16 O): FLOPs
    4*B*H*M*N*D against the 5.0 PF dense fp8 peak."""
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["c4f8"]
    dev = torch.device("cuda:0")
    q, k, v = workload_inputs(w)
    qd, kd = q.to(dev), k.to(dev)
    vtd = v.transpose(-1, -2).contiguous().to(dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def fn():
        attn.attn_fwd_fp8(qd, kd, vtd, is_causal=w.causal, scale=w.scale, out=(o, lse))
    ms, _, st = time_launches(fn, steps, 3)
    tf = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
    return {"c4f8": {"workload": w.describe() + " (vt transposed, bf16 O)",
                     "us_per_call": round(ms * 1e3, 3), "tflops": round(tf, 3),
                     "frac_compute_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "peak_tflops": PEAK_FP8_TFLOPS, "gbs": round(gbs, 1),
                     "timing": "%d calls" % steps, "repeat": st}}


def measure_dv(steps: int = 30):
    """Attention with a value head dim of its own, Dv = 64 beside D = 128: on
    the Thunder notebook's fp32 batch (96 x 512 x 512) and on the
    long-sequence bf16 shape (4 x 16 x 4096 x 4096). FLOPs
    2*B*H*M*N*(D + Dv); algorithmic bytes Q, K, V, O and L once."""
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import make_qkv
    dev = torch.device("cuda:0")
    res = {}
    for name, dtype, (B, H, M, N), seeds in (("dv_c2", "fp32", (96, 1, 512, 512), (2, 3)),
                                            ("dv_c4", "bf16", (4, 16, 4096, 4096), (4, 5))):
        D, Dv = 128, 64
        q, k, _ = (t.to(dev) for t in make_qkv(B, H, M, N, D, dtype, seed=seeds[0]))
        v = make_qkv(B, H, M, N, Dv, dtype, seed=seeds[1])[2].to(dev)
        o = torch.empty((B, H, M, Dv), dtype=q.dtype, device=dev)
        lse = torch.empty((B, H, M), dtype=torch.float32, device=dev)
        ms, _, st = time_launches(lambda: attn.attn_fwd(q, k, v, out=(o, lse)), steps, 3)
        es = q.element_size()
        flops = 2 * B * H * M * N * (D + Dv)
        nbytes = es * B * H * (M * D + N * D + N * Dv + M * Dv) + 4 * B * H * M
        tf = flops / (ms * 1e-3) / 1e12
        peak = PEAK_FP32_TFLOPS if dtype == "fp32" else PEAK_BF16_TFLOPS
        res[name] = {
            "workload": f"{dtype} B={B} H={H} M={M} N={N} D={D} Dv={Dv} non-causal "
                        "(value head dim of its own)",
            "us_per_call": round(ms * 1e3, 3), "tflops": round(tf, 3),
            "frac_compute_peak": round(tf / peak, 4),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "flops_per_call": flops,
            "timing": "%d calls" % steps, "repeat": st}
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return res


def measure_axial_block(steps: int = 200):
    """The fused axial-attention block on the pages' images (4 of 32 x 32
    tokens, C = 64, 4 heads of 16): each pass alone and the whole block (two
    launches), HIP graph of `steps` calls. FLOPs per pass: 2*C*3C + 2*C*C per
    token for the projections plus 4*L*d per token and head for the two
    attention products; algorithmic bytes per pass: the image read once and
    written once plus the pass's weights."""
    import torch
    import scaled_dot_product_12_amd as attn
    from scaled_dot_product_12_amd.inputs import make_axial_block
    x, row, col = make_axial_block()
    B, Hh, W, C = x.shape
    heads, d = 4, C // 4
    dev = torch.device("cuda:0")
    x = x.to(dev)
    row = tuple(t.to(dev) for t in row)
    col = tuple(t.to(dev) for t in col)
    out = torch.empty_like(x)
    tokens = B * Hh * W
    wbytes = 4 * (2 * C + 3 * C * C + C * C + C)
    pass_bytes = 2 * 4 * tokens * C + wbytes
    res = {}
    for name, fn, L in (
            ("axial_row_pass", lambda: attn.axial_pass(x, row, attn.MI355_AXIAL_ROW, out=out), W),
            ("axial_col_pass", lambda: attn.axial_pass(x, col, attn.MI355_AXIAL_COL, out=out), Hh),
            ("axial_block", lambda: attn.axial_block(x, row, col, out=out), None)):
        ms, _, st = time_launches(fn, steps, 3, graph=True)
        if L is None:
            flops = sum(tokens * (8 * C * C + 4 * heads * l * d) for l in (W, Hh))
            nbytes = 2 * pass_bytes
        else:
            flops = tokens * (8 * C * C + 4 * heads * L * d)
            nbytes = pass_bytes
        tf = flops / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {
            "workload": f"fused axial {name[6:].replace('_', ' ')} fp32 B={B} Hh={Hh} W={W} "
                        f"C={C} heads={heads}",
            "us_per_call": round(ms * 1e3, 3), "tflops": round(tf, 4),
            "frac_compute_peak": round(tf / PEAK_FP32_TFLOPS, 4),
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "flops_per_call": flops, "algorithmic_bytes": nbytes,
            "timing": "HIP graph of %d calls" % steps, "repeat": st,
        }
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the attention "
              "forward here has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import __graft_entry__ as ge
    from scaled_dot_product_12_amd.inputs import WORKLOADS
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    ge.ensure_built()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if a.axial_only:
        print(json.dumps(measure_axial_block(a.steps)), flush=True)
        return
    if a.backward_only:
        w = WORKLOADS[a.workload]
        for one_pass in (True, False):
            ms, tf, st, path = measure_bwd(w, a.steps, a.warmup, one_pass)
            print(json.dumps({"backward": w.describe(), "path": path,
                              "us_per_call": round(ms * 1e3, 3), "tflops": round(tf, 3),
                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "repeat": st}), flush=True)
        return
    w = WORKLOADS[a.workload]
    print(f"[bench] headline {w.describe()}", file=sys.stderr, flush=True)
    ms, wall, tflops, gbs, tensors, head_st = measure(w, a.steps, a.warmup, graph=False)
    del tensors
    torch.cuda.empty_cache()
    print(f"[bench] {ms*1e3:.1f} us/step {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
    half = w.dtype in ("bf16", "fp16")
    peak = PEAK_BF16_TFLOPS if half else PEAK_FP32_TFLOPS
    traffic = stored_traffic(w.name)

    extra = {}
    if not a.no_extra:
        for name in ("c1", "c2", "c2c", "c3r", "c3c", "c3", "c5", "p64", "p128", "c4h"):
            if name == w.name:
                continue
            x = WORKLOADS[name]
            small = x.flops < 1e9
            steps = 200 if small else max(5, min(50, int(2e12 / x.flops)))
            print(f"[bench] extra {x.describe()}", file=sys.stderr, flush=True)
            xms, _, xtf, xgbs, xt, xst = measure(x, steps, 3, graph=small)
            del xt
            torch.cuda.empty_cache()
            xpeak = PEAK_BF16_TFLOPS if x.dtype in ("bf16", "fp16") else PEAK_FP32_TFLOPS
            extra[name] = {
                "workload": x.describe(), "us_per_call": round(xms * 1e3, 3),
                "tflops": round(xtf, 3), "frac_compute_peak": round(xtf / xpeak, 4),
                "gbs": round(xgbs, 1), "frac_hbm_peak": round(xgbs / PEAK_HBM_GBS, 4),
                "timing": "HIP graph of %d calls" % steps if small else "%d calls" % steps,
                "repeat": xst,
            }
            if name in ("c1", "c3r", "c3c", "c3"):
                cus, nsets, cst = measure_cold(x)
                cgbs = x.algorithmic_bytes() / (cus * 1e-6) / 1e9
                extra[name].update({
                    "cold_us_per_call": round(cus, 3), "cold_repeat": cst,
                    "cold_buffer_sets": nsets, "cold_gbs": round(cgbs, 1),
                    "cold_frac_hbm_peak": round(cgbs / PEAK_HBM_GBS, 4)})
            if x.axial:
                cus = same_bytes_copy_us(x.algorithmic_bytes())
                extra[name]["same_bytes_copy_us"] = round(cus, 3)
                extra[name]["frac_of_copy_rate"] = round(cus / (xms * 1e3), 4)
                ccus = same_bytes_copy_cold_us(x.algorithmic_bytes())
                extra[name]["same_bytes_copy_cold_us"] = round(ccus, 3)
                extra[name]["cold_frac_of_copy_rate"] = round(
                    ccus / extra[name]["cold_us_per_call"], 4)

    if not a.no_extra:
        print("[bench] extra fused axial block", file=sys.stderr, flush=True)
        extra.update(measure_axial_block())
        print("[bench] extra value head dim of its own", file=sys.stderr, flush=True)
        extra.update(measure_dv())
        print("[bench] extra fp8 inputs", file=sys.stderr, flush=True)
        extra.update(measure_fp8())

    if not a.no_extra:
        for name in ("c4", "c5", "p64", "c4h"):
            x = WORKLOADS[name]
            steps = max(5, min(30, int(4e12 / bwd_flops(x))))
            print(f"[bench] backward {x.describe()}", file=sys.stderr, flush=True)
            bms, btf, bst, path = measure_bwd(x, steps, 3)
            torch.cuda.empty_cache()
            extra["bwd_" + name] = {
                "workload": "backward (dQ, dK, dV) " + x.describe(), "path": path,
                "us_per_call": round(bms * 1e3, 3), "tflops": round(btf, 3),
                "flops_per_call": bwd_flops(x), "frac_compute_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                "timing": "%d calls" % steps, "repeat": bst,
            }
            if path.startswith("one pass"):
                tms, ttf, tst, tpath = measure_bwd(x, steps, 3, one_pass=False)
                torch.cuda.empty_cache()
                extra["bwd_" + name + "_two_kernels"] = {
                    "workload": "backward (dQ, dK, dV) " + x.describe(), "path": tpath,
                    "us_per_call": round(tms * 1e3, 3), "tflops": round(ttf, 3),
                    "flops_per_call": bwd_flops(x),
                    "frac_compute_peak": round(ttf / PEAK_BF16_TFLOPS, 4),
                    "timing": "%d calls" % steps, "repeat": tst,
                }

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, a.cpu_seconds)

    line = {
        "metric": "attention fwd TFLOP/s on 1 MI355X (4*B*H*M*N*D)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": (f"synthetic (seeded N(0,1), rounded to {w.dtype})" if half
                 else "synthetic (seeded N(0,1))"),
        "config": {"workload": w.describe(), "B": w.B, "H": w.H, "M": w.M, "N": w.N,
                   "D": w.D, "causal": w.causal, "seed": w.seed,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "hbm_gbs_algorithmic": round(gbs, 1),
        "wall_s_timed": round(wall, 4),
        "repeat": head_st,
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
