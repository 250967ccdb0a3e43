"""Benchmark of varlen GQA attention on one MI355X: forward and forward+backward.

One step = one pass of the whole path over one batch: attn_varlen_fwd (with the
LSE) followed by attn_varlen_bwd (Delta preprocess, dK/dV, dQ), inputs resident
in HBM. Timing follows the pages' benchmark method ("FA2 vs NATTEN on A100"
issue, benchmark script: warm-up iterations, then timed iterations with
device events; the LSE repro warms the GPU with 1 s of bf16 GEMMs first).

Work accounting (same as the pages: forward 4 * n^2 * heads * head_dim per
sequence, forward+backward 3.5x that; causal counts half):
    fwd_flop = 4 * sum_b Lq_b * Lk_b * Hq * D * (1/2 if causal)

Prints one JSON line. Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "varlen GQA attn TFLOP/s fwd & fwd+bwd, bf16 hd128 @16K; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def warm_gpu(min_s: float = 0.5, max_s: float = 3.0, tol: float = 0.02):
    """Bring the chip to its loaded operating point before timing (the pages warm
    up with bf16 matrix products before their timed runs: "[FA4/B200]
    return_lse=True ..." repro script, GPU warm-up). Here: batches of eight
    4096^3 bf16 products, each batch timed with device events, until three
    batches in a row agree within `tol` (the clock has settled) and at least
    `min_s` has passed, or `max_s` is reached. Returns the number of batches."""
    import torch

    a = torch.randn(4096, 4096, device="cuda:0", dtype=torch.bfloat16)
    c = torch.empty_like(a)
    t0 = time.perf_counter()
    recent = []
    batches = 0
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            torch.mm(a, a, out=c)
        e1.record()
        e1.synchronize()
        batches += 1
        recent = (recent + [e0.elapsed_time(e1)])[-3:]
        elapsed = time.perf_counter() - t0
        settled = len(recent) == 3 and (max(recent) - min(recent)) <= tol * min(recent)
        if (settled and elapsed >= min_s) or elapsed >= max_s:
            return batches


def kernel_flop(name: str, wl) -> float:
    """Algorithmic flop of one launch of the named kernel (MFMA work it must do)."""
    pairs = sum(a * b for a, b in zip(wl.seqlens_q, wl.seqlens_k)) * (0.5 if wl.causal else 1.0)
    per_pair = {"attn_fwd": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 6, "attn_bwd_dq_ds": 2}.get(name)
    if per_pair is None:
        return 0.0
    return per_pair * pairs * wl.n_q_heads * wl.head_dim


def kernel_bytes(name: str, wl, stored_ds: bool = False) -> float:
    """Algorithmic HBM bytes of one launch (each tensor read or written once; the
    stored dS, bf16 per visible (query, key) pair and query head, written by dK / dV
    and read by the stored-dS dQ kernel)."""
    tq, tk, hq, hkv, d = wl.total_q, wl.total_k, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    q = 2 * tq * hq * d
    kv = 2 * tk * hkv * d
    rows = 4 * tq * hq
    ds = 2 * sum(a * b for a, b in zip(wl.seqlens_q, wl.seqlens_k)) * (0.5 if wl.causal else 1.0) * hq
    return {
        "attn_fwd": q + 2 * kv + q + rows,
        "attn_bwd_prep": 2 * q + 3 * rows,
        "attn_bwd_dkdv": 2 * q + 2 * kv + 2 * rows + 2 * kv + (ds if stored_ds else 0),
        "attn_bwd_dq": 2 * q + 2 * kv + 2 * rows + q,
        "attn_bwd_dq_ds": ds + kv + q,
    }.get(name, 0.0)


# library event name -> kernel symbol stem used in the profiler summaries
KERNEL_SYMBOL = {"attn_fwd": "fwd_kernel", "attn_bwd_prep": "bwd_prep_kernel", "attn_bwd_dkdv": "bwd_dkdv_kernel",
                 "attn_bwd_dq": "bwd_dq_kernel", "attn_bwd_dq_ds": "bwd_dq_ds_kernel"}


def measured_traffic(kernel: str, workload_tag: str):
    """HBM bytes per launch (read + write) of `kernel` from the committed
    FETCH_SIZE / WRITE_SIZE summary in profiles/, only if that summary was taken
    with the library binary loaded now; otherwise None."""
    import hashlib

    import exact_attention_varlen_amd._lib as L

    path = os.path.join(ROOT, "profiles", f"attn_kernels_{workload_tag}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(L.LIB_PATH, "rb").read()).hexdigest()
    for line in open(path):
        line = line.strip()
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
            if rec.get("lib_sha256") != sha:
                return None
            k = rec["kernels"].get(KERNEL_SYMBOL.get(kernel, ""))
            return None if k is None else k["read_bytes"] + k["write_bytes"]
    return None


def time_steps(fn, steps: int, warmup: int):
    """Run warmup untimed, then `steps` timed calls; returns (ms per step, per-step event ms list)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / max(1, steps)
    per = [s.elapsed_time(e) for s, e in evs]
    return wall, per


def time_graph(fn, steps: int, warmup: int):
    """Capture fn into a HIP graph (after eager warm-up) and time `steps` replays.

    Returns (ms per replay over the bracketed region, per-replay event ms)."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return time_steps(g.replay, steps, warmup)


def time_graph_steps(fn, steps: int, warmup: int):
    """Capture `steps` back-to-back calls of fn in one HIP graph (after eager
    warm-up, and one untimed replay), then time one replay of it bracketed by
    synchronizations. Returns (wall ms per call, event ms per call): the steps
    run back to back as in a training loop, without the per-replay dispatch gap
    of a one-step graph."""
    import torch

    for _ in range(max(3, warmup)):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / max(1, steps)
    return wall, s.elapsed_time(e) / max(1, steps)


def time_graph_steady(fn, reps: int = 10, rounds: int = 5):
    """Per-call ms of `reps` back-to-back calls captured in one HIP graph (median
    over rounds): the steady-state rate without per-launch dispatch gaps."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    return statistics.median(per)


def read_clocks():
    """One `amd-smi metric` sample: socket power (W) and the graphics clock of
    each XCD (MHz). Returns None when the tool is unavailable."""
    import re
    import subprocess

    try:
        txt = subprocess.run(["amd-smi", "metric"], capture_output=True, text=True, timeout=20).stdout
    except Exception:  # pragma: no cover
        return None
    power = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    clks = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", txt)]
    if not clks:
        return None
    return {"power_w": float(power[0]) if power else None, "gfx_mhz": clks}


def gemm_reference(n: int = 8192, reps: int = 20):
    """Rate of a plain square bf16 GEMM (torch.mm, i.e. the vendor GEMM library)
    on this board, back to back after a warm-up: context for the attention
    kernels' fraction of the published MFMA peak, which the board's power limit
    keeps out of reach of any kernel."""
    import torch

    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(5):
        torch.mm(a, b, out=c)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        torch.mm(a, b, out=c)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))[reps // 2]
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"op": f"torch.mm bf16 {n}x{n}x{n}", "ms_median": ms, "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS}


def power_phase(fn, seconds: float = 4.0):
    """Run fn back to back for `seconds` and sample clocks / power from a side
    thread in the second half: the sustained operating point of this work."""
    import threading

    import torch

    samples = []
    stop = threading.Event()

    def sampler():
        if stop.wait(seconds * 0.4):
            return
        while not stop.is_set() and len(samples) < 3:
            r = read_clocks()
            if r is None:
                return
            samples.append(r)

    th = threading.Thread(target=sampler, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    stop.set()
    th.join(timeout=30)
    if not samples:
        return {"error": "amd-smi metric gave no clock readings"}
    clks = [c for s in samples for c in s["gfx_mhz"]]
    pw = [s["power_w"] for s in samples if s["power_w"] is not None]
    return {
        "sclk_mhz_mean": sum(clks) / len(clks),
        "sclk_mhz_min": min(clks),
        "sclk_mhz_max": max(clks),
        "sclk_mhz_nominal_max": 2400.0,
        "socket_power_w": (sum(pw) / len(pw)) if pw else None,
        "samples": len(samples),
        "calls": n,
        "source": "amd-smi metric (per-XCD GFX clocks, socket power) while the step runs back to back",
    }


# Numbers the pages print for workloads this bench also runs, on other GPUs
# ("FA2 vs NATTEN on A100" results table: 16K single sequence, 32/8 heads, hd128,
# non-causal; "[FA4/B200] return_lse=True ..." repro: 2x16384, 16 heads, hd64,
# with the LSE). Context only: different hardware, not the target.
PAGE_NUMBERS = {
    "single-16384-gqa32/8-d128-full": {"source": "A100, FA2 (flash-attn 2.7.4)", "fwd_tflops": 216.0,
                                       "fwdbwd_tflops": 196.0},
    "2x16384-mha16-d64-full": {"source": "B200, FA4 forward with LSE", "fwd_tflops": 2.199e3 / 2.5281},
}


def context_other_hardware(secondary):
    out = {}
    s16 = secondary.get("single-16384-gqa32/8-d128-full")
    if s16:
        ref = PAGE_NUMBERS["single-16384-gqa32/8-d128-full"]
        out["single-16384-gqa32/8-d128-full"] = {
            "page": ref, "ours_fwd_tflops": s16["fwd_tflops"], "ours_fwdbwd_tflops": s16["fwdbwd_tflops"],
            "fwd_ratio": s16["fwd_tflops"] / ref["fwd_tflops"],
            "fwdbwd_ratio": s16["fwdbwd_tflops"] / ref["fwdbwd_tflops"]}
    lr = secondary.get("lse_ratio")
    if lr:
        ref = PAGE_NUMBERS["2x16384-mha16-d64-full"]
        out["2x16384-mha16-d64-full"] = {"page": ref, "ours_fwd_tflops_with_lse": lr["with_lse_tflops"],
                                         "fwd_ratio": lr["with_lse_tflops"] / ref["fwd_tflops"]}
    return out


def lse_ratio(wl, rounds: int = 5, reps: int = 10):
    """Forward with and without the LSE output, timed in alternating rounds (the
    pages' with / without LSE comparison); returns medians and their ratio."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl, with_dout=False).items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")

    def f(with_lse):
        return lambda: A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                         wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out,
                                         lse=lse if with_lse else None)

    t_no, t_with = [], []
    for _ in range(rounds):
        t_no.append(time_graph_steady(f(False), reps, 1))
        t_with.append(time_graph_steady(f(True), reps, 1))
    no, wi = statistics.median(t_no), statistics.median(t_with)
    fl = wl.accounted_fwd_flop()
    return {"workload": wl.name, "no_lse_ms": no, "with_lse_ms": wi, "no_lse_over_with_lse": no / wi,
            "no_lse_tflops": fl / (no * 1e-3) / 1e12, "with_lse_tflops": fl / (wi * 1e-3) / 1e12}


def bwd_ws_bytes(wl, stored_ds=False) -> int:
    """Backward workspace for a workload: the recomputing backward's, or the
    stored-dS one's (attn_varlen_bwd_stored_ds)."""
    import exact_attention_varlen_amd as A

    return A.bwd_workspace_bytes(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.max_seqlen_q, wl.max_seqlen_k,
                                 wl.n_q_heads, wl.n_kv_heads, wl.head_dim, stored_ds)


def run_workload(wl, steps, warmup, profile=True, stored_ds=False):
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    inp = W.make_inputs(wl)
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    mq, mk = wl.max_seqlen_q, wl.max_seqlen_k
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
    dq = torch.empty_like(d["q"])
    dk = torch.empty_like(d["k"])
    dv = torch.empty_like(d["v"])
    ws = torch.empty(max(16, bwd_ws_bytes(wl, stored_ds)), dtype=torch.uint8, device="cuda:0")

    def fwd():
        A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk, wl.softmax_scale,
                          wl.causal, out=out, lse=lse)

    def step():
        fwd()
        A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk,
                          wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv, workspace=ws, stored_ds=stored_ds)

    res = {}
    res["stored_ds"] = bool(stored_ds)
    fwd_flop = wl.accounted_fwd_flop()
    # 1) eager calls with per-launch event timing inside the library
    if profile:
        A.attn_varlen_profile_enable(True)
    eager_step_ms, _ = time_steps(step, steps, warmup)
    recs = []
    if profile:
        A.attn_varlen_profile_enable(False)
        recs = A.attn_varlen_profile_records()
    # 2) the same work replayed from HIP graphs: no host launch overhead
    fwd_ms, fwd_per = time_graph(fwd, steps, warmup)
    step_single_ms, step_per = time_graph(step, steps, warmup)
    # the step figure: all timed steps back to back in one graph
    step_ms, step_event_ms = time_graph_steps(step, steps, warmup)
    # the forward figure: event-timed, ten forwards back to back in one graph
    # (per call, median of five rounds), free of the per-launch dispatch gap
    # that a single-kernel graph replay adds
    res["fwd_ms"] = time_graph_steady(fwd)
    res["fwd_tflops"] = fwd_flop / (res["fwd_ms"] * 1e-3) / 1e12
    res["_step_fn"] = step
    res["fwd_ms_single_replay"] = fwd_ms
    res["fwd_ms_single_replay_median"] = statistics.median(fwd_per)
    res["fwd_tflops_single_replay"] = fwd_flop / (fwd_ms * 1e-3) / 1e12
    res["step_ms"] = step_ms
    res["step_ms_event"] = step_event_ms
    res["step_ms_single_replay"] = step_single_ms
    res["step_ms_single_replay_median"] = statistics.median(step_per)
    res["fwdbwd_tflops"] = 3.5 * fwd_flop / (step_ms * 1e-3) / 1e12
    res["eager_step_ms"] = eager_step_ms
    # per-kernel averages over the timed eager steps (the session also saw the
    # warm-up steps: drop their launches)
    per_kernel = {}
    if recs:
        n_per_step = len(recs) // (steps + warmup)
        timed = recs[warmup * n_per_step:]
        for name, ms in timed:
            per_kernel.setdefault(name, []).append(ms)
    res["kernels"] = {k: {"avg_ms": sum(v) / len(v), "launches": len(v)} for k, v in per_kernel.items()}
    return res


def cpu_baseline(wl, budget_s: float = 20.0):
    """Time the float64 oracle (forward + backward) on a bounded sample of the workload.

    The sample is whole sequences from the front of the batch with all heads, grown
    until the estimated cost reaches the budget; the rate is reported in accounted
    TFLOP/s of forward+backward, the same unit as the GPU figure."""
    import numpy as np

    import oracle.attention as O
    import workloads as W

    threads, cpu_model = _host_cpu()
    inp = W.make_inputs(wl)
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    cu = wl.cu_seqlens_q
    # grow a sample of heads of the first sequence until it takes ~budget
    L = wl.seqlens_q[0]
    heads = 1
    sample_desc = None
    spent = 0.0
    flop_done = 0.0
    h_done = 0
    seq = slice(cu[0], cu[1])
    t_start = time.perf_counter()
    while h_done < wl.n_q_heads and (time.perf_counter() - t_start) < budget_s:
        r = wl.n_q_heads // wl.n_kv_heads
        g = h_done // r
        # one query head (with its KV head) at a time, as a one-head problem
        qs = q[seq, h_done:h_done + 1]
        ks = k[seq, g:g + 1]
        vs = v[seq, g:g + 1]
        dos = do[seq, h_done:h_done + 1]
        t0 = time.perf_counter()
        O.forward(qs, ks, vs, [0, L], [0, L], wl.softmax_scale, wl.causal)
        O.backward(qs, ks, vs, [0, L], [0, L], wl.softmax_scale, wl.causal, dos)
        spent += time.perf_counter() - t0
        flop_done += 3.5 * 4.0 * L * L * wl.head_dim * (0.5 if wl.causal else 1.0)
        h_done += 1
    sample_desc = f"sequence 0 ({L} tokens), {h_done} of {wl.n_q_heads} query heads, forward+backward"
    return {
        "value": flop_done / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": sample_desc,
        "seconds": spent,
        "cpu_model": cpu_model,
        "host_cpus_visible": len(os.sched_getaffinity(0)),
        "blas_threads": int(threads),
    }


def named_workload(name: str):
    """A workload of the benchmark set by name (`--workload`)."""
    import workloads as W

    known = {wl.name: wl for wl in W.all_configs() + [W.single_16k_full()]}
    if name not in known:
        raise SystemExit(f"unknown workload {name!r}; known: {sorted(known)}")
    return known[name]


def eager_only(wl, steps: int, warmup: int, stored_ds: bool = False):
    """warmup + steps eager forward+backward steps (forward only for a
    forward-only workload), no graphs and no extra timing machinery: the command
    profilers wrap. stored_ds: the backward stores dS for dQ
    (attn_varlen_bwd_stored_ds) instead of recomputing it."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
    ws = None
    if wl.backward:
        ws = torch.empty(max(16, bwd_ws_bytes(wl, stored_ds)), dtype=torch.uint8, device="cuda:0")
    for i in range(warmup + steps):
        out, lse = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                                     wl.max_seqlen_k, wl.softmax_scale, wl.causal, return_lse=True)
        if not wl.backward:
            continue
        A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                          wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, workspace=ws,
                          stored_ds=stored_ds)
    torch.cuda.synchronize()
    print(json.dumps({"workload": wl.name, "eager_steps": warmup + steps, "stored_ds": bool(stored_ds)}), flush=True)
    return 0


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) of a profiler run: each launch reads and writes
    `nbytes`."""
    import torch

    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)
    return 0


def visible_pairs(wl) -> int:
    """Exact number of visible (query, key) pairs per head, with the causal
    mask and the local window of the workload (bottom-right aligned band)."""
    import numpy as np

    wl_, wr_ = (-1, -1) if wl.window is None else wl.window
    if wl.causal:
        wr_ = 0 if wr_ < 0 else min(wr_, 0)
    total = 0
    for Lq, Lk in zip(wl.seqlens_q, wl.seqlens_k):
        i = np.arange(Lq, dtype=np.int64)
        lo = np.zeros(Lq, dtype=np.int64) if wl_ < 0 else np.clip(i + Lk - Lq - wl_, 0, Lk)
        hi = np.full(Lq, Lk, dtype=np.int64) if wr_ < 0 else np.clip(i + Lk - Lq + wr_ + 1, 0, Lk)
        total += int(np.maximum(hi - lo, 0).sum())
    return total


def window_split_secondary():
    """Local-window and split-KV forward timings (steady state, HIP graphs).

    Work is counted as 4 * D * Hq per visible (query, key) pair (exact count),
    the forward's algorithmic flop; fwd+bwd as 3.5 x that."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    out_rows = {}
    cases = [
        ("window", W.Workload("single-16384-gqa32/8-d128-causal-w4096", [16384], 32, 8, 128, True,
                              window=(4096, -1)), None),
        ("window", W.Workload("single-16384-gqa32/8-d128-causal-w512", [16384], 32, 8, 128, True,
                              window=(512, -1)), None),
        ("window", W.Workload("single-16384-gqa32/8-d128-full-w1024_1024", [16384], 32, 8, 128, False,
                              window=(1024, 1024)), None),
        ("split", W.Workload("2x256-vs-32768-gqa32/8-d128-causal", [256, 256], 32, 8, 128, True,
                             seqlens_k=[32768, 32768]), (1, 0)),
        ("split", W.Workload("1x128-vs-65536-mha16-d64-full", [128], 16, 16, 64, False, seqlens_k=[65536]),
         (1, 0)),
        ("split", W.Workload("4x64-vs-8192-gqa8/1-d256-causal", [64] * 4, 8, 1, 256, True, seqlens_k=[8192] * 4),
         (1, 0)),
    ]
    for kind, wl, splits in cases:
        log(f"{kind} workload {wl.name}")
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
        mq, mk = wl.max_seqlen_q, wl.max_seqlen_k
        win = (-1, -1) if wl.window is None else wl.window
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        flop = 4.0 * visible_pairs(wl) * wl.n_q_heads * wl.head_dim
        row = {**wl.describe(), "visible_pairs_per_head": visible_pairs(wl), "fwd_gflop": flop / 1e9}
        for ns in (splits or (1,)):
            n = ns if ns else A.attn_varlen_fwd_num_splits(len(wl.seqlens_q), wl.total_q, mq, mk, wl.n_q_heads,
                                                           wl.n_kv_heads, wl.head_dim)
            ws = torch.empty(max(16, A.attn_varlen_fwd_splitkv_workspace_size(wl.total_q, wl.n_q_heads,
                                                                              wl.head_dim, n)),
                             dtype=torch.uint8, device="cuda:0")

            def fwd():
                A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk,
                                  wl.softmax_scale, wl.causal, out=out, lse=lse, window_size=win, num_splits=n,
                                  workspace=ws)

            ms = time_graph_steady(fwd, 10, 3)
            key = "fwd" if splits is None else f"fwd_splits_{n}"
            row[key + "_ms"] = ms
            row[key + "_tflops"] = flop / (ms * 1e-3) / 1e12
        if kind == "window":
            dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
            wsb = torch.empty(max(16, bwd_ws_bytes(wl)), dtype=torch.uint8, device="cuda:0")

            def step():
                A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk,
                                  wl.softmax_scale, wl.causal, out=out, lse=lse, window_size=win)
                A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"],
                                  d["cu_seqlens_k"], mq, mk, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv,
                                  workspace=wsb, window_size=win)

            ms = time_graph_steady(step, 5, 3)
            row["fwdbwd_ms"] = ms
            row["fwdbwd_tflops"] = 3.5 * flop / (ms * 1e-3) / 1e12
        out_rows[wl.name] = row
        del d, out, lse
        torch.cuda.empty_cache()
    return out_rows


def bwd_paths(wl, rounds: int = 3):
    """The step (forward with LSE + backward) with dS stored for dQ against the
    recomputing dQ, steady state, alternating rounds, with per-kernel times of
    eager steps for each."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
    mq, mk = wl.max_seqlen_q, wl.max_seqlen_k
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    ws = {s: torch.empty(max(16, bwd_ws_bytes(wl, s)), dtype=torch.uint8, device="cuda:0") for s in (True, False)}

    def step(s):
        def f():
            A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk, wl.softmax_scale,
                              wl.causal, out=out, lse=lse)
            A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                              mq, mk, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv, workspace=ws[s], stored_ds=s)
        return f

    times = {True: [], False: []}
    for _ in range(rounds):
        for s in (True, False):
            times[s].append(time_graph_steady(step(s), 5, 1))
    row = {"workload": wl.name}
    for s, tag in ((True, "stored_ds"), (False, "recompute")):
        A.attn_varlen_profile_enable(True)
        for _ in range(3):
            step(s)()
        torch.cuda.synchronize()
        A.attn_varlen_profile_enable(False)
        recs = A.attn_varlen_profile_records()
        per = {}
        for name, ms in recs[len(recs) // 3:]:
            per.setdefault(name, []).append(ms)
        ms = statistics.median(times[s])
        row[tag] = {"step_ms": ms, "fwdbwd_tflops": wl.accounted_fwdbwd_flop() / (ms * 1e-3) / 1e12,
                    "kernels_ms": {k: sum(v) / len(v) for k, v in per.items()},
                    "workspace_bytes": ws[s].numel()}
    row["stored_ds_speedup"] = row["recompute"]["step_ms"] / row["stored_ds"]["step_ms"]
    return row


def persistent_vs_grid(wl, rounds: int = 3):
    """Forward with the one-workgroup-per-item grid against the persistent
    scheduler (attn_varlen_fwd_persistent), steady state, alternating rounds."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl, with_dout=False).items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
    sched = torch.zeros(A.SCHED_BYTES, dtype=torch.uint8, device="cuda:0")

    def fwd(pers):
        return lambda: A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                         wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out,
                                         lse=lse, persistent=pers, sched=sched)

    times = {False: [], True: []}
    for _ in range(rounds):
        for pers in (False, True):
            times[pers].append(time_graph_steady(fwd(pers), 10, 3))
    g, p = statistics.median(times[False]), statistics.median(times[True])
    fl = wl.accounted_fwd_flop()
    return {"workload": wl.name, "grid_fwd_ms": g, "persistent_fwd_ms": p, "grid_tflops": fl / (g * 1e-3) / 1e12,
            "persistent_tflops": fl / (p * 1e-3) / 1e12, "persistent_speedup": g / p}


def _host_cpu():
    """(BLAS threads, CPU model) of this host, for the oracle's timing lines."""
    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return int(threads), cpu_model


def oracle_table(budget_s: float = 4.0, max_sample_len: int = 8192, whole_flop: float = 2e10):
    """Wall-clock of the float64 oracle, forward and forward+backward, for every
    config: one JSON object per config on stdout. A config whose whole oracle
    run fits the budget is timed whole ("measured"). Otherwise the sample is the
    first sequence (cut to its first max_sample_len tokens), one query head with
    its KV head at a time, heads added until the budget is spent; the full time
    is the config's accounted work divided by the sample's rate ("extrapolated")."""
    import oracle.attention as O
    import workloads as W

    threads, cpu_model = _host_cpu()
    warm = W.make_inputs(W.tiny(True))  # first BLAS calls start the thread pool: untimed
    O.forward(*(W.to_f64(warm[x]) for x in ("q", "k", "v")), W.tiny(True).cu_seqlens_q, W.tiny(True).cu_seqlens_k,
              0.125, True)
    for wl in W.all_configs() + [W.single_16k_full()]:
        log(f"oracle timing {wl.name}")
        inp = W.make_inputs(wl)
        fl = wl.accounted_fwd_flop()
        whole = 3.5 * fl < whole_flop  # by default a few seconds of fp64 BLAS on a multi-core host
        if whole:
            q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
            t0 = time.perf_counter()
            O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal)
            t_f = time.perf_counter() - t0
            O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do)
            t_b = time.perf_counter() - t0 - t_f
            row = {"config": wl.name, "kind": "measured", "sample": "whole config", "oracle_fwd_s": t_f,
                   "oracle_fwdbwd_s": t_f + t_b}
        else:
            L = min(wl.seqlens_q[0], max_sample_len)
            r = wl.n_q_heads // wl.n_kv_heads
            sample_fl, t_f, t_b, heads = 0.0, 0.0, 0.0, 0
            while heads < wl.n_q_heads and (heads == 0 or t_f + t_b < budget_s):
                h, g = heads, heads // r
                qs = W.to_f64(inp["q"][:L, h:h + 1])
                ks = W.to_f64(inp["k"][:L, g:g + 1])
                vs = W.to_f64(inp["v"][:L, g:g + 1])
                dos = W.to_f64(inp["dout"][:L, h:h + 1])
                t0 = time.perf_counter()
                O.forward(qs, ks, vs, [0, L], [0, L], wl.softmax_scale, wl.causal)
                t1 = time.perf_counter()
                O.backward(qs, ks, vs, [0, L], [0, L], wl.softmax_scale, wl.causal, dos)
                t_f += t1 - t0
                t_b += time.perf_counter() - t1
                sample_fl += 4.0 * L * L * wl.head_dim * (0.5 if wl.causal else 1.0)
                heads += 1
            row = {"config": wl.name, "kind": "extrapolated",
                   "sample": f"sequence 0 cut to {L} tokens, {heads} of {wl.n_q_heads} query heads",
                   "sample_fwd_s": t_f, "sample_fwdbwd_s": t_f + t_b,
                   "oracle_fwd_s": fl * t_f / sample_fl, "oracle_fwdbwd_s": fl * (t_f + t_b) / sample_fl}
        row.update({"accounted_fwd_gflop": fl / 1e9,
                    "oracle_fwd_gflops": fl / row["oracle_fwd_s"] / 1e9,
                    "oracle_fwdbwd_gflops": 3.5 * fl / row["oracle_fwdbwd_s"] / 1e9,
                    "threads": threads, "cpu_model": cpu_model,
                    "host_cpus_visible": len(os.sched_getaffinity(0))})
        print(json.dumps(row), flush=True)
        del inp
    return 0


def all_configs_table(include_long: bool):
    """Forward and forward+backward time of every config (fwd with LSE; steady
    state, several calls per HIP graph): one JSON object per config on stdout."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    rows = []
    for wl in W.all_configs():
        if not include_long and wl.total_q > 40000:
            continue
        log(f"config {wl.name}")
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
        mq, mk = wl.max_seqlen_q, wl.max_seqlen_k
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        ws = torch.empty(max(16, bwd_ws_bytes(wl)), dtype=torch.uint8, device="cuda:0")

        def fwd():
            A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk,
                              wl.softmax_scale, wl.causal, out=out, lse=lse)

        def step():
            fwd()
            A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"], mq,
                              mk, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv, workspace=ws)

        fl = wl.accounted_fwd_flop()
        reps = max(1, min(10, int(2e13 / max(fl, 1.0))))
        f_ms = time_graph_steady(fwd, reps, 3)
        s_ms = time_graph_steady(step, reps, 3) if wl.backward else None
        row = {"config": wl.name, **wl.describe(), "fwd_ms": f_ms, "fwd_tflops": fl / (f_ms * 1e-3) / 1e12,
               "fwdbwd_ms": s_ms, "fwdbwd_tflops": (3.5 * fl / (s_ms * 1e-3) / 1e12) if s_ms else None}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del d, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return 0


def many_docs_table(total: int = 65536):
    """Forward and forward+backward of batches of equal causal documents (32/8
    heads, hd128) at a fixed token count, from 16 to 4096 documents: the cost of
    the work decode as the number of sequences grows (one JSON line each)."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    for n in (16, 64, 65, 256, 1024, 4096):
        L = total // n
        wl = W.Workload(f"docs{n}x{L}-gqa32/8-d128-causal", [L] * n, 32, 8, 128, True)
        log(f"many documents {wl.name}")
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        ws = torch.empty(max(16, bwd_ws_bytes(wl)), dtype=torch.uint8, device="cuda:0")

        def fwd():
            A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], L, L, wl.softmax_scale,
                              True, out=out, lse=lse)

        def step():
            fwd()
            A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"], L, L,
                              wl.softmax_scale, True, dq=dq, dk=dk, dv=dv, workspace=ws)

        fl = wl.accounted_fwd_flop()
        f_ms = time_graph_steady(fwd, 10, 3)
        s_ms = time_graph_steady(step, 5, 3)
        print(json.dumps({"workload": wl.name, "documents": n, "tokens_each": L, "fwd_ms": f_ms,
                          "fwd_tflops": fl / (f_ms * 1e-3) / 1e12, "fwdbwd_ms": s_ms,
                          "fwdbwd_tflops": 3.5 * fl / (s_ms * 1e-3) / 1e12}), flush=True)
        del d, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return 0


def few_kv_heads_table():
    """Forward and backward of short sequences with few KV heads (MQA / narrow
    GQA), where the head dim 64 / 128 dK / dV work splits a group's query heads
    over several work items (one JSON line each)."""
    import torch

    import exact_attention_varlen_amd as A
    import workloads as W

    for wl in (W.Workload("4096-gqa32/8-d128-full", [4096], 32, 8, 128, False),
               W.Workload("4096-mqa32-d128-full", [4096], 32, 1, 128, False),
               W.Workload("4096-mqa32-d128-causal", [4096], 32, 1, 128, True),
               W.Workload("2x2048-mqa16-d64-causal", [2048, 2048], 16, 1, 64, True),
               W.Workload("8192-gqa64/2-d128-causal", [8192], 64, 2, 128, True)):
        log(f"few KV heads {wl.name}")
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        ws = torch.empty(max(16, bwd_ws_bytes(wl)), dtype=torch.uint8, device="cuda:0")
        mq, mk = wl.max_seqlen_q, wl.max_seqlen_k

        def fwd():
            A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk, wl.softmax_scale,
                              wl.causal, out=out, lse=lse)

        def bwd():
            A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"], mq,
                              mk, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv, workspace=ws)

        fwd()
        fl = wl.accounted_fwd_flop()
        f_ms = time_graph_steady(fwd, 10, 3)
        b_ms = time_graph_steady(bwd, 5, 3)
        print(json.dumps({"workload": wl.name, "fwd_ms": f_ms, "fwd_tflops": fl / (f_ms * 1e-3) / 1e12,
                          "bwd_ms": b_ms, "bwd_tflops": 2.5 * fl / (b_ms * 1e-3) / 1e12}), flush=True)
        del d, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return 0


def kernel_times(rounds: int = 3, steps: int = 8):
    """Per-kernel times (library events, eager forward+backward steps) of one
    workload per head dim, for comparing builds of the library: one JSON line
    naming the library file, with each kernel's median over rounds of its mean
    over steps."""
    import torch

    import exact_attention_varlen_amd as A
    import exact_attention_varlen_amd._lib as L
    import workloads as W

    rows = {}
    for wl in (W.packed_16k(), W.single_16k_full(), W.Workload("2x16384-mha16-d64-full-bwd", [16384, 16384], 16, 16,
                                                                64, False), W.hd256_gqa(2, 16384, True)):
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl).items()}
        mq, mk = wl.max_seqlen_q, wl.max_seqlen_k
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        ws = torch.empty(max(16, bwd_ws_bytes(wl)), dtype=torch.uint8, device="cuda:0")

        def step():
            A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk, wl.softmax_scale,
                              wl.causal, out=out, lse=lse)
            A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                              mq, mk, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv, workspace=ws)

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        per = {}
        for _ in range(rounds):
            A.attn_varlen_profile_enable(True)
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            A.attn_varlen_profile_enable(False)
            got = {}
            for name, ms in A.attn_varlen_profile_records():
                got.setdefault(name, []).append(ms)
            for name, v in got.items():
                per.setdefault(name, []).append(sum(v) / len(v))
        rows[wl.name] = {k: statistics.median(v) for k, v in per.items()}
        del d, out, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    print(json.dumps({"library": os.path.basename(L.LIB_PATH), "kernels_ms": rows}), flush=True)
    return 0


def fwd_table():
    """Steady-state forward time (with and without the LSE) of one workload per
    head dim, for comparing builds of the library (ATTN_VARLEN_LIBRARY selects a
    variant, e.g. one that computes a share of the exponentials on the FMA pipe):
    one JSON line naming the library file and its exponential setting."""
    import ctypes

    import numpy as np
    import torch

    import exact_attention_varlen_amd as A
    import exact_attention_varlen_amd._lib as L
    import workloads as W

    one = np.zeros(1, dtype=np.float32)
    emu = L.lib().attn_varlen_exp2_fma_host(one.ctypes.data_as(ctypes.c_void_p), one.ctypes.data_as(ctypes.c_void_p),
                                            1)
    rows = {}
    for wl in (W.hd64_mha(), W.single_16k_full(), W.packed_16k(), W.hd256_gqa(2, 16384, False)):
        d = {k: v.to("cuda:0") for k, v in W.make_inputs(wl, with_dout=False).items()}
        out = torch.empty_like(d["q"])
        lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device="cuda:0")
        fl = wl.accounted_fwd_flop()
        row = {}
        for with_lse in (True, False):
            def fwd():
                A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                                  wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out,
                                  lse=lse if with_lse else None)
            ms = time_graph_steady(fwd, 10, 5)
            tag = "lse" if with_lse else "no_lse"
            row[f"fwd_ms_{tag}"] = ms
            row[f"fwd_tflops_{tag}"] = fl / (ms * 1e-3) / 1e12
        rows[wl.name] = row
        del d, out, lse
        torch.cuda.empty_cache()
    print(json.dumps({"library": os.path.basename(L.LIB_PATH), "exp2_emulated_every": emu, "forward": rows}),
          flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the extra workloads")
    ap.add_argument("--stored-ds", action="store_true",
                    help="with --eager-only: the backward stores dS for dQ instead of recomputing it")
    ap.add_argument("--eager-only", action="store_true",
                    help="only run warmup + steps eager fwd+bwd steps of the main workload (for profilers) and exit")
    ap.add_argument("--workload", default=None,
                    help="with --eager-only: the workload to run (a config name; default: the packed 16K batch)")
    ap.add_argument("--all-configs", action="store_true",
                    help="only time forward and forward+backward of every config (one JSON line each) and exit")
    ap.add_argument("--long", action="store_true", help="with --all-configs: include the 64K and 128K sequences")
    ap.add_argument("--window-split", action="store_true",
                    help="only time the local-window and split-KV workloads (one JSON line) and exit")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the float64 oracle (forward, forward+backward) for every config, whole or on a "
                         "bounded sample with an extrapolated full time (one JSON line each) and exit")
    ap.add_argument("--bwd-paths", action="store_true",
                    help="only time the step with dS stored for dQ against the recomputing dQ on workloads of "
                         "every head dim <= 128 (one JSON line each) and exit")
    ap.add_argument("--kernel-times", action="store_true",
                    help="only time each kernel of eager forward+backward steps on one workload per head dim for the "
                         "loaded library build (one JSON line) and exit")
    ap.add_argument("--fwd-table", action="store_true",
                    help="only time the forward (with and without the LSE) of one workload per head dim for the "
                         "loaded library build (one JSON line) and exit")
    ap.add_argument("--many-docs", action="store_true",
                    help="only time forward and forward+backward of 16 to 4096 equal causal documents at 65536 "
                         "tokens (one JSON line each) and exit")
    ap.add_argument("--few-kv-heads", action="store_true",
                    help="only time forward and backward of short sequences with 1 or 2 KV heads (one JSON line "
                         "each) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (to scale profiler byte counters) and exit")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); this attention path has no multi-GPU mode",
              file=sys.stderr)
        return 2
    import torch

    import workloads as W

    if a.oracle_table:  # CPU only
        return oracle_table()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if a.copy_calibration:
        return copy_calibration()
    if a.all_configs:
        warm_gpu()
        return all_configs_table(a.long)
    if a.fwd_table:
        warm_gpu()
        return fwd_table()
    if a.many_docs:
        warm_gpu()
        return many_docs_table()
    if a.few_kv_heads:
        warm_gpu()
        return few_kv_heads_table()
    if a.kernel_times:
        warm_gpu()
        return kernel_times()
    if a.bwd_paths:
        warm_gpu()
        for wl in (W.packed_16k(), W.a100_shape(4096), W.single_16k_full(),
                   W.Workload("packed16k-docs-gqa32/8-d64-causal", list(W.PACKED_16K_DOC_LENGTHS), 32, 8, 64, True),
                   W.Workload("2x16384-mha16-d64-full-bwd", [16384, 16384], 16, 16, 64, False),
                   W.Workload("packed16k-docs-gqa32/8-d128-full", list(W.PACKED_16K_DOC_LENGTHS), 32, 8, 128,
                              False)):
            log(f"backward paths {wl.name}")
            print(json.dumps(bwd_paths(wl)), flush=True)
        return 0
    if a.window_split:
        warm_gpu()
        print(json.dumps(window_split_secondary()), flush=True)
        return 0
    if a.eager_only:
        return eager_only(named_workload(a.workload) if a.workload else W.packed_16k(), a.steps, a.warmup,
                          stored_ds=a.stored_ds)
    primary = W.packed_16k()
    log(f"device {torch.cuda.get_device_name(0)}; warming up")
    warm_gpu()
    log(f"primary workload {primary.name}")
    res = run_workload(primary, a.steps, a.warmup, profile=True)
    secondary = {}
    if not a.no_secondary:
        for wl in (W.single_16k_full(), W.a100_shape(4096)):
            log(f"secondary workload {wl.name}")
            r = run_workload(wl, max(3, a.steps // 4), 2, profile=True)
            secondary[wl.name] = {
                "fwd_tflops": r["fwd_tflops"], "fwdbwd_tflops": r["fwdbwd_tflops"], "fwd_ms": r["fwd_ms"],
                "fwd_ms_single_replay": r["fwd_ms_single_replay"],
                "step_ms": r["step_ms"], "frac_fwd": r["fwd_tflops"] / PEAK_BF16_TFLOPS,
                "frac_fwdbwd": r["fwdbwd_tflops"] / PEAK_BF16_TFLOPS,
                "kernels": r["kernels"],
            }
        log("forward with / without LSE, head_dim 64")
        secondary["lse_ratio"] = lse_ratio(W.hd64_mha())
        secondary["window_and_split_kv"] = window_split_secondary()
        secondary["persistent_scheduler"] = persistent_vs_grid(primary)
        log("backward with stored dS against the recomputing dQ")
        secondary["backward_paths"] = {wl.name: bwd_paths(wl) for wl in (primary, W.single_16k_full())}
    log("sustained clocks and power of the primary step")
    clocks = power_phase(res.pop("_step_fn"))
    log("reference GEMM rate")
    gemm = gemm_reference()
    # dominant kernel of the step: the one with the largest total time
    kern = res["kernels"]
    dom = max(kern, key=lambda k: kern[k]["avg_ms"]) if kern else "attn_fwd"
    dom_ms = kern[dom]["avg_ms"] if kern else res["fwd_ms"]
    flop = kernel_flop(dom, primary)
    roofline = {
        "kernel": dom,
        "bound": "mfma",
        "achieved": flop / (dom_ms * 1e-3) / 1e12,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": flop / (dom_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "traffic": measured_traffic(dom, "packed16k-causal-d128"),
        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "avg_ms": dom_ms,
        "flop_per_launch": flop,
        "achieved_vs_gemm_reference": flop / (dom_ms * 1e-3) / 1e12 / gemm["tflops"],
    }
    for k, v in kern.items():
        f = kernel_flop(k, primary)
        v["tflops"] = f / (v["avg_ms"] * 1e-3) / 1e12 if f else None
        v["gbs"] = kernel_bytes(k, primary, res["stored_ds"]) / (v["avg_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": res["fwdbwd_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": res["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": primary.name, **primary.describe(), "pass": "fwd (with LSE) + bwd",
                   "backward": "dS stored for dQ" if res["stored_ds"] else "dQ recomputes S, P, dP"},
        "fwd_tflops": res["fwd_tflops"],
        "fwd_ms": res["fwd_ms"],
        "fwd_timing": ("fwd_ms / fwd_tflops (the forward figure, against which the forward share of the peak "
                       "is judged): HIP events around one graph of ten back-to-back forwards with the LSE, per "
                       "call, median of five rounds. fwd_ms_single_replay: host wall clock over graph replays "
                       "of one forward each, which adds the per-launch dispatch gap"),
        "frac_of_peak_fwd": res["fwd_tflops"] / PEAK_BF16_TFLOPS,
        "frac_of_peak_fwdbwd": res["fwdbwd_tflops"] / PEAK_BF16_TFLOPS,
        "fwd_ms_single_replay": res["fwd_ms_single_replay"],
        "fwd_tflops_single_replay": res["fwd_tflops_single_replay"],
        "clocks": clocks,
        # the published peak assumes 2400 MHz; this is the peak at the clock the
        # chip held (power-limited) while running the step
        "frac_of_peak_fwdbwd_at_sclk": (res["fwdbwd_tflops"] / (PEAK_BF16_TFLOPS * clocks["sclk_mhz_mean"] / 2400.0)
                                        if "sclk_mhz_mean" in clocks else None),
        "step_ms_event": res["step_ms_event"],
        "step_ms_single_replay": res["step_ms_single_replay"],
        "step_ms_single_replay_median": res["step_ms_single_replay_median"],
        "fwd_ms_single_replay_median": res["fwd_ms_single_replay_median"],
        "eager_step_ms": res["eager_step_ms"],
        "timing": ("value / ms_per_step: the K timed steps (forward with LSE, then backward) captured back to "
                   "back in one HIP graph, host wall clock over one replay of it bracketed by synchronizations "
                   "(step_ms_event: HIP events around the same replay). step_ms_single_replay: a graph of one "
                   "step replayed K times, which adds the per-replay dispatch gap. Per-kernel times from eager "
                   "steps with library events on the launch stream"),
        "kernels": kern,
        "roofline": roofline,
        "gemm_reference": gemm,
        "secondary": secondary,
        "context_other_hardware": context_other_hardware(secondary),
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (float64 oracle)")
        line["cpu_baseline"] = cpu_baseline(primary)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
