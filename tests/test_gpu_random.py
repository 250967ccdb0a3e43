"""Randomized GPU parity: seeded random small problems over every option the
path has (head dim, GQA ratio, ragged and empty sequences, Lq != Lk, causal,
local windows, split-KV, the persistent scheduler, softmax scale), each
compared with the float64 oracle at the stated tolerances. The cases are fixed
by their seeds, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import exact_attention_varlen_amd as A
import oracle.attention as O
import workloads as W
from parity import announce, check_grad, check_lse, check_out, check_out_rounded, f64, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 48
N_LONG = 16
N_BROAD = 24


def random_case(seed: int):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    r = int(rng.choice([1, 2, 4, 8]))
    nseq = int(rng.integers(1, 5))
    lq = [int(x) for x in rng.integers(0, 400, size=nseq)]
    same = rng.random() < 0.6
    lk = list(lq) if same else [int(x) for x in rng.integers(0, 400, size=nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    causal = bool(rng.random() < 0.5)
    window = None
    if rng.random() < 0.4:
        left = int(rng.choice([-1, 0, 7, 64, 150]))
        right = int(rng.choice([-1, 0, 5, 90]))
        window = (left, right)
    splits = int(rng.choice([1, 1, 2, 3, 5]))
    persistent = splits == 1 and rng.random() < 0.5
    scale = float(rng.choice([D ** -0.5, 0.03, -0.07]))
    backward = bool(rng.random() < 0.75)
    wl = W.Workload(f"rand{seed}", lq, hkv * r, hkv, D, causal, seqlens_k=lk, seed=seed, softmax_scale=scale,
                    window=window)
    return wl, splits, persistent, backward


def random_long_case(seed: int):
    """Fewer heads, longer sequences (up to 2000 tokens): many key blocks and
    query steps per sequence, end-aligned query blocks, ragged tails."""
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 4]))
    nseq = int(rng.integers(1, 4))
    lq = [int(x) for x in rng.integers(300, 2001, size=nseq)]
    same = rng.random() < 0.7
    lk = list(lq) if same else [int(x) for x in rng.integers(1, 2001, size=nseq)]
    causal = bool(rng.random() < 0.6)
    window = None
    if rng.random() < 0.3:
        window = (int(rng.choice([-1, 100, 700])), int(rng.choice([-1, 0, 300])))
    splits = int(rng.choice([1, 1, 1, 3]))
    persistent = splits == 1 and rng.random() < 0.3
    wl = W.Workload(f"long{seed}", lq, hkv * r, hkv, D, causal, seqlens_k=lk, seed=seed, window=window)
    return wl, splits, persistent, True


def random_broad_case(seed: int):
    """Up to 64 query heads and 8 sequences of 0-2500 tokens, band edges at tile
    boundaries, up to 64 splits, scales from 1e-3 to 0.3, and max_seqlen bounds
    above the true maximum (allowed: they are upper bounds)."""
    rng = np.random.default_rng(70000 + seed)
    while True:
        D = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        r = int(rng.choice([1, 2, 4, 8, 16]))
        if hkv * r > 64:
            continue
        n = int(rng.integers(1, 9))

        def lengths():
            out = []
            for _ in range(n):
                u = rng.random()
                out.append(0 if u < 0.1 else 1 if u < 0.2 else int(rng.integers(2, 130)) if u < 0.5
                           else int(rng.integers(130, 2500)))
            return out
        lq = lengths()
        lk = list(lq) if rng.random() < 0.5 else lengths()
        if sum(lq) == 0:
            lq[0] = 1
        if sum(a * b for a, b in zip(lq, lk)) * hkv * r * D <= 3e9:  # keeps the oracle to seconds
            break
    causal = bool(rng.random() < 0.5)
    edges = [-1, 0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 1000]
    window = (int(rng.choice(edges)), int(rng.choice(edges))) if rng.random() < 0.35 else None
    splits = int(rng.choice([1, 1, 2, 3, 8, 17, 64]))
    persistent = splits == 1 and rng.random() < 0.3
    scale = float(rng.choice([D ** -0.5, 1e-3, 0.3, -0.2, 0.0]))
    wl = W.Workload(f"broad{seed}", lq, hkv * r, hkv, D, causal, seqlens_k=lk, seed=seed, softmax_scale=scale,
                    window=window)
    mq = wl.max_seqlen_q + (int(rng.integers(0, sum(lq) - wl.max_seqlen_q + 1)) if rng.random() < 0.3 else 0)
    mk = wl.max_seqlen_k + (int(rng.integers(0, sum(lk) - wl.max_seqlen_k + 1)) if rng.random() < 0.3 else 0)
    return wl, splits, persistent, bool(rng.random() < 0.7), mq, mk


@pytest.mark.parametrize("seed", list(range(N_BROAD)))
def test_random_broad_case(seed):
    _run_case(f"random broad seed={seed}", *random_broad_case(seed))


@pytest.mark.parametrize("seed", list(range(N_CASES)))
def test_random_case(seed):
    _run_case(f"random seed={seed}", *random_case(seed))


@pytest.mark.parametrize("seed", list(range(N_LONG)))
def test_random_long_case(seed):
    _run_case(f"random long seed={seed}", *random_long_case(seed))


def _run_case(tag, wl, splits, persistent, backward, mq=None, mk=None):
    win = (-1, -1) if wl.window is None else wl.window
    mq = wl.max_seqlen_q if mq is None else mq
    mk = wl.max_seqlen_k if mk is None else mk
    announce(f"{tag} seqlens_q={wl.seqlens_q} seqlens_k={wl.seqlens_k} Hq={wl.n_q_heads} "
             f"Hkv={wl.n_kv_heads} D={wl.head_dim} causal={wl.causal} window={wl.window} splits={splits} "
             f"persistent={persistent} scale={wl.softmax_scale:.4f} backward={backward} max_seqlen=({mq}, {mk})")
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    out, lse = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], mq, mk,
                                 wl.softmax_scale, wl.causal, return_lse=True, window_size=win,
                                 num_splits=splits, persistent=persistent)
    if backward:
        dq, dk, dv = A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"],
                                       d["cu_seqlens_k"], mq, mk, wl.softmax_scale,
                                       wl.causal, window_size=win)
    torch.cuda.synchronize()
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    ro, rl = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, window=wl.window)
    # |O| >= 4: bf16's own spacing exceeds the absolute bound (check_out_rounded)
    (check_out_rounded if ro.size and np.abs(ro).max() >= 4.0 else check_out)(f64(out), ro)
    check_lse(f64(lse), rl)
    if backward:
        rq, rk, rv = O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do,
                                window=wl.window)
        for x, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            if np.any(ref != 0):
                check_grad(f64(x), ref, name)
            else:  # exactly zero (no visible key, or one key per row): rounding leaves ~1e-7
                assert x.numel() == 0 or float(x.abs().max()) <= 1e-5, name
