"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs, run the float64 oracle on the same bits, compare with the stated
tolerances.

Tolerances (fixed for this attention path, bf16 inputs and outputs):
  out    max |gpu - ref| <= 1e-2  and  ||gpu - ref||_F / ||ref||_F <= 5e-3
  lse    max |gpu - ref| <= 1e-3 over rows with a visible key; -inf elsewhere
  dq, dk, dv   ||gpu - ref||_F / ||ref||_F <= 2e-2 over the whole tensor, and
               no head-dim column's error beyond its even share of that bound
               (check_grad_columns): a fault confined to a few columns (a
               stale accumulator register, say) stays under the whole-tensor
               norm but not under its column's share
"""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import exact_attention_varlen_amd as A
import workloads as W

OUT_MAX_ABS = 1e-2
OUT_REL_FRO = 5e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_FRO = 2e-2


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives a lost process)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def device() -> torch.device:
    return torch.device("cuda:0")


def to_dev(inp: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    dev = device()
    return {k: v.to(dev) for k, v in inp.items()}


def window_of(wl: W.Workload):
    return (-1, -1) if wl.window is None else tuple(wl.window)


def gpu_fwd(wl: W.Workload, d: Dict[str, torch.Tensor], return_lse: bool = True):
    return A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                             wl.max_seqlen_k, wl.softmax_scale, wl.causal, return_lse=return_lse,
                             window_size=window_of(wl))


def gpu_bwd(wl: W.Workload, d: Dict[str, torch.Tensor], out, lse, stored_ds: bool = False):
    """The backward through the C ABI: attn_varlen_bwd (dQ recomputes dS), or with
    stored_ds attn_varlen_bwd_stored_ds."""
    return A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                             wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal,
                             window_size=window_of(wl), stored_ds=stored_ds)


def bwd_paths(wl: W.Workload):
    """Backward paths to check for a workload: the recomputing dQ (the default),
    plus the stored-dS one where it is available (head dims 64 / 128)."""
    ds = A.attn_varlen_bwd_ds_workspace_size(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.max_seqlen_q,
                                             wl.max_seqlen_k, wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    return [False, True] if ds > 0 else [False]


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def check_out(x: np.ndarray, ref: np.ndarray, what: str = "out"):
    """O against the exact result: max-abs 1e-2 and rel-Frobenius 5e-3. Where
    |ref| >= 4 half a bf16 spacing (2^-6 and up) already exceeds 1e-2, so no bf16
    output can meet the absolute bound there; such elements (rows with one or two
    visible keys hold single V values, and peaked rows come close to them) may
    differ by 1e-2 beyond half a bf16 spacing. Every other element keeps the
    plain 1e-2."""
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = np.abs(x - ref)
    allow = np.where(np.abs(ref) >= 4.0, bf16_half_ulp(ref), 0.0) if x.size else 0.0
    mabs = float((err - allow).max()) if x.size else 0.0
    rf = rel_fro(x, ref)
    assert mabs <= OUT_MAX_ABS, f"{what}: max-abs {mabs:.3e} > {OUT_MAX_ABS} (beyond bf16 rounding where |O| >= 4)"
    assert rf <= OUT_REL_FRO, f"{what}: rel-Frobenius {rf:.3e} > {OUT_REL_FRO}"
    return mabs, rf


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 values (8 significant bits) at |ref|: the
    closest a bf16 output can be to an exact value of that size."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 8)


def check_out_rounded(x: np.ndarray, ref: np.ndarray, what: str = "out"):
    """The output check for attention so peaked that |O| reaches 4 or more. There
    the bf16 spacing alone exceeds the 1e-2 absolute bound, so each element may
    differ from the exact value by 1e-2 beyond half a bf16 spacing. The
    rel-Frobenius bound is unchanged."""
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = np.abs(x - ref)
    excess = float((err - bf16_half_ulp(ref)).max()) if x.size else 0.0
    assert excess <= OUT_MAX_ABS, f"{what}: {excess:.3e} beyond half a bf16 spacing > {OUT_MAX_ABS}"
    rf = rel_fro(x, ref)
    assert rf <= OUT_REL_FRO, f"{what}: rel-Frobenius {rf:.3e} > {OUT_REL_FRO}"
    return excess, rf


def check_lse(x: np.ndarray, ref: np.ndarray, what: str = "lse"):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), f"{what}: finite pattern differs"
    assert np.all(x[~fin] == -np.inf), f"{what}: rows without a visible key must be -inf"
    mabs = float(np.abs(x[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert mabs <= LSE_MAX_ABS, f"{what}: max-abs {mabs:.3e} > {LSE_MAX_ABS}"
    return mabs


def check_grad(x: np.ndarray, ref: np.ndarray, what: str):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    rf = rel_fro(x, ref)
    assert rf <= GRAD_REL_FRO, f"{what}: rel-Frobenius {rf:.3e} > {GRAD_REL_FRO}"
    check_grad_columns(x, ref, what)
    return rf


GRAD_ZERO_ABS = 1e-5


def check_grad_columns(x: np.ndarray, ref: np.ndarray, what: str) -> float:
    """The gradient bound applied to each head-dim column of a (rows, heads, D)
    tensor: ||x_d - ref_d|| <= 2e-2 * ||ref||_F / sqrt(D) + 1e-5 * sqrt(n), for
    every d (n = rows x heads). The first term is the whole-tensor bound spread
    evenly over the columns, so the check implies the whole-tensor one and adds
    that no column may take more than its share; a column-confined fault (a
    stale accumulator register corrupting a few d, say) fails it even when the
    whole-tensor norm hides it. Each column is measured against the tensor's
    column scale rather than its own norm: with few contributing rows a
    column's exact values can nearly cancel while its rounding does not, which
    makes its own-norm ratio meaningless. The 1e-5 term covers exact zeros (a
    row whose only visible key gives P = 1 has dS = 0), where summation order
    leaves ~1e-7."""
    if x.ndim != 3 or x.size == 0:
        return 0.0
    err = np.sqrt(((x - ref) ** 2).sum(axis=(0, 1)))
    share = np.linalg.norm(ref) / np.sqrt(x.shape[2])
    floor = GRAD_ZERO_ABS * np.sqrt(x.shape[0] * x.shape[1])
    if share == 0:
        assert np.all(np.abs(x) <= GRAD_ZERO_ABS), f"{what}: non-zero values where the gradient is exactly zero"
        return 0.0
    col = (err - floor) / share
    worst = int(np.argmax(col))
    assert col[worst] <= GRAD_REL_FRO, (f"{what}: head-dim column {worst} error {col[worst]:.3e} of the column "
                                        f"scale (beyond the 1e-5 rounding floor) > {GRAD_REL_FRO}")
    return float(col[worst])


def sample_rows(cu, per_seq: int = 6, extra: int = 64, seed: int = 0, tail_only: bool = False,
                tail: int = 256) -> np.ndarray:
    """Deterministic query/key rows: each sequence's edges and middle, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    total = cu[-1]
    for b in range(len(cu) - 1):
        c, L = cu[b], cu[b + 1] - cu[b]
        if L == 0:
            continue
        if tail_only:
            lo = max(0, L - tail)
            cand = [L - 1, L - 2, lo, (lo + L) // 2]
        else:
            cand = [0, 1, L // 3, L // 2, L - 2, L - 1]
        for x in cand[:per_seq]:
            if 0 <= x < L:
                rows.add(c + x)
    if extra and total > 0:
        if tail_only:
            pool = np.concatenate([np.arange(max(cu[b], cu[b + 1] - tail), cu[b + 1]) for b in range(len(cu) - 1)])
            pick = rng.choice(pool, size=min(extra, pool.size), replace=False) if pool.size else []
        else:
            pick = rng.choice(total, size=min(extra, total), replace=False)
        rows.update(int(x) for x in pick)
    return np.array(sorted(rows), dtype=np.int64)


def band_subsequence(L: int, s: int, n: int, left: int, right: int):
    """Tokens [a, e) of a sequence of L queries and L keys that hold, for a band of
    `left` keys before and `right` after each query's diagonal (right = 0 when
    causal), every key that query rows [s, s + n) see, every query that sees keys
    [s, s + n), and every key such a query sees. On that sub-sequence the oracle
    gives the full problem's O, LSE and dQ of rows [s, s + n) and dK, dV of keys
    [s, s + n) exactly: the queries and keys involved see the same sets."""
    assert left >= 0 and right >= 0 and 0 <= s and s + n <= L
    return max(0, s - left - right), min(L, s + n + left + right)
