"""fp64 CPU oracle for exact attention over packed variable-length sequences.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
module; only the tests, the smoke check and the bench's CPU-baseline leg do. It
shares no code with the HIP kernels or their host library.

What it computes is the plain definition of scaled-dot-product attention, written
out in float64 NumPy, one packed sequence and one query head at a time:

* Exact attention ``softmax(Q K^T * scale + mask) V`` is what the pages validate
  their kernels against ("[FA4/B200] return_lse=True makes D64 forward about 19%
  faster", repro script, ``main``: the FA4 output is compared with PyTorch's
  ``scaled_dot_product_attention``).
* Packed variable-length batches are delimited by cumulative sequence lengths and
  every sequence attends only within itself ("FA2 vs NATTEN on A100" issue,
  benchmark script ``call``: ``cumulative_seqlen_Q`` / ``cumulative_seqlen_KV`` /
  ``max_seqlen``; FlashAttention repository guide, Public API,
  ``flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, ...)``).
* Grouped-query attention: 32 query heads share 8 KV heads in the A100 issue's
  script; the repository guide's Other Components describe packing several query
  heads per KV head. Reading: query head ``h`` uses KV head ``h // (Hq // Hkv)``
  (contiguous groups, the same as repeating each KV head ``Hq // Hkv`` times).
* The log-sum-exp output: the LSE repro allocates an fp32 ``lse`` buffer of shape
  (batch, heads, seqlen) beside ``out`` (``make_call``). Reading: LSE is the
  natural log of the sum of exp of the scaled, masked scores; its varlen layout is
  ``(Hq, total_q)``.
* Causal masking (the head_dim=256 regression check's tables have a causal column;
  the repository guide's Core Abstractions list causal masks). Reading: key ``j``
  of a sequence is visible to query ``i`` when ``j <= i + Lk - Lq`` (aligned at the
  bottom-right; with ``Lq == Lk`` this is the lower triangle with the diagonal).
* Local (sliding-window) attention: the repository guide's Public API lists
  ``window_size_left/right`` among the key parameters and Core Abstractions list a
  local / sliding-window mask (``mask.py``); the pages define neither. Reading: with
  ``window = (left, right)``, key ``j`` is visible to query ``i`` when
  ``i + Lk - Lq - left <= j <= i + Lk - Lq + right``, a negative bound meaning
  unbounded on that side; ``causal`` is the window's right bound 0, and the two
  masks combine by intersection. ``(-1, -1)`` is full attention.
* A query row with no visible key (possible when causal with ``Lq > Lk``, with a
  window that leaves it no key, or ``Lk == 0``) has output 0, LSE ``-inf`` and
  contributes no gradient.

The backward is the analytic gradient of the same definition, given ``dout``:
``dP = dO V^T``; ``Delta_i = sum_j P_ij dP_ij``; ``dS = P * (dP - Delta)``;
``dQ = scale * dS K``; ``dK = scale * dS^T Q`` and ``dV = P^T dO``, each summed
over the query heads of a KV head's group (FlashAttention repository guide,
Backward Kernels: a preprocess, a main kernel and a postprocess; the gradient
itself is the textbook derivative of softmax attention).

Rows are processed in chunks of at most ``chunk`` queries, each against its full
key row, so every softmax still runs over its whole row: this is the definition,
not a tiled or online algorithm.

Every function here is pinned by tests that do not re-type these formulas:
closed forms, finite differences, PyTorch's float64 SDPA special case, a hand-worked
example and invariants (see ``tests/test_oracle.py``).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "kv_head_of",
    "visible",
    "forward",
    "backward",
    "probabilities",
    "forward_rows",
    "backward_dq_rows",
    "backward_dkdv_rows",
    "token_sequence",
]


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head used by query head ``h``: contiguous groups of ``Hq // Hkv`` query heads."""
    return h // (n_q_heads // n_kv_heads)


Window = Optional[Tuple[int, int]]


def visible(Lq: int, Lk: int, causal: bool, rows: Optional[np.ndarray] = None, window: Window = None) -> np.ndarray:
    """Boolean ``(len(rows), Lk)`` matrix: may query ``i`` of the sequence see key ``j``?"""
    i = np.arange(Lq) if rows is None else np.asarray(rows)
    j = np.arange(Lk)
    left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    diag = i[:, None] + (Lk - Lq)  # the key aligned with query i (bottom-right)
    ok = np.ones((i.shape[0], Lk), dtype=bool)
    if causal:
        ok &= j[None, :] <= diag
    if right >= 0:
        ok &= j[None, :] <= diag + right
    if left >= 0:
        ok &= j[None, :] >= diag - left
    return ok


def _check(q, k, v, cu_q, cu_k):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    assert q.ndim == 3 and k.ndim == 3 and v.shape == k.shape
    assert len(cu_q) == len(cu_k) and len(cu_q) >= 2
    assert cu_q[-1] == q.shape[0] and cu_k[-1] == k.shape[0]
    assert q.shape[1] % k.shape[1] == 0 and q.shape[2] == k.shape[2]
    return q, k, v, cu_q, cu_k


def _row_softmax(s: np.ndarray, vis: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax of each row over its visible entries; returns (P, LSE).

    ``LSE = m + log(sum exp(s - m))`` with ``m`` the row's largest visible score.
    A row with nothing visible gets ``P = 0`` and ``LSE = -inf``.
    """
    s_vis = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s_vis.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s_vis - m[:, None]), 0.0)
    z = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(any_vis, m + np.log(np.where(any_vis, z, 1.0)), -np.inf)
        p = np.where(any_vis[:, None], e / np.where(any_vis, z, 1.0)[:, None], 0.0)
    return p, lse


def _chunks(n: int, chunk: int) -> Iterable[Tuple[int, int]]:
    for r0 in range(0, n, chunk):
        yield r0, min(n, r0 + chunk)


def forward(q, k, v, cu_q: Sequence[int], cu_k: Sequence[int], scale: float, causal: bool,
            chunk: int = 2048, window: Window = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention output ``(total_q, Hq, D)`` and LSE ``(Hq, total_q)``, both float64."""
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_q, cu_k)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    lse = np.full((Hq, Tq), -np.inf, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        if Lq == 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kb = k[ck:ck + Lk, g, :]
            vb = v[ck:ck + Lk, g, :]
            for r0, r1 in _chunks(Lq, chunk):
                s = scale * (q[cq + r0:cq + r1, h, :] @ kb.T)
                p, l = _row_softmax(s, visible(Lq, Lk, causal, np.arange(r0, r1), window))
                out[cq + r0:cq + r1, h, :] = p @ vb
                lse[h, cq + r0:cq + r1] = l
    return out, lse


def probabilities(q, k, cu_q, cu_k, scale: float, causal: bool, b: int, h: int, window: Window = None) -> np.ndarray:
    """The full ``(Lq, Lk)`` attention matrix P of sequence ``b``, query head ``h`` (small cases)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    cq, Lq = int(cu_q[b]), int(cu_q[b + 1]) - int(cu_q[b])
    ck, Lk = int(cu_k[b]), int(cu_k[b + 1]) - int(cu_k[b])
    g = kv_head_of(h, Hq, Hkv)
    s = scale * (q[cq:cq + Lq, h, :] @ k[ck:ck + Lk, g, :].T)
    p, _ = _row_softmax(s, visible(Lq, Lk, causal, None, window))
    return p


def backward(q, k, v, cu_q, cu_k, scale: float, causal: bool, dout,
             chunk: int = 2048, window: Window = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients ``(dq, dk, dv)`` of ``sum(dout * out)`` with respect to q, k, v (float64)."""
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_q, cu_k)
    dout = np.asarray(dout, dtype=np.float64)
    assert dout.shape == q.shape
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        if Lq == 0 or Lk == 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kb = k[ck:ck + Lk, g, :]
            vb = v[ck:ck + Lk, g, :]
            for r0, r1 in _chunks(Lq, chunk):
                qr = q[cq + r0:cq + r1, h, :]
                dor = dout[cq + r0:cq + r1, h, :]
                s = scale * (qr @ kb.T)
                p, _ = _row_softmax(s, visible(Lq, Lk, causal, np.arange(r0, r1), window))
                dp = dor @ vb.T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[cq + r0:cq + r1, h, :] = scale * (ds @ kb)
                dk[ck:ck + Lk, g, :] += scale * (ds.T @ qr)
                dv[ck:ck + Lk, g, :] += p.T @ dor
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Row-sampled forms for sequences too long for the full oracle. Each query row's
# output, LSE and dQ depend only on that row and its sequence's keys, so they are
# computed exactly, one row set at a time, by the same definition as above.
# ---------------------------------------------------------------------------

def token_sequence(cu: Sequence[int], tokens: np.ndarray) -> np.ndarray:
    """Index of the packed sequence that holds each global token index."""
    cu = np.asarray([int(x) for x in cu])
    return np.searchsorted(cu, np.asarray(tokens), side="right") - 1


def _rows_by_sequence(cu_q, rows):
    rows = np.sort(np.unique(np.asarray(rows, dtype=np.int64)))
    seq = token_sequence(cu_q, rows)
    for b in np.unique(seq):
        yield int(b), rows[seq == b]


def forward_rows(q, k, v, cu_q, cu_k, scale: float, causal: bool, rows,
                 window: Window = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Output and LSE of the given global query rows only.

    Returns ``(rows_sorted, out_rows (n, Hq, D), lse_rows (Hq, n))``.
    """
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_q, cu_k)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    all_rows, outs, lses = [], [], []
    for b, rws in _rows_by_sequence(cu_q, rows):
        cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        local = rws - cq
        o = np.zeros((len(rws), Hq, D))
        l = np.full((Hq, len(rws)), -np.inf)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            s = scale * (q[rws, h, :] @ k[ck:ck + Lk, g, :].T)
            p, lh = _row_softmax(s, visible(Lq, Lk, causal, local, window))
            o[:, h, :] = p @ v[ck:ck + Lk, g, :]
            l[h] = lh
        all_rows.append(rws)
        outs.append(o)
        lses.append(l)
    return np.concatenate(all_rows), np.concatenate(outs, axis=0), np.concatenate(lses, axis=1)


def backward_dq_rows(q, k, v, cu_q, cu_k, scale: float, causal: bool, dout, rows,
                     window: Window = None) -> Tuple[np.ndarray, np.ndarray]:
    """dQ of the given global query rows only. Returns ``(rows_sorted, dq_rows (n, Hq, D))``."""
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_q, cu_k)
    dout = np.asarray(dout, dtype=np.float64)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    all_rows, dqs = [], []
    for b, rws in _rows_by_sequence(cu_q, rows):
        cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        local = rws - cq
        dq = np.zeros((len(rws), Hq, D))
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kb = k[ck:ck + Lk, g, :]
            s = scale * (q[rws, h, :] @ kb.T)
            p, _ = _row_softmax(s, visible(Lq, Lk, causal, local, window))
            dp = dout[rws, h, :] @ v[ck:ck + Lk, g, :].T
            delta = (p * dp).sum(axis=1)
            dq[:, h, :] = scale * ((p * (dp - delta[:, None])) @ kb)
        all_rows.append(rws)
        dqs.append(dq)
    return np.concatenate(all_rows), np.concatenate(dqs, axis=0)


def backward_dkdv_rows(q, k, v, cu_q, cu_k, scale: float, causal: bool, dout, key_rows,
                       chunk: int = 1024, window: Window = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dK and dV of the given global key rows only.

    Every query row that can see one of the keys is visited with its full key row
    (for its LSE and ``Delta``), so the cost is that of the query rows involved:
    cheap for keys near the end of a causal sequence, a full pass otherwise.
    Returns ``(key_rows_sorted, dk_rows (n, Hkv, D), dv_rows (n, Hkv, D))``.
    """
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_q, cu_k)
    dout = np.asarray(dout, dtype=np.float64)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    all_rows, dks, dvs = [], [], []
    for b, krws in _rows_by_sequence(cu_k, key_rows):
        cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        kloc = krws - ck
        dk = np.zeros((len(krws), Hkv, D))
        dv = np.zeros((len(krws), Hkv, D))
        # first query row that can see the earliest requested key (rows before it
        # see none of them: key j needs i >= j - (Lk - Lq) - right)
        bounds = ([0] if causal else []) + ([int(window[1])] if window is not None and int(window[1]) >= 0 else [])
        right = min(bounds) if bounds else -1
        i0 = max(0, int(kloc.min()) - (Lk - Lq) - right) if right >= 0 else 0
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kb = k[ck:ck + Lk, g, :]
            vb = v[ck:ck + Lk, g, :]
            for r0, r1 in _chunks(Lq - i0, chunk):
                rr = np.arange(i0 + r0, i0 + r1)
                qr = q[cq + rr, h, :]
                dor = dout[cq + rr, h, :]
                s = scale * (qr @ kb.T)
                p, _ = _row_softmax(s, visible(Lq, Lk, causal, rr, window))
                dp = dor @ vb.T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dk[:, g, :] += scale * (ds[:, kloc].T @ qr)
                dv[:, g, :] += p[:, kloc].T @ dor
        all_rows.append(krws)
        dks.append(dk)
        dvs.append(dv)
    return np.concatenate(all_rows), np.concatenate(dks, axis=0), np.concatenate(dvs, axis=0)
