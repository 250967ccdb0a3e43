"""Runs the float64 oracle on independent pieces of a problem, in threads.

Attention of one query head over one packed sequence depends only on that
head's queries and its KV head's keys and values; the KV gradients of a group
are the sums of its query heads' contributions. So the oracle can be called on
each (sequence, query head) piece as a one-head problem and the results put
back together: the same definition, with no step of the arithmetic changed.
NumPy releases the GIL inside its element-wise loops and BLAS, so the pieces run
in parallel threads (each with one BLAS thread). This is test plumbing around
`oracle.attention`; it computes nothing itself beyond assembling the pieces and
summing the KV gradients of a group's heads in head order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

import oracle.attention as O

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - then each piece uses the BLAS default
    threadpool_limits = None


def workers() -> int:
    """Host threads for the pieces: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunk(Lk: int) -> int:
    """Query rows per oracle chunk: about 2^25 scores (256 MiB of float64) at a time."""
    return int(max(64, min(2048, (1 << 25) // max(1, Lk))))


def _pieces(cu_q, cu_k, Hq):
    for b in range(len(cu_q) - 1):
        if cu_q[b + 1] > cu_q[b]:
            for h in range(Hq):
                yield b, h


def _run(fn, items, nthreads: Optional[int] = None):
    n = nthreads or workers()
    if threadpool_limits is not None:
        with threadpool_limits(1):
            with ThreadPoolExecutor(n) as ex:
                return list(ex.map(fn, items))
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def _piece_args(q, k, v, cu_q, cu_k, b, h):
    r = q.shape[1] // k.shape[1]
    g = O.kv_head_of(h, q.shape[1], k.shape[1])
    assert g == h // r
    cq, cq1, ck, ck1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
    return (q[cq:cq1, h:h + 1], k[ck:ck1, g:g + 1], v[ck:ck1, g:g + 1], [0, cq1 - cq], [0, ck1 - ck], g)


def forward(q, k, v, cu_q: Sequence[int], cu_k: Sequence[int], scale: float, causal: bool, window=None,
            nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """`oracle.attention.forward`, piece by piece."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Tq, Hq, D = q.shape
    out = np.zeros((Tq, Hq, D))
    lse = np.full((Hq, Tq), -np.inf)

    def one(bh):
        b, h = bh
        qp, kp, vp, cq, ck, _ = _piece_args(q, k, v, cu_q, cu_k, b, h)
        return O.forward(qp, kp, vp, cq, ck, scale, causal, chunk=_chunk(ck[1]), window=window)

    items = list(_pieces(cu_q, cu_k, Hq))
    for (b, h), (o, l) in zip(items, _run(one, items, nthreads)):
        out[cu_q[b]:cu_q[b + 1], h] = o[:, 0]
        lse[h, cu_q[b]:cu_q[b + 1]] = l[0]
    return out, lse


def backward(q, k, v, cu_q, cu_k, scale: float, causal: bool, dout, window=None,
             nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """`oracle.attention.backward`, piece by piece; a KV head's gradients are the
    sum of its query heads' pieces, added in head order."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Hq = q.shape[1]
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)

    def one(bh):
        b, h = bh
        qp, kp, vp, cq, ck, _ = _piece_args(q, k, v, cu_q, cu_k, b, h)
        dop = dout[cu_q[b]:cu_q[b + 1], h:h + 1]
        return O.backward(qp, kp, vp, cq, ck, scale, causal, dop, chunk=_chunk(ck[1]), window=window)

    items = list(_pieces(cu_q, cu_k, Hq))
    for (b, h), (gq, gk, gv) in zip(items, _run(one, items, nthreads)):
        g = O.kv_head_of(h, Hq, k.shape[1])
        dq[cu_q[b]:cu_q[b + 1], h] = gq[:, 0]
        dk[cu_k[b]:cu_k[b + 1], g] += gk[:, 0]
        dv[cu_k[b]:cu_k[b + 1], g] += gv[:, 0]
    return dq, dk, dv


def backward_dkdv_rows(q, k, v, cu_q, cu_k, scale: float, causal: bool, dout, key_rows, window=None,
                       nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """`oracle.attention.backward_dkdv_rows`, piece by piece (sorted unique key rows)."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    key_rows = np.sort(np.unique(np.asarray(key_rows, dtype=np.int64)))
    seq = O.token_sequence(cu_k, key_rows)
    dk = np.zeros((len(key_rows), Hkv, D))
    dv = np.zeros((len(key_rows), Hkv, D))
    items: List[Tuple[int, int]] = [(int(b), h) for b in np.unique(seq) for h in range(Hq)
                                    if cu_q[int(b) + 1] > cu_q[int(b)]]

    def one(bh):
        b, h = bh
        qp, kp, vp, cq, ck, _ = _piece_args(q, k, v, cu_q, cu_k, b, h)
        dop = dout[cu_q[b]:cu_q[b + 1], h:h + 1]
        local = key_rows[seq == b] - cu_k[b]
        return O.backward_dkdv_rows(qp, kp, vp, cq, ck, scale, causal, dop, local, chunk=_chunk(ck[1]),
                                    window=window)

    for (b, h), (rows, gk, gv) in zip(items, _run(one, items, nthreads)):
        g = O.kv_head_of(h, Hq, Hkv)
        sel = np.nonzero(seq == b)[0]
        assert np.array_equal(rows, key_rows[sel] - cu_k[b])
        dk[sel, g] += gk[:, 0]
        dv[sel, g] += gv[:, 0]
    return key_rows, dk, dv
