"""Writes the stored dK / dV rows of the longest workloads (tests/golden/dkdv_*.npz).

The GPU parity tests compare dK and dV element by element on sampled key rows
at full size. For sequences of 64K and 128K tokens the oracle needs every query
row's full softmax (its LSE and Delta) before any key's gradient is known, a full
float64 pass that takes far longer than a test should. This script does that
pass once and stores the result; the tests check a checksum of the inputs first.

It calls only `oracle.attention` (through tests/oracle_pool.py, which runs the
oracle per query head in threads) and `workloads` (shapes and the seeded draw).
Key rows: the first 256 keys of the sequence (they are seen by every query row,
the longest sums a causal backward forms) and 64 more drawn at random from the
rest, seed 0. The keys at the end of a causal sequence are cheap and are
computed in the test itself.

Usage (about an hour on 8 cores for all three):
    python tests/golden/make_dkdv_golden.py [name ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path[:0] = [ROOT, os.path.dirname(HERE)]

import oracle_pool as P  # noqa: E402
import workloads as W  # noqa: E402

EARLY = 256
SPREAD = 64


def golden_workloads():
    return {
        "single-65536-gqa32-8-d128-causal": W.long_65k(),
        "1x131072-gqa8-1-d256-full": W.hd256_gqa(1, 131072, False),
        "1x131072-gqa8-1-d256-causal": W.hd256_gqa(1, 131072, True),
    }


def golden_key_rows(wl: W.Workload) -> np.ndarray:
    rng = np.random.default_rng(0)
    rows = []
    for b in range(len(wl.seqlens_k)):
        c, L = wl.cu_seqlens_k[b], wl.seqlens_k[b]
        rows.extend(range(c, c + min(EARLY, L)))
        if L > EARLY:
            rows.extend((c + rng.choice(np.arange(EARLY, L), size=min(SPREAD, L - EARLY), replace=False)).tolist())
    return np.array(sorted(set(int(x) for x in rows)), dtype=np.int64)


def path_of(name: str) -> str:
    return os.path.join(HERE, f"dkdv_{name}.npz")


def make(name: str, wl: W.Workload) -> None:
    t0 = time.time()
    inp = W.make_inputs(wl)
    sha = W.inputs_sha256(inp)
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    del inp
    rows = golden_key_rows(wl)
    print(f"{name}: {len(rows)} key rows, {P.workers()} threads", flush=True)
    r, dk, dv = P.backward_dkdv_rows(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do,
                                     rows, window=wl.window)
    assert np.array_equal(r, rows)
    np.savez_compressed(path_of(name), workload=np.array(wl.name), input_sha256=np.array(sha), key_rows=rows,
                        dk=dk.astype(np.float32), dv=dv.astype(np.float32))
    print(f"{name}: written in {time.time() - t0:.0f} s", flush=True)


def main(argv):
    todo = golden_workloads()
    names = argv or list(todo)
    for n in names:
        make(n, todo[n])
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
