"""Sequences at the library's size limit, on the GPU, against the float64 oracle.

Within one sequence the kernels address rows with 32-bit buffer offsets below
2 GiB, so the library accepts a sequence when its rows plus the tiles' overrun
past its end span less than 2 GiB: (max_seqlen_q + 128) * Hq * head_dim * 2 and
(max_seqlen_k + 64) * Hkv * head_dim * 2 bytes below 2^31 (the dK / dV kernel's
query steps are 128 rows, key tiles 64). Each case packs the longest sequence
that limit allows
and a second one whose rows run past the 2 GiB mark of the query tensor, so both
the largest in-sequence offsets and 64-bit base addresses are exercised.

A local window keeps the work small (each query sees a band of at most a few
hundred keys), which also lets the oracle run on a sub-sequence around each
compared range (parity.band_subsequence, pinned on the CPU against the oracle
on whole sequences): it gives exactly the full problem's O, LSE and dQ of the
compared rows and dK, dV of the compared keys.
"""
import pytest
import torch

import oracle.attention as O
import workloads as W
from parity import announce, band_subsequence, check_grad, check_lse, check_out, f64, gpu_bwd, gpu_fwd, to_dev

pytestmark = pytest.mark.gpu


def longest_sequence(heads: int, head_dim: int, overrun: int) -> int:
    """The longest sequence the library accepts for this row pitch and tile overrun."""
    return ((1 << 31) - 1) // (heads * head_dim * 2) - overrun


# name, head_dim, query heads, KV heads, causal, window (left, right), length of the second sequence
CASES = [
    ("d128-gqa32/8-causal-left192", 128, 32, 8, True, (192, -1), 3000),
    ("d256-gqa8/1-band100/60", 256, 8, 1, False, (100, 60), 2500),
    ("d64-mha16-causal-left64", 64, 16, 16, True, (64, -1), 3000),
]
ROWS = 256


def regions(lengths):
    """(sequence, first row) of the compared row / key ranges: start, middle and end
    of the long sequence, and the end of the second one (past 2 GiB)."""
    L0, L1 = lengths
    return [(0, 0), (0, L0 // 2 + 37), (0, L0 - ROWS), (1, L1 - ROWS)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parity_at_the_size_limit(case):
    name, D, Hq, Hkv, causal, window, tail = case
    L = min(longest_sequence(Hq, D, 128), longest_sequence(Hkv, D, 64))
    wl = W.Workload(f"maxsize-{name}", [L, tail], Hq, Hkv, D, causal, window=window, seed=11)
    pitch = Hq * D * 2  # bytes per query row
    assert (L + 128) * pitch < (1 << 31) <= (L + 129) * pitch
    # the compared rows of the second sequence lie past the 2 GiB mark of the query tensor
    assert (wl.cu_seqlens_q[1] + tail - ROWS) * pitch >= (1 << 31)
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    announce(f"size limit {wl.name}: lengths {wl.seqlens_q}, forward and backward")
    out, lse = gpu_fwd(wl, d)
    dq, dk, dv = gpu_bwd(wl, d, out, lse)
    torch.cuda.synchronize()

    left = window[0]
    right = 0 if causal else window[1]
    assert left >= 0 and right >= 0
    cu = wl.cu_seqlens_q
    for b, s in regions(wl.seqlens_q):
        a, e = band_subsequence(wl.seqlens_q[b], s, ROWS, left, right)
        g0, g1 = cu[b] + a, cu[b] + e  # the sub-sequence's global tokens
        sub = {k: W.to_f64(inp[k][g0:g1]) for k in ("q", "k", "v", "dout")}
        cs = [0, e - a]
        o_ref, lse_ref = O.forward(sub["q"], sub["k"], sub["v"], cs, cs, wl.softmax_scale, causal, window=window)
        dq_ref, dk_ref, dv_ref = O.backward(sub["q"], sub["k"], sub["v"], cs, cs, wl.softmax_scale, causal,
                                            sub["dout"], window=window)
        r0, r1 = s - a, s - a + ROWS  # the compared rows within the sub-sequence
        t0, t1 = cu[b] + s, cu[b] + s + ROWS  # and within the packed batch
        what = f"{wl.name} seq {b} rows {s}..{s + ROWS}"
        check_out(f64(out[t0:t1]), o_ref[r0:r1], f"out ({what})")
        check_lse(f64(lse[:, t0:t1]), lse_ref[:, r0:r1], f"lse ({what})")
        check_grad(f64(dq[t0:t1]), dq_ref[r0:r1], f"dq ({what})")
        check_grad(f64(dk[t0:t1]), dk_ref[r0:r1], f"dk ({what})")
        check_grad(f64(dv[t0:t1]), dv_ref[r0:r1], f"dv ({what})")
    del d, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
