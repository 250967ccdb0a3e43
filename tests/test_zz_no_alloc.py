"""The allocation-free backward (attn_varlen_bwd_noalloc, static device scratch)
against the allocating one (attn_varlen_bwd with the recomputing backward's
workspace) through the C ABI: bit-identical
gradients, over calls in a row on one GPU whose problems shrink, so that each
call finds the previous call's contents in the scratch."""
import pytest
import torch

import exact_attention_varlen_amd as A
import oracle.attention as O
import workloads as W
from parity import announce, check_grad, f64, gpu_fwd, to_dev

pytestmark = pytest.mark.gpu

CALLS = [
    W.Workload("noalloc-d128-c", [700, 33, 1200, 0, 400], 8, 2, 128, True),
    W.Workload("noalloc-d256-gqa-f", [300, 190], 8, 1, 256, False),  # partial dK / dV sums in the scratch
    W.Workload("noalloc-d64-f", [150, 77], 4, 4, 64, False),
]


def test_noalloc_backward_matches_the_allocating_one():
    for wl in CALLS:
        need = A.attn_varlen_bwd_workspace_size(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.n_q_heads,
                                                wl.n_kv_heads, wl.head_dim)
        assert 0 < need <= A.NOALLOC_SCRATCH_BYTES
        d = to_dev(W.make_inputs(wl))
        announce(f"noalloc backward {wl.name}")
        out, lse = gpu_fwd(wl, d)
        # attn_varlen_bwd with the recomputing backward's workspace (the path the
        # allocation-free call takes)
        ref = A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                                wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, stored_ds=False)
        got = A.attn_varlen_bwd_noalloc(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"],
                                        d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale,
                                        wl.causal)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"{wl.name}: {name} differs from attn_varlen_bwd"


def test_noalloc_with_fewer_splits_than_the_allocating_call():
    """One query head of 128 on a single KV head and 8 key blocks: the allocating
    backward splits the dK / dV work 128 ways (partial sums of 128 MiB), the
    static scratch holds 16 of them. The allocation-free call then sums the heads
    in fewer, larger parts: the same dQ bit for bit, dK and dV against the
    oracle and, to fp32 summation order, against the allocating call."""
    wl = W.Workload("noalloc-mqa128-d128-c", [1024], 128, 1, 128, True)
    need = A.attn_varlen_bwd_workspace_size(1, wl.total_q, wl.total_k, 128, 1, 128)
    assert need > A.NOALLOC_SCRATCH_BYTES
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    announce(f"noalloc backward with fewer splits {wl.name}")
    out, lse = gpu_fwd(wl, d)
    ref = A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                            wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, stored_ds=False)
    got = A.attn_varlen_bwd_noalloc(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"],
                                    d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0])
    for a, b in zip(got[1:], ref[1:]):
        rel = float((a.float() - b.float()).norm() / b.float().norm())
        assert rel < 5e-3, rel
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    rq, rk, rv = O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do)
    check_grad(f64(got[1]), rk, "dk (noalloc)")
    check_grad(f64(got[2]), rv, "dv (noalloc)")
