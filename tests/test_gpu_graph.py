"""HIP-graph capture of the forward + backward calls: every replay must equal
the eager result bit for bit, with eager work and synchronisations between the
replays (the benchmark times graph replays)."""
import pytest
import torch

import exact_attention_varlen_amd as A
import workloads as W
from parity import announce, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [W.Workload("graph-causal-d128", [300, 77, 900], 8, 2, 128, True),
                                W.Workload("graph-full-d64", [500, 260], 4, 4, 64, False),
                                W.Workload("graph-causal-d256", [200, 333], 8, 1, 256, True)],
                         ids=lambda w: w.name)
def test_graph_replays_match_eager(wl):
    d = to_dev(W.make_inputs(wl))
    dev = d["q"].device
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    ws = torch.empty(A.attn_varlen_bwd_workspace_size(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.n_q_heads,
                                                      wl.n_kv_heads, wl.head_dim), dtype=torch.uint8, device=dev)

    def step():
        A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                          wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out, lse=lse)
        A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                          wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv,
                          workspace=ws)

    announce(f"graph eager {wl.name}")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    announce(f"graph capture {wl.name}")
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, dq, dk, dv):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        announce(f"graph replay {rep} {wl.name}")
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager result"


@pytest.mark.parametrize("wl,splits", [
    (W.Workload("graph-split-window-d128", [130, 700], 8, 2, 128, True, seqlens_k=[2000, 700], window=(300, -1)), 4),
    (W.Workload("graph-split-d256", [64, 1], 8, 1, 256, False, seqlens_k=[3000, 900]), 6),
], ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_graph_replays_match_eager_splitkv_window(wl, splits):
    d = to_dev(W.make_inputs(wl))
    dev = d["q"].device
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    ws = torch.empty(A.attn_varlen_bwd_workspace_size(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.n_q_heads,
                                                      wl.n_kv_heads, wl.head_dim), dtype=torch.uint8, device=dev)
    wsf = torch.empty(A.attn_varlen_fwd_splitkv_workspace_size(wl.total_q, wl.n_q_heads, wl.head_dim, splits),
                      dtype=torch.uint8, device=dev)
    win = wl.window or (-1, -1)

    def step():
        A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                          wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out, lse=lse, window_size=win,
                          num_splits=splits, workspace=wsf)
        A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                          wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, wl.causal, dq=dq, dk=dk, dv=dv,
                          workspace=ws, window_size=win)

    announce(f"graph eager {wl.name} splits={splits}")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    announce(f"graph capture {wl.name}")
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, dq, dk, dv, wsf):
            t.zero_()  # eager work between replays, partial results cleared too
        torch.cuda.synchronize()
        announce(f"graph replay {rep} {wl.name}")
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager result"


def test_graph_replays_match_eager_persistent():
    wl = W.Workload("graph-persistent-d128", [300, 77, 900], 8, 2, 128, True)
    d = to_dev(W.make_inputs(wl, with_dout=False))
    dev = d["q"].device
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.n_q_heads, wl.total_q), dtype=torch.float32, device=dev)
    sched = torch.zeros(A.SCHED_BYTES, dtype=torch.uint8, device=dev)

    def fwd():
        A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                          wl.max_seqlen_k, wl.softmax_scale, wl.causal, out=out, lse=lse, persistent=True,
                          sched=sched)

    announce(f"graph eager {wl.name}")
    fwd()
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    announce(f"graph capture {wl.name}")
    with torch.cuda.graph(g, stream=stream):
        fwd()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        announce(f"graph replay {rep} {wl.name}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep} differs"
        assert int(sched.count_nonzero()) == 0
