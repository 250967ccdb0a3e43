"""Host-side checks of bench.py (CPU only): argument handling, the accounted-work
formulas and the oracle timing table's arithmetic."""
import json
import re

import pytest

import bench
import workloads as W


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_kernel_flop_counts():
    wl = W.packed_16k()
    pairs = sum(L * L for L in wl.seqlens_q) * 0.5
    base = pairs * wl.n_q_heads * wl.head_dim
    assert bench.kernel_flop("attn_fwd", wl) == pytest.approx(4 * base)
    assert bench.kernel_flop("attn_bwd_dq", wl) == pytest.approx(6 * base)
    assert bench.kernel_flop("attn_bwd_dkdv", wl) == pytest.approx(8 * base)
    # the accounted forward (the pages' formula) is the forward kernel's work
    assert wl.accounted_fwd_flop() == pytest.approx(bench.kernel_flop("attn_fwd", wl))


def test_oracle_table_lines(monkeypatch, capsys):
    causal = W.Workload("small-causal", [1000, 600], 4, 2, 64, True)
    full = W.Workload("small-full", [1500], 2, 1, 64, False)
    monkeypatch.setattr(W, "all_configs", lambda: [W.tiny(False), causal])
    monkeypatch.setattr(W, "single_16k_full", lambda: full)
    # tiny (0.5 GFLOP forward+backward) runs whole; the other two are sampled
    assert bench.oracle_table(budget_s=0.05, max_sample_len=128, whole_flop=1e9) == 0
    rows = [json.loads(l) for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert [r["config"] for r in rows] == ["tiny-varlen-gqa-d64-full", "small-causal", "small-full"]
    assert [r["kind"] for r in rows] == ["measured", "extrapolated", "extrapolated"]
    for r, wl in zip(rows, [W.tiny(False), causal, full]):
        assert r["oracle_fwd_s"] > 0 and r["oracle_fwdbwd_s"] >= r["oracle_fwd_s"]
        fl = wl.accounted_fwd_flop()
        assert r["accounted_fwd_gflop"] == pytest.approx(fl / 1e9)
        assert r["oracle_fwd_gflops"] == pytest.approx(fl / r["oracle_fwd_s"] / 1e9)
        assert r["oracle_fwdbwd_gflops"] == pytest.approx(3.5 * fl / r["oracle_fwdbwd_s"] / 1e9)
        if r["kind"] == "extrapolated":
            L, heads = (int(x) for x in re.match(r"sequence 0 cut to (\d+) tokens, (\d+) of", r["sample"]).groups())
            assert L == 128 and 1 <= heads <= wl.n_q_heads
            sample_fl = heads * 4.0 * L * L * wl.head_dim * (0.5 if wl.causal else 1.0)
            # the full time is the config's work at the sample's rate
            assert r["oracle_fwd_s"] == pytest.approx(r["sample_fwd_s"] * fl / sample_fl)
            assert r["oracle_fwdbwd_s"] == pytest.approx(r["sample_fwdbwd_s"] * fl / sample_fl)


def test_named_workloads_for_profiling():
    assert bench.named_workload("2x16384-mha16-d64-full").backward is False
    assert bench.named_workload("single-16384-gqa32/8-d128-full").head_dim == 128
    with pytest.raises(SystemExit):
        bench.named_workload("no-such-workload")
