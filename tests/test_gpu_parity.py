"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle on
the same seeded inputs, element by element, plus the bitwise and structural
checks of the kernels. Tolerances are in tests/parity.py."""
import os

import numpy as np
import pytest
import torch

import exact_attention_varlen_amd as A
import oracle.attention as O
import oracle_pool as OP
import workloads as W
from parity import (announce, bwd_paths, check_grad, check_lse, check_out, check_out_rounded, f64, gpu_bwd,
                    gpu_fwd, sample_rows, to_dev, window_of)

pytestmark = pytest.mark.gpu


def full_parity(wl: W.Workload, backward: bool = True):
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    announce(f"fwd {wl.name} seqlens_q={wl.seqlens_q} seqlens_k={wl.seqlens_k} Hq={wl.n_q_heads} "
             f"Hkv={wl.n_kv_heads} D={wl.head_dim} causal={wl.causal} window={wl.window}")
    out, lse = gpu_fwd(wl, d)
    torch.cuda.synchronize()
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    ref_o, ref_l = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal,
                             window=wl.window)
    check_out(f64(out), ref_o)
    check_lse(f64(lse), ref_l)
    if not backward:
        return
    rq, rk, rv = O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do,
                            window=wl.window)
    for path in bwd_paths(wl):
        announce(f"bwd {wl.name} stored_ds={path}")
        dq, dk, dv = gpu_bwd(wl, d, out, lse, path)
        torch.cuda.synchronize()
        check_grad(f64(dq), rq, f"dq ({path})")
        check_grad(f64(dk), rk, f"dk ({path})")
        check_grad(f64(dv), rv, f"dv ({path})")


# --------------------------------------------------------------------------
# small and medium problems: full tensors, several tiles, ragged tails
# --------------------------------------------------------------------------

SMALL = [
    W.tiny(False),
    W.tiny(True),
]
for D in (64, 128, 256):
    for c in (False, True):
        SMALL.append(W.Workload(f"ragged-d{D}-{'c' if c else 'f'}", [1, 77, 300, 513, 0, 129], 8, 2, D, c))
SMALL += [
    W.Workload("mha-d64-f", [640, 383], 4, 4, 64, False),
    W.Workload("mqa-d128-c", [257, 64, 191], 8, 1, 128, True),
    W.Workload("lq-ne-lk-d128-f", [100, 300, 5, 0], 4, 1, 128, False, seqlens_k=[250, 64, 0, 33]),
    W.Workload("lq-ne-lk-d128-c", [100, 300, 5, 0], 4, 1, 128, True, seqlens_k=[250, 64, 0, 33]),
    W.Workload("lq-ne-lk-d64-c", [129, 3, 200], 2, 2, 64, True, seqlens_k=[300, 1, 70]),
    W.Workload("lq-ne-lk-d256-c", [65, 190], 2, 1, 256, True, seqlens_k=[200, 64]),
    W.Workload("single-token-seqs-d128-c", [1, 1, 2, 1], 4, 2, 128, True),
    W.Workload("scale-zero-d64-f", [150, 90], 2, 1, 64, False, softmax_scale=0.0),
    W.Workload("scale-large-d128-c", [200], 4, 2, 128, True, softmax_scale=0.5),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_parity_small(wl):
    full_parity(wl)


# more sequences than a wave has lanes: the work-item decode then leaves its
# one-load-per-lane path (up to 64 sequences) for the general one. Ragged
# lengths including empty sequences, Lq != Lk, every head dim, both masks.
def _many_lengths(n, seed):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(0, 160, size=n)], [int(x) for x in rng.integers(0, 160, size=n)]


MANY_SEQS = []
for n, D, causal, seed in ((64, 128, True, 1), (65, 64, False, 2), (65, 128, True, 3), (150, 256, True, 4),
                           (150, 128, False, 5)):
    lq, lk = _many_lengths(n, seed)
    MANY_SEQS.append(W.Workload(f"many{n}-d{D}-{'c' if causal else 'f'}", lq, 4, 2, D, causal, seqlens_k=lk))
# Past 1024 sequences each lane of the decode owns more than 16 of them (block
# counts reloaded in rounds); 4097 makes 65 per lane, the last lane's chunk short.
for n, D, causal, seed, hi in ((1000, 128, True, 6, 90), (1500, 64, False, 7, 40), (4097, 64, True, 8, 24),
                               (4097, 256, False, 9, 12)):
    rng = np.random.default_rng(seed)
    lq = [int(x) for x in rng.integers(0, hi, size=n)]
    lk = lq if causal else [int(x) for x in rng.integers(0, hi, size=n)]
    MANY_SEQS.append(W.Workload(f"many{n}-d{D}-{'c' if causal else 'f'}", lq, 4, 2, D, causal, seqlens_k=lk))


@pytest.mark.parametrize("wl", MANY_SEQS, ids=[w.name for w in MANY_SEQS])
def test_parity_many_sequences(wl):
    full_parity(wl)


# Few KV heads and few key blocks: the head dim 64 / 128 dK / dV work splits a
# group's query heads over several items (fp32 partial sums, ordered reduce).
SPLIT_DKDV = [
    (W.Workload("mqa16-d128-c", [1500, 700], 16, 1, 128, True), 16),
    (W.Workload("mqa8-d64-f-band", [900, 600], 8, 1, 64, False, window=(100, 50)), 8),
    (W.Workload("gqa32/2-d128-f", [2048], 32, 2, 128, False), 16),
    (W.Workload("gqa8/2-d64-c-ragged", [300, 0, 77, 513], 8, 2, 64, True, seqlens_k=[300, 5, 77, 700]), 4),
]


@pytest.mark.parametrize("wl,splits", SPLIT_DKDV, ids=[w.name for w, _ in SPLIT_DKDV])
def test_parity_split_dkdv(wl, splits):
    need = A.attn_varlen_bwd_workspace_size(len(wl.seqlens_q), wl.total_q, wl.total_k, wl.n_q_heads,
                                            wl.n_kv_heads, wl.head_dim)
    planes = 2 * (-(-wl.total_q * wl.n_q_heads * 4 // 256) * 256)
    part = -(-splits * wl.total_k * wl.n_kv_heads * wl.head_dim * 4 // 256) * 256
    assert need == planes + 2 * part  # the split count this case is for
    full_parity(wl)
    d = to_dev(W.make_inputs(wl))
    out, lse = gpu_fwd(wl, d)
    announce(f"split dK/dV determinism {wl.name}")
    a = gpu_bwd(wl, d, out, lse)
    b = gpu_bwd(wl, d, out, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# local (sliding-window) attention: band (left, right) around the bottom-right
# diagonal; causal fixes right = 0. Windows narrower than a tile, wider than a
# sequence, zero-width, one-sided, and bands that leave rows without a key.
WINDOWED = []
for D in (64, 128, 256):
    for c, win in ((False, (100, 37)), (False, (17, 3)), (False, (0, 0)), (False, (130, -1)),
                   (False, (-1, 50)), (True, (64, -1)), (True, (0, -1)), (True, (200, -1)), (True, (700, 5))):
        WINDOWED.append(W.Workload(f"ragged-d{D}-{'c' if c else 'f'}-w{win[0]}_{win[1]}",
                                   [1, 77, 300, 513, 0, 129], 8, 2, D, c, window=win))
WINDOWED += [
    W.Workload("lq-ne-lk-d128-f-w20_10", [100, 300, 5, 0], 4, 1, 128, False, seqlens_k=[250, 64, 0, 33],
               window=(20, 10)),
    W.Workload("lq-ne-lk-d128-c-w50", [100, 300, 5, 0], 4, 1, 128, True, seqlens_k=[250, 64, 0, 33],
               window=(50, -1)),
    W.Workload("lq-gt-lk-d64-f-w10_5", [300, 70], 2, 2, 64, False, seqlens_k=[64, 200], window=(10, 5)),
    W.Workload("lq-ne-lk-d256-c-w33", [65, 190], 2, 1, 256, True, seqlens_k=[200, 64], window=(33, -1)),
    W.Workload("long-band-d128-c-w256", [2100, 1500], 4, 2, 128, True, window=(256, -1)),
    W.Workload("long-band-d64-f-w300_200", [1800], 4, 4, 64, False, window=(300, 200)),
]


@pytest.mark.parametrize("wl", WINDOWED, ids=[w.name for w in WINDOWED])
def test_parity_window(wl):
    full_parity(wl)


# split-KV forward: the keys of every item are cut into chunks whose partial
# results are merged; the result is the same attention (oracle), and the LSE it
# returns drives the backward like the one-pass forward's.
def split_parity(wl: W.Workload, splits: int, backward: bool = False):
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    announce(f"split-kv fwd {wl.name} splits={splits} seqlens_q={wl.seqlens_q} seqlens_k={wl.seqlens_k} "
             f"D={wl.head_dim} causal={wl.causal} window={wl.window}")
    out, lse = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                                 wl.max_seqlen_k, wl.softmax_scale, wl.causal, return_lse=True,
                                 window_size=window_of(wl), num_splits=splits)
    torch.cuda.synchronize()
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    ref_o, ref_l = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal,
                             window=wl.window)
    check_out(f64(out), ref_o)
    check_lse(f64(lse), ref_l)
    if backward:
        announce(f"bwd after split-kv fwd {wl.name}")
        dq, dk, dv = gpu_bwd(wl, d, out, lse)
        torch.cuda.synchronize()
        rq, rk, rv = O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do,
                                window=wl.window)
        check_grad(f64(dq), rq, "dq")
        check_grad(f64(dk), rk, "dk")
        check_grad(f64(dv), rv, "dv")


SPLIT_CASES = []
for D in (64, 128, 256):
    for c in (False, True):
        for sp in (2, 7):
            SPLIT_CASES.append((W.Workload(f"ragged-d{D}-{'c' if c else 'f'}", [1, 77, 300, 513, 0, 129], 8, 2, D, c),
                                sp))
SPLIT_CASES += [
    (W.Workload("chunk-vs-long-d128-c", [100, 37], 8, 2, 128, True, seqlens_k=[1500, 900]), 3),
    (W.Workload("chunk-vs-long-d128-c", [100, 37], 8, 2, 128, True, seqlens_k=[1500, 900]), 64),
    (W.Workload("lq-ne-lk-d128-f", [100, 300, 5, 0], 4, 1, 128, False, seqlens_k=[250, 64, 0, 33]), 5),
    (W.Workload("lq-gt-lk-d64-c", [300, 70], 2, 2, 64, True, seqlens_k=[64, 200]), 3),
    (W.Workload("window-d128-f-w100_37", [1, 77, 300, 513, 0, 129], 8, 2, 128, False, window=(100, 37)), 4),
    (W.Workload("window-d256-c-w200", [700, 129], 8, 2, 256, True, window=(200, -1)), 3),
    (W.Workload("window-d64-c-w64", [1200], 4, 4, 64, True, window=(64, -1)), 16),
    (W.Workload("decode-like-d256-c", [1, 1, 2, 1], 8, 1, 256, True, seqlens_k=[700, 33, 1000, 64]), 8),
]


@pytest.mark.parametrize("wl,splits", SPLIT_CASES, ids=[f"{w.name}-s{s}" for w, s in SPLIT_CASES])
def test_parity_splitkv(wl, splits):
    split_parity(wl, splits)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_splitkv_drives_backward(D):
    split_parity(W.Workload(f"split-bwd-d{D}", [300, 129, 513], 8, 2, D, True), 3, backward=True)


def test_splitkv_one_split_is_the_plain_call_and_deterministic():
    wl = W.Workload("split-one", [700, 33, 1200], 8, 2, 128, True)
    d = to_dev(W.make_inputs(wl, with_dout=False))
    announce("split-kv splits=1 vs plain, determinism")
    args = (d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k,
            wl.softmax_scale, True)
    o1, l1 = A.attn_varlen_fwd(*args, return_lse=True)
    o2, l2 = A.attn_varlen_fwd(*args, return_lse=True, num_splits=1)
    o3, l3 = A.attn_varlen_fwd(*args, return_lse=True, num_splits=5)
    o4, l4 = A.attn_varlen_fwd(*args, return_lse=True, num_splits=5)
    o5 = A.attn_varlen_fwd(*args, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    assert torch.equal(o3, o5)


# --------------------------------------------------------------------------
# full-size workloads
# --------------------------------------------------------------------------

def pooled_parity(wl: W.Workload, backward: bool = True, lse_off_too: bool = False):
    """Full-size GPU run in the bench's launch configuration; the whole output,
    LSE and gradients compared element by element with the float64 oracle (run
    per (sequence, query head) in host threads, tests/oracle_pool.py)."""
    inp = W.make_inputs(wl, with_dout=backward)
    d = to_dev(inp)
    announce(f"fwd {wl.name} (full size, full tensors)")
    out, lse = gpu_fwd(wl, d)
    out_nolse = gpu_fwd(wl, d, return_lse=False) if lse_off_too else None
    grads = []
    if backward:
        for path in bwd_paths(wl):
            announce(f"bwd {wl.name} (full size, full tensors, stored_ds={path})")
            grads.append((path, gpu_bwd(wl, d, out, lse, path)))
    torch.cuda.synchronize()
    q, k, v = (W.to_f64(inp[x]) for x in ("q", "k", "v"))
    ref_o, ref_l = OP.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal,
                              window=wl.window)
    check_out(f64(out), ref_o)
    check_lse(f64(lse), ref_l)
    if out_nolse is not None:
        check_out(f64(out_nolse), ref_o, "out (no LSE)")
    if not backward:
        return
    do = W.to_f64(inp["dout"])
    rq, rk, rv = OP.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do,
                             window=wl.window)
    for path, g in grads:
        for x, ref, name in zip(g, (rq, rk, rv), ("dq", "dk", "dv")):
            check_grad(f64(x), ref, f"{name} ({path})")


# Full tensors: the A100 issue's shape, the packed document batch, the head_dim
# 64 pair with and without the LSE, every head_dim 256 batch of 32K tokens in
# both masks, the single 16K sequence, and windowed variants.
FULL_TENSOR = [
    (W.a100_shape(4096), True, False),
    (W.packed_16k(), True, False),
    (W.hd64_mha(), False, True),
    (W.hd256_gqa(8, 4096, False), True, False),
    (W.hd256_gqa(8, 4096, True), True, False),
    (W.hd256_gqa(2, 16384, False), True, False),
    (W.hd256_gqa(2, 16384, True), True, False),
    (W.hd256_gqa(1, 32768, False), True, False),
    (W.hd256_gqa(1, 32768, True), True, False),
    (W.single_16k_full(), True, False),
    (W.Workload("single-4096-gqa32/8-d128-full-w512_512", [4096], 32, 8, 128, False, window=(512, 512)), True,
     False),
    (W.Workload("packed16k-docs-gqa32/8-d128-causal-w1024", list(W.PACKED_16K_DOC_LENGTHS), 32, 8, 128, True,
                window=(1024, -1)), True, False),
    (W.Workload("8x4096-gqa8/1-d256-causal-w1000", [4096] * 8, 8, 1, 256, True, window=(1000, -1)), True, False),
]


@pytest.mark.parametrize("wl,backward,lse_off", FULL_TENSOR, ids=[w.name for w, _, _ in FULL_TENSOR])
def test_parity_full_size_full_tensors(wl, backward, lse_off):
    pooled_parity(wl, backward, lse_off)


def sampled_parity(wl: W.Workload):
    """Sequences of 64K and more: the GPU runs the whole problem; the oracle checks
    O, LSE and dQ on sampled query rows; dK and dV on the last 256 keys of each
    causal sequence (cheap) and on stored rows (the first 256 keys, which every
    query row sees, plus 64 random ones) written by tests/golden/make_dkdv_golden.py;
    and the any-size sums of dK and dV."""
    inp = W.make_inputs(wl, with_dout=True)
    golden = np.load(GOLDEN_DKDV[wl.name])
    assert str(golden["workload"]) == wl.name
    assert str(golden["input_sha256"]) == W.inputs_sha256(inp), "stored dK/dV rows were made for other inputs"
    d = to_dev(inp)
    cu_q, cu_k = wl.cu_seqlens_q, wl.cu_seqlens_k
    announce(f"fwd {wl.name} (full size, sampled oracle)")
    out, lse = gpu_fwd(wl, d)
    announce(f"bwd {wl.name} (full size, sampled oracle)")
    dq, dk, dv = gpu_bwd(wl, d, out, lse)
    torch.cuda.synchronize()
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    rows = sample_rows(cu_q, extra=64)
    r, ro, rl = O.forward_rows(q, k, v, cu_q, cu_k, wl.softmax_scale, wl.causal, rows, window=wl.window)
    check_out(f64(out[torch.as_tensor(r)]), ro)
    check_lse(f64(lse[:, torch.as_tensor(r)]), rl)
    r, rdq = O.backward_dq_rows(q, k, v, cu_q, cu_k, wl.softmax_scale, wl.causal, do, rows, window=wl.window)
    check_grad(f64(dq[torch.as_tensor(r)]), rdq, "dq(sampled rows)")
    if wl.causal:
        krows = sample_rows(cu_k, extra=32, tail_only=True)
        r, rdk, rdv = OP.backward_dkdv_rows(q, k, v, cu_q, cu_k, wl.softmax_scale, wl.causal, do, krows,
                                            window=wl.window)
        check_grad(f64(dk[torch.as_tensor(r)]), rdk, "dk(last keys)")
        check_grad(f64(dv[torch.as_tensor(r)]), rdv, "dv(last keys)")
    gr = torch.as_tensor(golden["key_rows"])
    check_grad(f64(dk[gr]), golden["dk"].astype(np.float64), "dk(stored rows)")
    check_grad(f64(dv[gr]), golden["dv"].astype(np.float64), "dv(stored rows)")
    check_gradient_sums(wl, d, dk, dv)


def check_gradient_sums(wl, d, dk, dv):
    """Any-size properties of the exact gradient, per sequence and KV head:
    sum_j dK_j = 0 and sum_j dV_j = sum over the group's heads and rows of dO_i
    (each query row with a visible key has softmax weights summing to one)."""
    r = wl.n_q_heads // wl.n_kv_heads
    cu_q, cu_k = wl.cu_seqlens_q, wl.cu_seqlens_k
    dkf = dk.float()
    dvf = dv.float()
    dof = d["dout"].float()
    for b in range(len(cu_q) - 1):
        ks, ke = cu_k[b], cu_k[b + 1]
        qs, qe = cu_q[b], cu_q[b + 1]
        if ke == ks or qe == qs:
            continue
        n = ke - ks
        for g in range(wl.n_kv_heads):
            sk = dkf[ks:ke, g].double().sum(0)
            sv = dvf[ks:ke, g].double().sum(0)
            want = dof[qs:qe, g * r:(g + 1) * r].double().sum((0, 1))
            scale_k = dkf[ks:ke, g].double().pow(2).mean().sqrt() * (n ** 0.5)
            scale_v = dvf[ks:ke, g].double().pow(2).mean().sqrt() * (n ** 0.5)
            assert float(sk.norm() / (scale_k * sk.numel() ** 0.5 + 1e-30)) < 0.05, "sum of dK is not ~0"
            assert float((sv - want).norm() / (scale_v * sv.numel() ** 0.5 + 1e-30)) < 0.05, "sum of dV mismatch"


GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GOLDEN_DKDV = {
    W.long_65k().name: os.path.join(GOLDEN_DIR, "dkdv_single-65536-gqa32-8-d128-causal.npz"),
    W.hd256_gqa(1, 131072, False).name: os.path.join(GOLDEN_DIR, "dkdv_1x131072-gqa8-1-d256-full.npz"),
    W.hd256_gqa(1, 131072, True).name: os.path.join(GOLDEN_DIR, "dkdv_1x131072-gqa8-1-d256-causal.npz"),
}
SAMPLED = [W.long_65k(), W.hd256_gqa(1, 131072, False), W.hd256_gqa(1, 131072, True)]


@pytest.mark.parametrize("wl", SAMPLED, ids=[w.name for w in SAMPLED])
def test_parity_full_size_sampled(wl):
    sampled_parity(wl)


# query chunks against long keys (few items per launch): the split-KV forward
# with the library's split count, sampled rows against the oracle
SPLIT_FULL = [
    W.Workload("2x256-vs-32768-gqa32/8-d128-causal", [256, 256], 32, 8, 128, True, seqlens_k=[32768, 32768],
               backward=False),
    W.Workload("4x64-vs-8192-gqa8/1-d256-causal", [64] * 4, 8, 1, 256, True, seqlens_k=[8192] * 4, backward=False),
    W.Workload("1x128-vs-65536-mha16-d64-full", [128], 16, 16, 64, False, seqlens_k=[65536], backward=False),
]


@pytest.mark.parametrize("wl", SPLIT_FULL, ids=[w.name for w in SPLIT_FULL])
def test_parity_splitkv_full_size_sampled(wl):
    inp = W.make_inputs(wl, with_dout=False)
    d = to_dev(inp)
    n = A.attn_varlen_fwd_num_splits(len(wl.seqlens_q), wl.total_q, wl.max_seqlen_q, wl.max_seqlen_k,
                                     wl.n_q_heads, wl.n_kv_heads, wl.head_dim)
    assert n > 1
    announce(f"split-kv fwd {wl.name} (full size, {n} splits, sampled oracle)")
    out, lse = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                                 wl.max_seqlen_k, wl.softmax_scale, wl.causal, return_lse=True, num_splits=0)
    torch.cuda.synchronize()
    q, k, v = (W.to_f64(inp[x]) for x in ("q", "k", "v"))
    rows = sample_rows(wl.cu_seqlens_q, extra=64)
    r, ro, rl = O.forward_rows(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, rows)
    check_out(f64(out[torch.as_tensor(r)]), ro)
    check_lse(f64(lse[:, torch.as_tensor(r)]), rl)


# --------------------------------------------------------------------------
# bitwise and structural properties of the kernels
# --------------------------------------------------------------------------

def _run_all(wl, d, stored_ds=False):
    out, lse = gpu_fwd(wl, d)
    dq, dk, dv = gpu_bwd(wl, d, out, lse, stored_ds)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("stored_ds", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_deterministic(causal, stored_ds):
    wl = W.Workload("det", [700, 33, 1200], 8, 2, 128, causal)
    d = to_dev(W.make_inputs(wl))
    announce(f"determinism causal={causal} stored_ds={stored_ds}")
    a = _run_all(wl, d, stored_ds)
    b = _run_all(wl, d, stored_ds)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [64, 128])
def test_stored_ds_matches_recompute(D):
    """dV comes from the same kernel and arithmetic on both paths (the stored-dS
    one only adds the dS stores): bit-identical. dK and dQ depend on the row
    term Delta, which the two paths sum in different orders (the row-term
    kernel against the recomputing dQ kernel), so they agree to rounding; each
    is checked against the oracle elsewhere. MHA, so that the recomputing path
    does not split the query heads of a group (the stored-dS path never does)."""
    wl = W.Workload("paths", [700, 33, 1200, 0, 257], 8, 8, D, True)
    d = to_dev(W.make_inputs(wl))
    announce(f"stored vs recomputed dS, D={D}")
    out, lse = gpu_fwd(wl, d)
    a = gpu_bwd(wl, d, out, lse, True)
    b = gpu_bwd(wl, d, out, lse, False)
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2])
    for x, y in zip(a[:2], b[:2]):
        rel = float((x.float() - y.float()).norm() / y.float().norm())
        assert rel < 5e-3, rel


def test_lse_flag_does_not_change_output():
    wl = W.Workload("lseflag", [333, 1000], 16, 16, 64, False)
    d = to_dev(W.make_inputs(wl, with_dout=False))
    announce("lse on/off")
    o1, _ = gpu_fwd(wl, d, return_lse=True)
    o2 = gpu_fwd(wl, d, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_separate_calls(causal):
    wl = W.Workload("varlen-sep", [300, 1, 517, 128], 8, 4, 128, causal)
    d = to_dev(W.make_inputs(wl))
    announce(f"varlen vs separate causal={causal}")
    out, lse, dq, dk, dv = _run_all(wl, d)
    cu = wl.cu_seqlens_q
    for b, L in enumerate(wl.seqlens_q):
        s = slice(cu[b], cu[b + 1])
        one = W.Workload("one", [L], 8, 4, 128, causal)
        db = {k: (v[s].contiguous() if k in ("q", "k", "v", "dout") else v) for k, v in d.items()}
        db["cu_seqlens_q"] = torch.tensor([0, L], dtype=torch.int32, device=out.device)
        db["cu_seqlens_k"] = db["cu_seqlens_q"]
        o1, l1, q1, k1, v1 = _run_all(one, db)
        assert torch.equal(out[s], o1)
        assert torch.equal(lse[:, s], l1)
        assert torch.equal(dq[s], q1)
        assert torch.equal(dk[s], k1)
        assert torch.equal(dv[s], v1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hkv", [2, 4])
def test_gqa_equals_mha_with_repeated_kv(causal, Hkv):
    """Grouped-query attention is attention of each query head against its
    group's KV head, which equals plain multi-head attention with every KV head
    repeated over its group. The LSE agrees bit for bit: each row visits its key
    tiles in the same order with the same fp32 row sums. The kernels put a KV
    group's heads in one workgroup (4 heads of 32 rows each for the groups of 4
    here, 2 of 64 for the groups of 2, 1 of 128 for MHA), so the layouts split a sequence's
    rows into different blocks, and a tile near a block's diagonal may take the
    masked path, whose P enters the PV product split into two bf16 parts, in one
    layout and not the other: O and the gradients agree to bf16 rounding."""
    Hq = 8
    wl = W.Workload("gqa", [400, 250], Hq, Hkv, 64, causal)
    d = to_dev(W.make_inputs(wl))
    announce(f"gqa vs mha causal={causal} Hkv={Hkv}")
    out, lse, dq, dk, dv = _run_all(wl, d)
    wm = W.Workload("mha", [400, 250], Hq, Hq, 64, causal)
    dm = dict(d)
    dm["k"] = d["k"].repeat_interleave(Hq // Hkv, dim=1).contiguous()
    dm["v"] = d["v"].repeat_interleave(Hq // Hkv, dim=1).contiguous()
    om, lm, qm, km, vm = _run_all(wm, dm)
    assert torch.equal(lse, lm)

    def rel(x, y):
        return float((x.float() - y.float()).norm() / y.float().norm())

    assert float((out.float() - om.float()).abs().max()) <= 1e-2
    assert rel(out, om) <= 5e-3
    assert rel(dq, qm) <= 1e-2
    km = km.float().reshape(km.shape[0], Hkv, Hq // Hkv, -1).sum(2)
    vm = vm.float().reshape(vm.shape[0], Hkv, Hq // Hkv, -1).sum(2)
    assert rel(dk, km) < 1e-2
    assert rel(dv, vm) < 1e-2


def test_no_writes_outside_outputs():
    """Canary bytes around every output buffer must survive fwd and bwd."""
    wl = W.Workload("canary", [130, 0, 77], 4, 2, 128, True, seqlens_k=[130, 40, 0])
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    dev = d["q"].device
    pad = 4096
    def padded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), 7, dtype=dtype, device=dev)
        return buf, buf[pad:pad + n].view(shape)
    ob, out = padded(d["q"].shape, torch.bfloat16)
    lb, lse = padded((4, wl.total_q), torch.float32)
    announce("canary fwd")
    A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                      wl.max_seqlen_k, wl.softmax_scale, True, out=out, lse=lse)
    qb, dq = padded(d["q"].shape, torch.bfloat16)
    kb, dk = padded(d["k"].shape, torch.bfloat16)
    vb, dv = padded(d["v"].shape, torch.bfloat16)
    announce("canary bwd")
    A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], out, lse, d["cu_seqlens_q"], d["cu_seqlens_k"],
                      wl.max_seqlen_q, wl.max_seqlen_k, wl.softmax_scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf in (ob, lb, qb, kb, vb):
        assert torch.all(buf[:pad] == 7) and torch.all(buf[-pad:] == 7)
    # keys of the middle sequence see no query (Lq = 0): zero gradients; rows of the
    # last sequence see no key (Lk = 0): zero output, -inf LSE, zero dq
    assert torch.all(dk[130:170] == 0) and torch.all(dv[130:170] == 0)
    assert torch.all(out[130:] == 0) and torch.all(dq[130:] == 0)
    assert torch.all(torch.isneginf(lse[:, 130:]))


# The device decode searches the block levels (ceil(max_seqlen_q / bm) of them)
# 64 at a time; more than 4096 levels take further narrowing passes: long
# sequences, and inflated max_seqlen bounds over short ones.
@pytest.mark.parametrize("lengths,bm,max_q", [
    ([200, 312], 128, None),
    (W.PACKED_16K_DOC_LENGTHS, 128, None),
    ([0, 5, 0, 130, 1, 128, 129, 0], 64, None),
    ([131072], 128, None),
    (list(range(0, 9000, 97)), 128, None),
    ([600000], 128, None),
    ([9000, 100], 128, 600000),
    ([3, 0, 700000, 5], 64, 2000000),
    ([600000, 1, 4096], 32, None),
    # more than 64 sequences: per-lane chunks of block counts, bisection over the levels
    ([7] * 65, 64, None),
    (list(np.random.default_rng(21).integers(0, 300, size=1000)), 64, None),
    (list(np.random.default_rng(22).integers(0, 40, size=4097)), 32, None),
    (list(np.random.default_rng(23).integers(0, 5, size=20000)), 128, None),
    ([600000] + list(np.random.default_rng(24).integers(0, 700, size=300)), 32, None),
    (list(np.random.default_rng(25).integers(0, 90, size=2000)), 64, 70000),
])
def test_device_schedule_matches_host(lengths, bm, max_q):
    lengths = [int(x) for x in lengths]
    cu = W.cu_from_lengths(lengths)
    host = A.attn_varlen_schedule_host(cu, bm)
    max_q = max(lengths) if max_q is None else max_q
    announce(f"schedule decode {len(lengths)} seqs bm={bm} max_seqlen_q={max_q}")
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    seq, blk = A.attn_varlen_schedule_device(cu_d, max_q, bm, len(host) + 5)
    torch.cuda.synchronize()
    seq, blk = seq.cpu().tolist(), blk.cpu().tolist()
    assert list(zip(seq[:len(host)], blk[:len(host)])) == host
    assert seq[len(host):] == [-1] * 5 and blk[len(host):] == [-1] * 5


@pytest.mark.parametrize("causal,win", [(False, (90, 40)), (True, (200, -1))])
def test_window_deterministic_and_autograd(causal, win):
    wl = W.Workload("win-autograd", [700, 33, 1200], 8, 2, 128, causal, window=win)
    d = to_dev(W.make_inputs(wl))
    announce(f"window determinism + autograd causal={causal} window={win}")
    a = _run_all(wl, d)
    b = _run_all(wl, d)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    q = d["q"].clone().requires_grad_(True)
    k = d["k"].clone().requires_grad_(True)
    v = d["v"].clone().requires_grad_(True)
    out = A.attn_varlen_func(q, k, v, d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                             wl.softmax_scale, causal, window_size=win)
    out.backward(d["dout"])
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), a[0])
    assert torch.equal(q.grad, a[2]) and torch.equal(k.grad, a[3]) and torch.equal(v.grad, a[4])


def test_unbounded_window_equals_plain_call():
    wl = W.Workload("win-unbounded", [300, 517], 8, 4, 128, True)
    d = to_dev(W.make_inputs(wl))
    announce("window (-1,-1) and wide windows vs plain")
    plain = _run_all(wl, d)
    for win in ((-1, -1), (100000, -1), (100000, 100000)):
        wlw = W.Workload("win-unbounded", [300, 517], 8, 4, 128, True, window=win)
        got = _run_all(wlw, d)
        for x, y in zip(plain, got):
            assert torch.equal(x, y), f"window {win}"


def test_autograd_wrapper_matches_direct_calls():
    wl = W.Workload("autograd", [90, 300], 4, 2, 64, True)
    d = to_dev(W.make_inputs(wl))
    announce("autograd wrapper")
    q = d["q"].clone().requires_grad_(True)
    k = d["k"].clone().requires_grad_(True)
    v = d["v"].clone().requires_grad_(True)
    out = A.attn_varlen_func(q, k, v, d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k,
                             wl.softmax_scale, True)
    out.backward(d["dout"])
    o2, l2, dq, dk, dv = _run_all(wl, d)
    assert torch.equal(out.detach(), o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


# persistent scheduler: the same items run by fewer workgroups that take them
# from per-XCD queues; every result must be bit-identical to the one-pass grid,
# and the scheduler scratch must be zero again after each call
PERSIST_CASES = [
    W.packed_16k(),
    W.Workload("ragged-d64-f", [1, 77, 300, 513, 0, 129], 8, 2, 64, False),
    W.Workload("ragged-d256-c", [1, 77, 300, 513, 0, 129], 8, 2, 256, True),
    W.Workload("window-d128-c-w300", [2100, 1500, 7], 8, 2, 128, True, window=(300, -1)),
    W.Workload("lq-ne-lk-d128-f-w20_10", [100, 300, 5, 0], 4, 1, 128, False, seqlens_k=[250, 64, 0, 33],
               window=(20, 10)),
    W.Workload("many-items-d128-c", [8192] * 4, 32, 8, 128, True, backward=False),
]


@pytest.mark.parametrize("wl", PERSIST_CASES, ids=[w.name for w in PERSIST_CASES])
def test_persistent_scheduler_matches_grid(wl):
    d = to_dev(W.make_inputs(wl, with_dout=False))
    sched = torch.zeros(A.SCHED_BYTES, dtype=torch.uint8, device=d["q"].device)
    args = (d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k,
            wl.softmax_scale, wl.causal)
    win = window_of(wl)
    announce(f"persistent vs grid {wl.name}")
    o1, l1 = A.attn_varlen_fwd(*args, return_lse=True, window_size=win)
    for rep in range(2):
        o2, l2 = A.attn_varlen_fwd(*args, return_lse=True, window_size=win, persistent=True, sched=sched)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"call {rep}: out differs"
        assert torch.equal(l1, l2), f"call {rep}: lse differs"
        assert int(sched.count_nonzero()) == 0, f"call {rep}: scheduler scratch not reset"


def test_persistent_scheduler_against_oracle_and_smaller_second_call():
    sched = torch.zeros(A.SCHED_BYTES, dtype=torch.uint8, device="cuda:0")
    for wl in (W.Workload("persist-a", [700, 33, 1200], 8, 2, 128, True),
               W.Workload("persist-b", [90, 300], 4, 2, 64, False)):
        inp = W.make_inputs(wl, with_dout=False)
        d = to_dev(inp)
        announce(f"persistent vs oracle {wl.name}")
        out, lse = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q,
                                     wl.max_seqlen_k, wl.softmax_scale, wl.causal, return_lse=True, persistent=True,
                                     sched=sched)
        torch.cuda.synchronize()
        q, k, v = (W.to_f64(inp[x]) for x in ("q", "k", "v"))
        ref_o, ref_l = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal)
        check_out(f64(out), ref_o)
        check_lse(f64(lse), ref_l)
        assert int(sched.count_nonzero()) == 0


# edge cases of the split-KV and persistent paths: zero and negative scale,
# single-token queries, one key, more splits than key tiles
EDGE = [
    (W.Workload("edge-scale0-d64-f", [150, 90], 2, 1, 64, False, softmax_scale=0.0), 3),
    (W.Workload("edge-negscale-d128-c", [200, 64], 4, 2, 128, True, softmax_scale=-0.09), 4),
    (W.Workload("edge-decode1-d256-f", [1, 1, 1], 8, 1, 256, False, seqlens_k=[1, 2000, 33]), 16),
    (W.Workload("edge-onekey-d128-c", [5, 1], 4, 4, 128, True, seqlens_k=[1, 1]), 2),
]
# more than 64 sequences through the split-KV chunks and the persistent queues
# (the decode's per-lane chunks): decode-like few queries against longer keys,
# and many short causal documents
_rng = np.random.default_rng(31)
EDGE += [
    (W.Workload("edge-many700-decode-d128-f", [int(x) for x in _rng.integers(1, 5, size=700)], 8, 2, 128, False,
                seqlens_k=[int(x) for x in _rng.integers(0, 600, size=700)]), 3),
    (W.Workload("edge-many1200-d64-c", [int(x) for x in _rng.integers(0, 70, size=1200)], 4, 2, 64, True), 5),
]


@pytest.mark.parametrize("wl,splits", EDGE, ids=[w.name for w, _ in EDGE])
def test_edge_cases_split_and_persistent(wl, splits):
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    q, k, v = (W.to_f64(inp[x]) for x in ("q", "k", "v"))
    ref_o, ref_l = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal)
    args = (d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], wl.max_seqlen_q, wl.max_seqlen_k,
            wl.softmax_scale, wl.causal)
    announce(f"edge split {wl.name} splits={splits}")
    o1, l1 = A.attn_varlen_fwd(*args, return_lse=True, num_splits=splits)
    announce(f"edge persistent {wl.name}")
    o2, l2 = A.attn_varlen_fwd(*args, return_lse=True, persistent=True)
    o3, l3 = A.attn_varlen_fwd(*args, return_lse=True)
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o2, l2)):
        check_out(f64(o), ref_o)
        check_lse(f64(l), ref_l)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)


# Sharply peaked attention (a scale several times D^-1/2 on unit-variance data):
# a row's output is nearly one V row, |O| reaches 4 and more, and there half a
# bf16 spacing (1/64) is above the 1e-2 absolute bound. Outputs are held to
# 1e-2 beyond that rounding (check_out_rounded); LSE and gradients to the usual
# bounds.
PEAKED = []
for D in (64, 128, 256):
    for c, sc in ((False, 0.5), (True, -0.4)):
        PEAKED.append(W.Workload(f"peaked-d{D}-{'c' if c else 'f'}-s{sc}", [900, 33, 400], 8, 2, D, c,
                                 softmax_scale=sc))


@pytest.mark.parametrize("wl", PEAKED, ids=[w.name for w in PEAKED])
def test_parity_peaked_attention(wl):
    inp = W.make_inputs(wl)
    d = to_dev(inp)
    announce(f"peaked {wl.name}")
    out, lse = gpu_fwd(wl, d)
    dq, dk, dv = gpu_bwd(wl, d, out, lse)
    torch.cuda.synchronize()
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    ref_o, ref_l = O.forward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal)
    assert np.abs(ref_o).max() >= 3.5  # the regime this test is for
    check_out_rounded(f64(out), ref_o)
    check_lse(f64(lse), ref_l)
    rq, rk, rv = O.backward(q, k, v, wl.cu_seqlens_q, wl.cu_seqlens_k, wl.softmax_scale, wl.causal, do)
    check_grad(f64(dq), rq, "dq")
    check_grad(f64(dk), rk, "dk")
    check_grad(f64(dv), rv, "dv")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_no_keys_or_no_queries_at_all(D, causal):
    """A batch without any key (total_k = 0) or without any query (total_q = 0):
    the empty tensors come with NULL data pointers, which the library accepts.
    Rows that see no key give O = 0 and LSE = -inf (and dQ = 0); keys that no
    row sees give dK = dV = 0."""
    nok = W.Workload(f"nokeys-d{D}", [37, 5], 4, 2, D, causal, seqlens_k=[0, 0])
    inp = W.make_inputs(nok)
    d = to_dev(inp)
    assert d["k"].numel() == 0
    q, k, v = (W.to_f64(inp[x]) for x in ("q", "k", "v"))
    ref_o, ref_l = O.forward(q, k, v, nok.cu_seqlens_q, nok.cu_seqlens_k, nok.softmax_scale, causal)
    args = (d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], nok.max_seqlen_q, nok.max_seqlen_k,
            nok.softmax_scale, causal)
    announce(f"no keys D={D} causal={causal}: plain, split-KV, persistent, backward")
    outs = [A.attn_varlen_fwd(*args, return_lse=True),
            A.attn_varlen_fwd(*args, return_lse=True, num_splits=3),
            A.attn_varlen_fwd(*args, return_lse=True, persistent=True)]
    o, l = outs[0]
    dq, dk, dv = A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], o, l, d["cu_seqlens_q"], d["cu_seqlens_k"],
                                   nok.max_seqlen_q, nok.max_seqlen_k, nok.softmax_scale, causal)
    torch.cuda.synchronize()
    assert np.all(ref_o == 0.0) and np.all(np.isneginf(ref_l))
    for oi, li in outs:
        assert int(torch.count_nonzero(oi)) == 0
        assert bool(torch.all(torch.isneginf(li)))
    assert dq.shape == d["q"].shape and int(torch.count_nonzero(dq)) == 0
    assert dk.numel() == 0 and dv.numel() == 0

    noq = W.Workload(f"noqueries-d{D}", [0, 0], 4, 2, D, causal, seqlens_k=[40, 9])
    d = to_dev(W.make_inputs(noq))
    assert d["q"].numel() == 0
    announce(f"no queries D={D} causal={causal}: forward, backward")
    o, l = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], noq.max_seqlen_q,
                             noq.max_seqlen_k, noq.softmax_scale, causal, return_lse=True)
    dq, dk, dv = A.attn_varlen_bwd(d["dout"], d["q"], d["k"], d["v"], o, l, d["cu_seqlens_q"], d["cu_seqlens_k"],
                                   noq.max_seqlen_q, noq.max_seqlen_k, noq.softmax_scale, causal)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0
    assert dk.shape == d["k"].shape and int(torch.count_nonzero(dk)) == 0
    assert dv.shape == d["v"].shape and int(torch.count_nonzero(dv)) == 0


@pytest.mark.parametrize("cu_q,cu_k,tq,tk,mq,mk,bits", [
    ([0, 5, 12], [0, 3, 12], 12, 12, 7, 9, 0),          # valid
    ([1, 5, 12], [0, 3, 12], 12, 12, 7, 9, 1),          # first entry not 0
    ([0, 7, 5, 12], [0, 3, 4, 12], 12, 12, 7, 8, 2),    # decreasing
    ([0, 5, 12], [0, 3, 11], 12, 12, 7, 9, 4),          # last entry != total
    ([0, 5, 12], [0, 3, 12], 12, 12, 6, 9, 8),          # longer than max_seqlen_q
    ([0, 7, 5, 12], [1, 3, 4, 11], 12, 12, 3, 3, 15),   # everything at once
])
def test_validate_seqlens(cu_q, cu_k, tq, tk, mq, mk, bits):
    announce(f"validate seqlens {cu_q} {cu_k}")
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda:0")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda:0")
    assert A.attn_varlen_validate_seqlens(cq, ck, tq, tk, mq, mk) == bits


def test_validate_env_raises_before_launch(monkeypatch):
    wl = W.Workload("validate-env", [40, 24], 2, 1, 64, True)
    d = to_dev(W.make_inputs(wl, with_dout=False))
    monkeypatch.setenv("ATTN_VARLEN_VALIDATE", "1")
    announce("validate env")
    out = A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], 40, 40)  # valid: runs
    torch.cuda.synchronize()
    with pytest.raises(ValueError):  # max_seqlen_q understated: rejected before any kernel runs
        A.attn_varlen_fwd(d["q"], d["k"], d["v"], d["cu_seqlens_q"], d["cu_seqlens_k"], 30, 40)
    assert out.shape == d["q"].shape
