"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments with its error codes before touching the device; the host
work ranking is checked by brute force."""
import ctypes
import os
import re

import numpy as np
import pytest

import exact_attention_varlen_amd as A
from exact_attention_varlen_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_varlen.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_varlen_\w+)\s*\(", text)))


def header_enums():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_VARLEN_\w+)\s*=\s*(-?\d+)", text)}


def test_library_loads_and_exports_every_declared_symbol():
    l = _lib.lib()
    names = header_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(l, n), n
    assert set(names) == set(_lib.exported_names())


def test_version_and_error_strings():
    assert A.attn_varlen_version() == (1, 8)
    for name, code in header_enums().items():
        s = A.attn_varlen_error_string(code)
        assert s and s != "unknown error code", name
    assert A.attn_varlen_error_string(12345) == "unknown error code"


E = header_enums()
FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced because validation fails first


def fwd_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=1, total_q=16, total_k=16, max_q=16, max_k=16,
             Hq=4, Hkv=2, D=96, scale=0.125, causal=0, out=FAKE, lse=None, stream=None)
    a.update(over)
    return _lib.lib().attn_varlen_fwd(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"], a["total_q"],
                                      a["total_k"], a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                      a["causal"], a["out"], a["lse"], a["stream"])


def bwd_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=1, total_q=16, total_k=16, max_q=16, max_k=16,
             Hq=4, Hkv=2, D=96, scale=0.125, causal=0, dout=FAKE, out=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(over)
    return _lib.lib().attn_varlen_bwd(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"], a["total_q"],
                                      a["total_k"], a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                      a["causal"], a["dout"], a["out"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                                      a["ws_bytes"], a["stream"])


# Each case is invalid in exactly the named way (D=96 is also invalid, so cases that
# test other checks fix D to a valid value and break one thing only where needed).
@pytest.mark.parametrize("over,code", [
    (dict(D=96), "ATTN_VARLEN_ERR_BAD_HEAD_DIM"),
    (dict(D=32), "ATTN_VARLEN_ERR_BAD_HEAD_DIM"),
    (dict(q=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(cu_k=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(D=128, out=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(D=128, Hq=6, Hkv=4), "ATTN_VARLEN_ERR_BAD_HEADS"),
    (dict(D=128, Hq=0), "ATTN_VARLEN_ERR_BAD_HEADS"),
    (dict(D=128, Hkv=-1), "ATTN_VARLEN_ERR_BAD_HEADS"),
    (dict(D=128, num_seqs=0), "ATTN_VARLEN_ERR_BAD_SEQLEN"),
    (dict(D=128, total_q=-1), "ATTN_VARLEN_ERR_BAD_SEQLEN"),
    (dict(D=128, max_q=17), "ATTN_VARLEN_ERR_BAD_SEQLEN"),
    (dict(D=128, max_k=-3), "ATTN_VARLEN_ERR_BAD_SEQLEN"),
    (dict(D=128, total_q=1 << 40, max_q=16), "ATTN_VARLEN_ERR_BAD_SEQLEN"),
    (dict(D=128, q=FAKE + 8), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=128, out=FAKE + 2), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=128, lse=FAKE + 2), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=128, cu_q=FAKE + 1), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=128, scale=float("nan")), "ATTN_VARLEN_ERR_BAD_SCALE"),
    (dict(D=128, scale=float("inf")), "ATTN_VARLEN_ERR_BAD_SCALE"),
    (dict(D=128, causal=2), "ATTN_VARLEN_ERR_BAD_FLAG"),
])
def test_fwd_argument_errors(over, code):
    assert fwd_call(**over) == E[code]


def test_fwd_empty_problem_is_a_no_op():
    # total_q == 0 returns success without launching anything
    assert fwd_call(D=64, total_q=0, max_q=0) == 0


def test_null_pointers_of_empty_tensors_are_accepted():
    # A tensor without rows may be passed as NULL. Each call below gets past the
    # pointer checks and stops at a later check (head_dim 96, a misaligned
    # pointer) or at the empty-problem return, so nothing is launched.
    assert fwd_call(k=None, v=None, total_k=0, max_k=0) == E["ATTN_VARLEN_ERR_BAD_HEAD_DIM"]
    assert fwd_call(q=None, out=None, total_q=0, max_q=0) == E["ATTN_VARLEN_ERR_BAD_HEAD_DIM"]
    assert fwd_call(D=64, q=None, out=None, total_q=0, max_q=0) == 0
    assert bwd_call(D=64, k=None, v=None, dk=None, dv=None, total_k=0, max_k=0,
                    dq=FAKE + 8) == E["ATTN_VARLEN_ERR_MISALIGNED"]
    assert bwd_call(D=64, q=None, dout=None, out=None, lse=None, dq=None, total_q=0, max_q=0,
                    dk=FAKE + 8) == E["ATTN_VARLEN_ERR_MISALIGNED"]
    # nothing to do at all: every data pointer and the (zero-byte) workspace NULL
    assert bwd_call(D=64, q=None, k=None, v=None, dout=None, out=None, lse=None, dq=None, dk=None, dv=None,
                    total_q=0, max_q=0, total_k=0, max_k=0, ws=None, ws_bytes=0) == 0


@pytest.mark.parametrize("over", [dict(k=None), dict(v=None), dict(q=None)])
def test_null_pointers_of_tensors_with_rows_are_rejected(over):
    assert fwd_call(**over) == E["ATTN_VARLEN_ERR_NULL_POINTER"]
    assert bwd_call(**over) == E["ATTN_VARLEN_ERR_NULL_POINTER"]


@pytest.mark.parametrize("over", [dict(dq=None), dict(dk=None), dict(out=None), dict(lse=None)])
def test_null_backward_outputs_with_rows_are_rejected(over):
    assert bwd_call(D=64, **over) == E["ATTN_VARLEN_ERR_NULL_POINTER"]


@pytest.mark.parametrize("over,code", [
    (dict(D=96), "ATTN_VARLEN_ERR_BAD_HEAD_DIM"),
    (dict(D=64, dout=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(D=64, lse=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(D=64, dv=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(D=64, ws=None), "ATTN_VARLEN_ERR_WORKSPACE"),
    (dict(D=64, ws_bytes=16 * 4 * 4 - 1), "ATTN_VARLEN_ERR_WORKSPACE"),
    (dict(D=64, ws=FAKE + 4), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=64, dk=FAKE + 8), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=64, lse=FAKE + 1), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(D=64, Hq=3, Hkv=2), "ATTN_VARLEN_ERR_BAD_HEADS"),
    (dict(D=64, causal=-1), "ATTN_VARLEN_ERR_BAD_FLAG"),
])
def test_bwd_argument_errors(over, code):
    assert bwd_call(**over) == E[code]


def test_bwd_workspace_size():
    ws = A.attn_varlen_bwd_workspace_size(3, 1000, 900, 32, 8, 128)
    assert ws >= 1000 * 32 * 4 and ws % 256 == 0
    assert A.attn_varlen_bwd_workspace_size(1, 0, 0, 4, 2, 64) == 0


def _pad(b):
    return -(-b // 256) * 256


@pytest.mark.parametrize("total, hq, hkv, d, splits", [
    (32768, 8, 1, 256, 8),        # 256 key blocks x 1 KV head: 8 splits reach 2048 items
    (131072, 8, 1, 256, 2),       # 1024 key blocks: 2 splits
    (16384, 16, 2, 256, 8),       # 128 blocks x 2 heads = 256 items: 8 of the 8 heads
    (300000, 8, 1, 256, 1),       # >= 2048 key blocks: no split
    (1000, 6, 1, 256, 6),         # too few items for any divisor: all 6 heads
    # head dims 64 / 128: no split from 256 items (key blocks x KV heads) on,
    # below that the smallest divisor reaching 1024 items
    (16384, 32, 8, 128, 1),       # 128 blocks x 8 heads = 1024 items
    (4096, 32, 8, 128, 1),        # 32 x 8 = 256 items
    (4096, 32, 1, 128, 32),       # 32 items: 32 splits reach 1024
    (8192, 16, 2, 64, 8),         # 64 x 2 = 128 items: 8 splits
    (1000, 32, 8, 128, 4),        # 7 x 8 = 56 items, no divisor of 4 reaches 1024: all 4
    (65536, 16, 16, 64, 1),       # MHA: nothing to split
])
def test_bwd_workspace_size_splits(total, hq, hkv, d, splits):
    """Two fp32 row planes [Hq][total_q], plus two fp32 partial dK / dV blocks of
    [splits][total_k][Hkv][D] when the split count exceeds 1."""
    planes = 2 * _pad(total * hq * 4)
    parts = 2 * _pad(splits * total * hkv * d * 4) if splits > 1 else 0
    assert A.attn_varlen_bwd_workspace_size(1, total, total, hq, hkv, d) == planes + parts


def split_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=1, total_q=16, total_k=16, max_q=16, max_k=16,
             Hq=4, Hkv=2, D=128, scale=0.125, causal=0, wl=-1, wr=-1, splits=2, out=FAKE, lse=None, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(over)
    return _lib.lib().attn_varlen_fwd_splitkv(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"],
                                              a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["Hq"], a["Hkv"],
                                              a["D"], a["scale"], a["causal"], a["wl"], a["wr"], a["splits"],
                                              a["out"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=96), "ATTN_VARLEN_ERR_BAD_HEAD_DIM"),
    (dict(out=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(causal=3), "ATTN_VARLEN_ERR_BAD_FLAG"),
    (dict(splits=0), "ATTN_VARLEN_ERR_BAD_SPLITS"),
    (dict(splits=-2), "ATTN_VARLEN_ERR_BAD_SPLITS"),
    (dict(splits=65), "ATTN_VARLEN_ERR_BAD_SPLITS"),
    (dict(ws=None), "ATTN_VARLEN_ERR_WORKSPACE"),
    (dict(ws_bytes=2 * 16 * 4 * 128 * 4), "ATTN_VARLEN_ERR_WORKSPACE"),
    (dict(ws=FAKE + 8), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(lse=FAKE + 2), "ATTN_VARLEN_ERR_MISALIGNED"),
])
def test_splitkv_argument_errors(over, code):
    assert split_call(**over) == E[code]


def test_splitkv_trivial_calls_need_no_workspace():
    # empty problem: success without a launch; one split needs no workspace (the
    # call is then the one-pass forward, whose launch is not reached here because
    # total_q == 0)
    assert split_call(total_q=0, max_q=0, ws=None, ws_bytes=0) == 0
    assert split_call(total_q=0, max_q=0, splits=1, ws=None, ws_bytes=0) == 0


@pytest.mark.parametrize("total_q, hq, d, splits", [(16, 4, 128, 2), (1000, 32, 64, 7), (513, 8, 256, 64),
                                                    (0, 4, 128, 3)])
def test_splitkv_workspace_size(total_q, hq, d, splits):
    """fp32 partial outputs [splits][total_q][Hq][D] and row sums [splits][2][Hq][total_q], 256-byte padded."""
    want = _pad(splits * total_q * hq * d * 4) + _pad(splits * 2 * hq * total_q * 4)
    assert A.attn_varlen_fwd_splitkv_workspace_size(total_q, hq, d, splits) == want
    assert A.attn_varlen_fwd_splitkv_workspace_size(total_q, hq, d, 1) == 0
    assert A.attn_varlen_fwd_splitkv_workspace_size(-1, hq, d, splits) == 0


@pytest.mark.parametrize("lengths_q, lengths_k, hq, hkv, d", [
    ([3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005], [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005],
     32, 8, 128),
    ([16384], [16384], 32, 8, 128),
    ([4096] * 8, [4096] * 8, 8, 1, 256),
    ([16384, 16384], [16384, 16384], 16, 16, 64),
])
def test_num_splits_is_one_when_items_fill_the_gpu(lengths_q, lengths_k, hq, hkv, d):
    n = A.attn_varlen_fwd_num_splits(len(lengths_q), sum(lengths_q), max(lengths_q), max(lengths_k), hq, hkv, d)
    assert n == 1


@pytest.mark.parametrize("num_seqs, lq, lk, hq, hkv, d", [
    (1, 128, 32768, 32, 8, 128),   # 32 items for 512 slots
    (2, 256, 32768, 32, 8, 128),
    (4, 64, 8192, 8, 1, 256),
    (1, 1, 131072, 16, 16, 64),
])
def test_num_splits_fills_the_gpu_for_few_items(num_seqs, lq, lk, hq, hkv, d):
    n = A.attn_varlen_fwd_num_splits(num_seqs, num_seqs * lq, lq, lk, hq, hkv, d)
    bn = 64 if d <= 128 else 32
    items = num_seqs * -(-lq // 128) * hq
    slots = 256 * (2 if d <= 128 else 1)
    assert 1 < n <= 64
    assert n <= -(-lk // bn) // 4                  # every chunk keeps at least 4 key tiles
    assert items * n >= 0.85 * slots or n == min(64, -(-lk // bn) // 4)


def test_num_splits_short_keys_and_errors():
    assert A.attn_varlen_fwd_num_splits(1, 128, 128, 128, 4, 4, 128) == 1   # 2 key tiles: nothing to split
    with pytest.raises(A.AttnVarlenError):
        A.attn_varlen_fwd_num_splits(1, 128, 128, 128, 4, 4, 96)
    with pytest.raises(A.AttnVarlenError):
        A.attn_varlen_fwd_num_splits(1, 128, 128, 128, 6, 4, 128)
    with pytest.raises(A.AttnVarlenError):
        A.attn_varlen_fwd_num_splits(0, 128, 128, 128, 4, 4, 128)


def persist_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=1, total_q=16, total_k=16, max_q=16, max_k=16,
             Hq=4, Hkv=2, D=128, scale=0.125, causal=0, wl=-1, wr=-1, out=FAKE, lse=None, sched=FAKE, stream=None)
    a.update(over)
    return _lib.lib().attn_varlen_fwd_persistent(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["num_seqs"],
                                                 a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["Hq"],
                                                 a["Hkv"], a["D"], a["scale"], a["causal"], a["wl"], a["wr"],
                                                 a["out"], a["lse"], a["sched"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=96), "ATTN_VARLEN_ERR_BAD_HEAD_DIM"),
    (dict(out=None), "ATTN_VARLEN_ERR_NULL_POINTER"),
    (dict(sched=None), "ATTN_VARLEN_ERR_WORKSPACE"),
    (dict(sched=FAKE + 2), "ATTN_VARLEN_ERR_MISALIGNED"),
    (dict(Hq=5), "ATTN_VARLEN_ERR_BAD_HEADS"),
    (dict(causal=7), "ATTN_VARLEN_ERR_BAD_FLAG"),
])
def test_persistent_argument_errors(over, code):
    assert persist_call(**over) == E[code]


def test_persistent_empty_problem_is_a_no_op():
    assert persist_call(total_q=0, max_q=0) == 0


def test_python_split_and_persistent_argument_errors():
    """The binding passes bad split counts and scratch straight to the C checks."""
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):  # CPU tensors are rejected before any call
        A.attn_varlen_fwd(q, q, q, cu, cu, 4, 4, num_splits=2)


def test_validate_seqlens_argument_errors():
    l = _lib.lib()
    assert l.attn_varlen_validate_seqlens(None, FAKE, 1, 4, 4, 4, 4, FAKE, None) == E["ATTN_VARLEN_ERR_NULL_POINTER"]
    assert l.attn_varlen_validate_seqlens(FAKE, FAKE, 1, 4, 4, 4, 4, None, None) == E["ATTN_VARLEN_ERR_NULL_POINTER"]
    assert l.attn_varlen_validate_seqlens(FAKE, FAKE, 0, 4, 4, 4, 4, FAKE, None) == E["ATTN_VARLEN_ERR_BAD_SEQLEN"]
    assert l.attn_varlen_validate_seqlens(FAKE, FAKE, 1, -1, 4, 4, 4, FAKE, None) == E["ATTN_VARLEN_ERR_BAD_SEQLEN"]
    assert l.attn_varlen_validate_seqlens(FAKE, FAKE, 1, 4, 4, 4, 4, FAKE + 2, None) == E["ATTN_VARLEN_ERR_MISALIGNED"]


def test_seqlen_bits_match_header():
    text = open(HEADER).read()
    for bit, name in ((1, "BAD_START"), (2, "DECREASING"), (4, "BAD_TOTAL"), (8, "OVER_MAX")):
        m = re.search(r"#define ATTN_VARLEN_SEQLEN_%s (\d+)" % name, text)
        assert m and int(m.group(1)) == bit and bit in A.SEQLEN_BITS


def test_sched_bytes_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_VARLEN_SCHED_BYTES (\d+)", text)
    assert m and int(m.group(1)) == A.SCHED_BYTES


def test_schedule_device_argument_errors():
    l = _lib.lib()
    assert l.attn_varlen_schedule_device(None, 1, 16, 128, FAKE, FAKE, 4, None) == E["ATTN_VARLEN_ERR_NULL_POINTER"]
    assert l.attn_varlen_schedule_device(FAKE, 0, 16, 128, FAKE, FAKE, 4, None) == E["ATTN_VARLEN_ERR_BAD_SEQLEN"]
    assert l.attn_varlen_schedule_device(FAKE, 1, 16, 128, FAKE, FAKE, 0, None) == 0


def brute_force_schedule(lengths, bm):
    items = []
    for b, L in enumerate(lengths):
        for m in range(-(-L // bm)):
            items.append((b, m))
    # descending block index, ties by ascending sequence
    return sorted(items, key=lambda t: (-t[1], t[0]))


@pytest.mark.parametrize("lengths,bm", [
    ([200, 312], 128),
    ([3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005], 128),
    ([0, 5, 0, 130, 1, 128, 129, 0], 64),
    ([131072], 128),
    ([0], 128),
    (list(range(0, 300, 7)), 32),
])
def test_schedule_host_matches_brute_force(lengths, bm):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    got = A.attn_varlen_schedule_host(cu, bm)
    assert got == brute_force_schedule(lengths, bm)
    # every block exactly once; the causal work (block index + 1) never increases along the order
    assert len(set(got)) == len(got) == sum(-(-L // bm) for L in lengths)
    work = [m for _, m in got]
    assert all(a >= b for a, b in zip(work, work[1:]))


def test_schedule_host_random():
    rng = np.random.default_rng(0)
    for _ in range(20):
        lengths = rng.integers(0, 600, size=rng.integers(1, 90)).tolist()
        bm = int(rng.choice([32, 64, 128]))
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        assert A.attn_varlen_schedule_host(cu, bm) == brute_force_schedule(lengths, bm)


@pytest.mark.parametrize("splits", [0, 2, 64])
def test_persistent_rejects_split_counts(splits):
    """The persistent scheduler runs the one-pass forward only: a split count
    other than 1 (including 0, the library's choice, which may pick several) is
    an error, raised before any tensor is looked at."""
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="num_splits must be 1"):
        A.attn_varlen_fwd(q, q, q, cu, cu, 4, 4, num_splits=splits, persistent=True)


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_VARLEN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == A.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("Hq,total,D,ok", [
    (32, 131072, 128, True),     # row terms 2 x 32 x 131072 x 4 B = 32 MiB: fits exactly
    (32, 131073, 128, False),    # one row more does not
    (8, 32768, 256, True),       # head_dim 256, few key blocks: its 8-split partial sums (512 MiB) do
                                 # not fit, so the allocation-free call runs with fewer splits
    (16, 262145, 64, False),     # head_dim 64: row terms 2 x 16 x 262145 x 4 B, beyond the scratch
])
def test_noalloc_rejects_problems_beyond_the_scratch(Hq, total, D, ok):
    """The allocation-free backward checks the workspace it needs without dK / dV
    head splits (the row terms) against the static scratch before any HIP call
    (no GPU needed to see the rejection); with splits it uses as many as fit."""
    l = _lib.lib()
    need = 2 * _pad(total * Hq * 4)  # Delta and lse2 planes
    assert (need <= A.NOALLOC_SCRATCH_BYTES) == ok
    if ok:
        return  # a fitting problem would launch kernels
    rc = l.attn_varlen_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, total, total, total, total, Hq,
                                   1 if D == 256 else 8, D, 0.1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == E["ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL"]
    assert "static scratch" in A.attn_varlen_error_string(rc)


def test_noalloc_argument_errors_come_first():
    l = _lib.lib()
    assert l.attn_varlen_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 64, 4, 2, 96, 0.1, 0, FAKE,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, None) == E["ATTN_VARLEN_ERR_BAD_HEAD_DIM"]
    assert l.attn_varlen_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 64, 4, 2, 64, 0.1, 0, None,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, None) == E["ATTN_VARLEN_ERR_NULL_POINTER"]


def test_stored_ds_workspace_size():
    """The stored-dS backward's workspace: the recomputing one's plus one bf16 row
    of 64 + 128 * ceil(max_seqlen_q / 128) columns per (query head, key), rounded
    up to 256 bytes; 0 where the path does not apply."""
    plain = A.attn_varlen_bwd_workspace_size(10, 16384, 16384, 32, 8, 128)
    got = A.attn_varlen_bwd_ds_workspace_size(10, 16384, 16384, 3523, 3523, 32, 8, 128)
    ds = 32 * 16384 * (64 + 128 * 28) * 2
    assert got == plain + (ds + 255) // 256 * 256
    assert A.attn_varlen_bwd_ds_workspace_size(1, 100, 90, 100, 90, 4, 2, 64) == (
        A.attn_varlen_bwd_workspace_size(1, 100, 90, 4, 2, 64) + (4 * 90 * (64 + 128) * 2 + 255) // 256 * 256)
    assert A.attn_varlen_bwd_ds_workspace_size(8, 32768, 32768, 4096, 4096, 8, 1, 256) == 0  # head dim 256
    assert A.attn_varlen_bwd_ds_workspace_size(1, 0, 100, 0, 100, 4, 2, 64) == 0              # no queries
    assert A.attn_varlen_bwd_ds_workspace_size(1, 65536, 65536, 65536, 65536, 32, 8, 128) == 0  # rows >= 2 GiB
    assert A.attn_varlen_bwd_ds_workspace_size(1, 100, 100, 100, 100, 4, 3, 64) == 0          # bad heads


def test_stored_ds_call_argument_errors():
    """attn_varlen_bwd_stored_ds: head dim 256 has no stored-dS path, and the
    workspace must hold the dS buffer; both are checked before any HIP call."""
    l = _lib.lib()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 64, 4, 2]
    tail = [0.1, 0, -1, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert l.attn_varlen_bwd_stored_ds(*args, 256, *tail, FAKE, 1 << 30, None) == E["ATTN_VARLEN_ERR_BAD_HEAD_DIM"]
    need = A.attn_varlen_bwd_ds_workspace_size(1, 64, 64, 64, 64, 4, 2, 128)
    assert need > A.attn_varlen_bwd_workspace_size(1, 64, 64, 4, 2, 128)
    assert l.attn_varlen_bwd_stored_ds(*args, 128, *tail, FAKE, need - 16, None) == E["ATTN_VARLEN_ERR_WORKSPACE"]
    assert l.attn_varlen_bwd_stored_ds(*args, 128, *tail, None, need, None) == E["ATTN_VARLEN_ERR_WORKSPACE"]


def longest_sequence(heads: int, head_dim: int, overrun: int) -> int:
    # one sequence's rows plus the kernels' tile overrun must span < 2 GiB (32-bit buffer offsets)
    return ((1 << 31) - 1) // (heads * head_dim * 2) - overrun


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 1, 256), (16, 16, 64)])
def test_sequence_length_limit(Hq, Hkv, D):
    # tiles run up to 127 query rows (the dK / dV kernel's query steps) and 63 key rows past a sequence's end
    lq, lk = longest_sequence(Hq, D, 128), longest_sequence(Hkv, D, 64)
    assert (lq + 128) * Hq * D * 2 < (1 << 31) <= (lq + 129) * Hq * D * 2
    assert (lk + 64) * Hkv * D * 2 < (1 << 31) <= (lk + 65) * Hkv * D * 2
    sizes = dict(D=D, Hq=Hq, Hkv=Hkv, total_q=lq + 100, total_k=lk + 100)
    # at the limit every size check passes: the call stops at the causal flag, checked after them
    assert fwd_call(max_q=lq, max_k=lk, causal=2, **sizes) == E["ATTN_VARLEN_ERR_BAD_FLAG"]
    assert bwd_call(max_q=lq, max_k=lk, causal=2, **sizes) == E["ATTN_VARLEN_ERR_BAD_FLAG"]
    # one row more on either side is rejected
    for mq, mk in ((lq + 1, lk), (lq, lk + 1)):
        assert fwd_call(max_q=mq, max_k=mk, **sizes) == E["ATTN_VARLEN_ERR_BAD_SEQLEN"]
        assert bwd_call(max_q=mq, max_k=mk, **sizes) == E["ATTN_VARLEN_ERR_BAD_SEQLEN"]
