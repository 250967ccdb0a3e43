"""Brute-force check of the kernels' tile plans on the CPU.

The kernels never test (query, key) pairs one by one outside the tiles they
mask: a work item visits a range of tiles, runs some of them without a mask and
masks the rest (FlashAttention repository guide, Core Abstractions: the
block-info helper that gives the key blocks a query block meets under causal and
local masks). The results are exact only if

  * every visible pair lies in a visited tile (tiles left out hold only hidden
    pairs),
  * every tile run without a mask holds only visible pairs of real rows and keys,
  * the forward's left-edge tiles (masked scores, unmasked probability path)
    cross no row's right edge and the end of the keys, and every row that reaches
    them sees at least a tile of keys.

`attn_varlen_tile_plan_host` returns the plan the kernels compute (the same
functions, compiled for the host); this test enumerates every (query, key) pair
of small sequences, for every head dim, causal and not, with windows of every
kind and Lq != Lk, and checks the three properties against the visibility rule
of the float64 oracle (`oracle.attention.visible`).
"""
import itertools

import numpy as np
import pytest

import exact_attention_varlen_amd as A
import oracle.attention as O

LENGTHS = [0, 1, 31, 63, 64, 65, 127, 128, 129, 200, 257, 383]
WINDOWS = [(-1, -1), (0, 0), (0, -1), (5, 3), (31, -1), (32, -1), (63, 2), (64, -1), (65, 10), (100, 37),
           (130, -1), (-1, 0), (-1, 50), (200, 200), (1000, -1), (-1, 1000)]


def _right_ok(Lq, Lk, causal, window):
    """Pairs that are not past their row's right band edge nor past the keys."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    diag = i + (Lk - Lq)
    ok = np.ones((Lq, Lk), dtype=bool)
    if causal:
        ok &= j <= diag
    if window[1] >= 0:
        ok &= j <= diag + window[1]
    return ok


def _check_query_blocks(kind, D, Lq, Lk, causal, window):
    vis = O.visible(Lq, Lk, causal, None, window) if Lq and Lk else np.zeros((Lq, Lk), dtype=bool)
    right_ok = _right_ok(Lq, Lk, causal, window)
    nvis = vis.sum(axis=1)
    heads = 4 if kind & A.PLAN_GROUP4 else 2 if kind & A.PLAN_GROUP2 else 1
    nblocks = -(-Lq // (128 // heads))
    covered = np.zeros(Lq, dtype=int)
    for m in range(nblocks):
        p = A.attn_varlen_tile_plan_host(kind, D, Lq, Lk, causal, window[0], window[1], m)
        bm, bn = p["size"], p["tile"]
        r0, r1 = max(p["start"], 0), min(p["start"] + bm, Lq)
        assert r0 < r1, (p, Lq)
        covered[r0:r1] += 1
        rows = vis[r0:r1]
        tag = (kind, D, Lq, Lk, causal, window, m, p)
        # visited tiles hold every visible pair
        jj = np.nonzero(rows.any(axis=0))[0]
        if jj.size:
            assert p["lo"] <= jj.min() // bn and jj.max() // bn < p["hi"], tag
        # unmasked tiles: every pair visible, every key real
        for t in range(p["full_lo"], p["full_hi"]):
            assert p["lo"] <= t < p["hi"], tag
            k0, k1 = t * bn, (t + 1) * bn
            assert k1 <= Lk, tag
            assert rows[:, k0:k1].all(), tag
        # forward left-edge tiles: no row's right edge or key end inside; rows
        # that reach them see at least a tile of keys
        assert bm == 128 // heads, tag
        if p["left_edge"]:
            assert kind & 0xF == A.PLAN_FWD and window[0] >= 0, tag
            k0, k1 = p["lo"] * bn, (p["lo"] + p["left_edge"]) * bn
            assert k1 <= Lk and right_ok[r0:r1, k0:k1].all(), tag
            reach = rows[:, k0:k1].any(axis=1)
            assert (nvis[r0:r1][reach] >= bn).all(), tag
            assert p["full_lo"] == p["lo"] + p["left_edge"], tag
    # the query blocks partition the rows
    assert (covered == 1).all()


def _check_key_blocks(D, Lq, Lk, causal, window):
    vis = O.visible(Lq, Lk, causal, None, window) if Lq and Lk else np.zeros((Lq, Lk), dtype=bool)
    nblocks = -(-Lk // 128)
    for n in range(nblocks):
        p = A.attn_varlen_tile_plan_host(A.PLAN_DKDV, D, Lq, Lk, causal, window[0], window[1], n)
        bnk, bmq = p["size"], p["tile"]
        c0, c1 = p["start"], min(p["start"] + bnk, Lk)
        assert c0 == n * bnk and c0 < c1
        cols = vis[:, c0:c1]
        tag = (D, Lq, Lk, causal, window, n, p)
        ii = np.nonzero(cols.any(axis=1))[0]
        if ii.size:
            assert p["lo"] <= ii.min() // bmq and ii.max() // bmq < p["hi"], tag
        for s in range(p["full_lo"], p["full_hi"]):
            assert p["lo"] <= s < p["hi"], tag
            # rows past Lq read as zero and add nothing: only real rows must see every key
            assert cols[s * bmq:min((s + 1) * bmq, Lq)].all(), tag


CASES = [(D, c, w) for D in (64, 128, 256) for c in (False, True) for w in WINDOWS]
# the forward and dQ blocks for KV groups of one head, of 2 and of 4 (or more)
QUERY_KINDS = [k | g for k in (A.PLAN_FWD, A.PLAN_DQ) for g in (0, A.PLAN_GROUP2, A.PLAN_GROUP4)]


@pytest.mark.parametrize("D,causal,window", CASES, ids=[f"d{D}-{'c' if c else 'f'}-w{w[0]}_{w[1]}"
                                                        for D, c, w in CASES])
def test_tile_plans_cover_every_visible_pair(D, causal, window):
    for Lq, Lk in itertools.product(LENGTHS, LENGTHS):
        for kind in QUERY_KINDS:
            _check_query_blocks(kind, D, Lq, Lk, causal, window)
        _check_key_blocks(D, Lq, Lk, causal, window)


def test_tile_plans_random_long():
    """Longer sequences (many tiles, tile-boundary band edges), drawn at random."""
    rng = np.random.default_rng(0)
    for _ in range(60):
        D = int(rng.choice([64, 128, 256]))
        Lq, Lk = (int(x) for x in rng.integers(1, 1200, size=2))
        causal = bool(rng.integers(0, 2))
        window = tuple(int(rng.choice([-1, int(rng.integers(0, 4)) * 32, int(rng.integers(0, 700))]))
                       for _ in range(2))
        for kind in QUERY_KINDS:
            _check_query_blocks(kind, D, Lq, Lk, causal, window)
        _check_key_blocks(D, Lq, Lk, causal, window)


def test_tile_plan_argument_errors():
    E = A.AttnVarlenError
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(A.PLAN_FWD, 96, 10, 10, False, -1, -1, 0)
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(A.PLAN_FWD, 64, 10, 10, False, -1, -1, 1)  # one query block only
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(A.PLAN_DKDV, 64, 10, 300, False, -1, -1, 3)
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(7, 64, 10, 10, False, -1, -1, 0)
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(A.PLAN_DQ, 64, -1, 10, False, -1, -1, 0)
    with pytest.raises(E):  # grouped heads apply to query blocks only
        A.attn_varlen_tile_plan_host(A.PLAN_DKDV | A.PLAN_GROUP4, 64, 10, 10, False, -1, -1, 0)
    with pytest.raises(E):
        A.attn_varlen_tile_plan_host(A.PLAN_FWD | A.PLAN_GROUP2 | A.PLAN_GROUP4, 64, 10, 10, False, -1, -1, 0)
    with pytest.raises(E):  # 32-row blocks: rows 0 .. 39 make two
        A.attn_varlen_tile_plan_host(A.PLAN_FWD | A.PLAN_GROUP4, 64, 40, 40, False, -1, -1, 2)


@pytest.mark.parametrize("field,delta", [("hi", -1), ("lo", 1), ("full_hi", 1), ("full_lo", -1), ("left_edge", 2)])
def test_checker_catches_a_plan_off_by_one_tile(monkeypatch, field, delta):
    """Planted mistakes in the plan (one tile too few visited, one too many
    unmasked) must fail the brute-force check somewhere in the sweep."""
    real = A.attn_varlen_tile_plan_host

    def shifted(*args):
        p = real(*args)
        p[field] += delta
        return p

    monkeypatch.setattr(A, "attn_varlen_tile_plan_host", shifted)
    with pytest.raises(AssertionError):
        for D, causal, window in [(128, True, (-1, -1)), (64, False, (100, 37)), (256, True, (200, -1)),
                                  (128, False, (130, -1))]:
            for Lq, Lk in itertools.product(LENGTHS, LENGTHS):
                for kind in QUERY_KINDS:
                    _check_query_blocks(kind, D, Lq, Lk, causal, window)
                _check_key_blocks(D, Lq, Lk, causal, window)
