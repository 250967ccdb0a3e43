"""Pins for the float64 CPU oracle.

None of these re-types the oracle's formulas. Each check rests on something
outside the oracle: a hand-worked example, a closed form, an invariant of the
mathematics, central finite differences, or PyTorch's float64
``scaled_dot_product_attention`` (the library the pages validate against: "[FA4/B200]
return_lse=True makes D64 forward about 19% faster", repro script, ``main``).
The checks are written as functions of an oracle module so that the mutation
tests at the bottom can show that planted mistakes in the oracle are caught.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seqlens_q, Hq, Hkv, D, seed=0, seqlens_k=None):
    rng = np.random.default_rng(seed)
    seqlens_k = seqlens_q if seqlens_k is None else seqlens_k
    cu_q = W.cu_from_lengths(seqlens_q)
    cu_k = W.cu_from_lengths(seqlens_k)
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    do = rng.standard_normal((cu_q[-1], Hq, D))
    return q, k, v, do, cu_q, cu_k


# ---------------------------------------------------------------------------
# pin functions (take the oracle module so mutations can be tested)
# ---------------------------------------------------------------------------

def check_hand_worked(mod):
    with open(os.path.join(GOLDEN, "hand_worked_2key.json")) as f:
        g = json.load(f)
    q, k, v, do = (np.array(g[x]) for x in ("q", "k", "v", "dout"))
    e = g["expected"]
    out, lse = mod.forward(q, k, v, g["cu_seqlens_q"], g["cu_seqlens_k"], g["softmax_scale"], False)
    np.testing.assert_allclose(out, e["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, e["lse"], rtol=0, atol=1e-14)
    dq, dk, dv = mod.backward(q, k, v, g["cu_seqlens_q"], g["cu_seqlens_k"], g["softmax_scale"], False, do)
    np.testing.assert_allclose(dq, e["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, e["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, e["dv"], rtol=0, atol=1e-14)
    c = g["causal_variant"]
    out, lse = mod.forward(np.array(c["q"]), k, v, c["cu_seqlens_q"], c["cu_seqlens_k"], g["softmax_scale"], True)
    np.testing.assert_allclose(out, c["expected_out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, c["expected_lse"], rtol=0, atol=1e-14)


def check_zero_query_closed_form(mod, causal):
    # Q = 0 makes every visible score 0, so P is uniform over the visible keys:
    # O_i is the mean of the visible v_j and LSE_i = log(#visible).
    seqlens = [5, 9, 1, 7]
    q, k, v, do, cu, _ = rand_problem(seqlens, 4, 2, 8, seed=1)
    q[:] = 0.0
    out, lse = mod.forward(q, k, v, cu, cu, 0.37, causal)
    for b, L in enumerate(seqlens):
        c = cu[b]
        for h in range(4):
            g = h // 2
            for i in range(L):
                n = (i + 1) if causal else L
                exp_o = v[c:c + n, g, :].mean(axis=0)
                np.testing.assert_allclose(out[c + i, h], exp_o, rtol=0, atol=1e-13)
                assert abs(lse[h, c + i] - math.log(n)) < 1e-13


def check_single_key(mod):
    # One visible key: P = 1, O = v_0, LSE = s_00 (no log-sum beyond one term).
    q, k, v, do, cu_q, cu_k = rand_problem([3], 2, 1, 16, seed=2, seqlens_k=[1])
    scale = 0.25
    out, lse = mod.forward(q, k, v, cu_q, cu_k, scale, False)
    for h in range(2):
        for i in range(3):
            np.testing.assert_allclose(out[i, h], v[0, 0], rtol=0, atol=1e-14)
            assert abs(lse[h, i] - scale * float(q[i, h] @ k[0, 0])) < 1e-13


def check_identical_keys(mod):
    # All keys equal: every score in a row is equal, so P is uniform.
    q, k, v, do, cu, _ = rand_problem([6], 2, 2, 8, seed=3)
    k[:] = k[0:1]
    out, lse = mod.forward(q, k, v, cu, cu, 0.5, False)
    for h in range(2):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(v[:, h].mean(0), (6, 8)), atol=1e-13)
        s0 = 0.5 * (q[:, h] @ k[0, h])
        np.testing.assert_allclose(lse[h], s0 + math.log(6), atol=1e-13)


def check_key_shift(mod, causal):
    # Adding c to every key of a sequence adds scale*q_i.c to every visible score
    # of row i: softmax is unchanged, LSE moves by scale*q_i.c.
    q, k, v, do, cu, _ = rand_problem([7, 4], 2, 1, 8, seed=4)
    scale = 0.3
    out, lse = mod.forward(q, k, v, cu, cu, scale, causal)
    c = np.linspace(-1, 1, 8)
    out2, lse2 = mod.forward(q, k + c, v, cu, cu, scale, causal)
    np.testing.assert_allclose(out2, out, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * np.einsum("thd,d->ht", q, c), atol=1e-12)


def check_permutation(mod):
    # Non-causal: permuting keys together with values leaves O and LSE unchanged;
    # permuting queries permutes O and LSE the same way.
    q, k, v, do, cu, _ = rand_problem([9], 2, 2, 8, seed=5)
    out, lse = mod.forward(q, k, v, cu, cu, 0.4, False)
    pk = np.random.default_rng(6).permutation(9)
    out2, lse2 = mod.forward(q, k[pk], v[pk], cu, cu, 0.4, False)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = np.random.default_rng(7).permutation(9)
    out3, lse3 = mod.forward(q[pq], k, v, cu, cu, 0.4, False)
    np.testing.assert_allclose(out3, out[pq], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[:, pq], atol=1e-13)


def check_row_sums(mod, causal):
    q, k, v, do, cu, _ = rand_problem([11, 6], 4, 2, 8, seed=8)
    for b in range(2):
        for h in range(4):
            p = mod.probabilities(q, k, cu, cu, 0.7, causal, b, h)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
            assert (p >= 0).all()
            if causal:
                assert np.all(np.triu(p, 1) == 0)


def check_probabilities(mod, causal, window=None):
    """The attention matrix against torch's float64 softmax of the masked,
    scaled scores (K/V heads repeated with repeat_interleave; the mask built
    from tril/triu at the bottom-right diagonal), and P V against the forward's
    output and log-sum-exp of the same scores against its LSE."""
    q, k, v, do, cu_q, cu_k = rand_problem([9, 14, 5], 6, 2, 8, seed=21, seqlens_k=[12, 14, 3])
    scale = 0.6
    out, lse = mod.forward(q, k, v, cu_q, cu_k, scale, causal, window=window)
    kr = torch.tensor(k).repeat_interleave(3, dim=1)
    vr = torch.tensor(v).repeat_interleave(3, dim=1)
    for b in range(3):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        ones = torch.ones(Lq, Lk, dtype=torch.bool)
        keep = ones.clone()
        if causal:
            keep &= torch.tril(ones, diagonal=Lk - Lq)
        if window is not None and window[1] >= 0:
            keep &= torch.tril(ones, diagonal=Lk - Lq + window[1])
        if window is not None and window[0] >= 0:
            keep &= torch.triu(ones, diagonal=Lk - Lq - window[0])
        for h in range(6):
            qh = torch.tensor(q[cu_q[b]:cu_q[b + 1], h])
            kh = kr[cu_k[b]:cu_k[b + 1], h]
            s = (qh @ kh.T) * scale
            s = s.masked_fill(~keep, float("-inf"))
            want = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0).numpy()
            p = mod.probabilities(q, k, cu_q, cu_k, scale, causal, b, h, window=window)
            np.testing.assert_allclose(p, want, rtol=0, atol=1e-13)
            np.testing.assert_allclose(p @ vr[cu_k[b]:cu_k[b + 1], h].numpy(), out[cu_q[b]:cu_q[b + 1], h],
                                       rtol=0, atol=1e-13)
            np.testing.assert_allclose(torch.logsumexp(s, dim=-1).numpy(), lse[h, cu_q[b]:cu_q[b + 1]],
                                       rtol=0, atol=1e-13)


def sdpa_reference(q, k, v, cu_q, cu_k, scale, causal, Hq, Hkv, requires_grad=False):
    """Per-sequence torch float64 SDPA with the library's own GQA grouping."""
    outs, lses, leaves = [], [], []
    for b in range(len(cu_q) - 1):
        qb = torch.tensor(q[cu_q[b]:cu_q[b + 1]]).permute(1, 0, 2).contiguous().requires_grad_(requires_grad)
        kb = torch.tensor(k[cu_k[b]:cu_k[b + 1]]).permute(1, 0, 2).contiguous().requires_grad_(requires_grad)
        vb = torch.tensor(v[cu_k[b]:cu_k[b + 1]]).permute(1, 0, 2).contiguous().requires_grad_(requires_grad)
        Lq, Lk = qb.shape[1], kb.shape[1]
        mask = None
        if causal:
            i = torch.arange(Lq)[:, None]
            j = torch.arange(Lk)[None, :]
            mask = j <= i + (Lk - Lq)
        ob = F.scaled_dot_product_attention(qb[None], kb[None], vb[None], attn_mask=mask, scale=scale,
                                            enable_gqa=(Hq != Hkv))[0]
        kr = kb.detach().repeat_interleave(Hq // Hkv, dim=0)
        sc = scale * (qb.detach() @ kr.transpose(1, 2))
        if causal:
            sc = sc.masked_fill(~mask, -math.inf)
        lses.append(torch.logsumexp(sc, dim=-1))
        outs.append(ob.permute(1, 0, 2))
        leaves.append((qb, kb, vb))
    return outs, lses, leaves


def check_against_sdpa(mod, causal):
    wl = W.tiny(causal)
    inp = W.make_inputs(wl)
    q, k, v, do = (W.to_f64(inp[x]) for x in ("q", "k", "v", "dout"))
    cu = wl.cu_seqlens_q
    out, lse = mod.forward(q, k, v, cu, cu, wl.softmax_scale, causal)
    outs, lses, leaves = sdpa_reference(q, k, v, cu, cu, wl.softmax_scale, causal, 4, 2, requires_grad=True)
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        np.testing.assert_allclose(out[sl], outs[b].detach().numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, sl], lses[b].numpy(), rtol=0, atol=1e-12)
    dq, dk, dv = mod.backward(q, k, v, cu, cu, wl.softmax_scale, causal, do)
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        dob = torch.tensor(do[sl])
        (outs[b] * dob).sum().backward()
        qb, kb, vb = leaves[b]
        np.testing.assert_allclose(dq[sl], qb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[sl], kb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[sl], vb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)


def check_finite_differences(mod, causal, seqlens_q=(3, 5), seqlens_k=None, window=None):
    q, k, v, do, cu_q, cu_k = rand_problem(list(seqlens_q), 4, 2, 4, seed=9,
                                           seqlens_k=None if seqlens_k is None else list(seqlens_k))
    scale = 0.6
    kw = {} if window is None else {"window": window}
    dq, dk, dv = mod.backward(q, k, v, cu_q, cu_k, scale, causal, do, **kw)

    def loss(qq, kk, vv):
        o, _ = mod.forward(qq, kk, vv, cu_q, cu_k, scale, causal, **kw)
        return float((o * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(num).max())
        assert err < 1e-6, (name, err)


def check_gradient_invariants(mod, causal):
    # sum_j dS_ij = 0 for each row  =>  sum_j dK_j = 0 per sequence and KV head.
    # sum_j P_ij = 1 for each row    =>  sum_j dV_j = sum over the group's heads and rows of dO_i.
    seqlens = [13, 4, 8]
    q, k, v, do, cu, _ = rand_problem(seqlens, 6, 2, 8, seed=10)
    dq, dk, dv = mod.backward(q, k, v, cu, cu, 0.45, causal, do)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        for g in range(2):
            np.testing.assert_allclose(dk[sl, g].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[sl, g].sum(axis=0), do[sl, 3 * g:3 * g + 3].sum(axis=(0, 1)), atol=1e-12)


def check_zero_query_dv(mod, causal):
    # Q = 0: P_ij = 1/#visible_i, so dV_j = sum_{h in group} sum_{i sees j} dO_i / #visible_i.
    seqlens = [6, 3]
    q, k, v, do, cu, _ = rand_problem(seqlens, 4, 2, 4, seed=11)
    q[:] = 0
    _, _, dv = mod.backward(q, k, v, cu, cu, 1.0, causal, do)
    for b, L in enumerate(seqlens):
        c = cu[b]
        for g in range(2):
            for j in range(L):
                acc = np.zeros(4)
                for h in (2 * g, 2 * g + 1):
                    for i in range(L):
                        n = (i + 1) if causal else L
                        if (not causal) or j <= i:
                            acc += do[c + i, h] / n
                np.testing.assert_allclose(dv[c + j, g], acc, atol=1e-13)


def check_varlen_equals_separate(mod, causal):
    seqlens = [5, 12, 7]
    q, k, v, do, cu, _ = rand_problem(seqlens, 4, 1, 8, seed=12)
    out, lse = mod.forward(q, k, v, cu, cu, 0.5, causal)
    dq, dk, dv = mod.backward(q, k, v, cu, cu, 0.5, causal, do)
    for b in range(3):
        sl = slice(cu[b], cu[b + 1])
        L = seqlens[b]
        o1, l1 = mod.forward(q[sl], k[sl], v[sl], [0, L], [0, L], 0.5, causal)
        g1 = mod.backward(q[sl], k[sl], v[sl], [0, L], [0, L], 0.5, causal, do[sl])
        np.testing.assert_allclose(out[sl], o1, atol=1e-14)
        np.testing.assert_allclose(lse[:, sl], l1, atol=1e-14)
        for a, bb in zip((dq[sl], dk[sl], dv[sl]), g1):
            np.testing.assert_allclose(a, bb, atol=1e-13)


def check_gqa_equals_mha(mod, causal):
    # KV head g serves query heads [g*r, (g+1)*r): the same as MHA on K/V repeated
    # head-wise with torch.repeat_interleave (PyTorch's own GQA convention).
    seqlens = [6, 10]
    Hq, Hkv = 8, 2
    q, k, v, do, cu, _ = rand_problem(seqlens, Hq, Hkv, 8, seed=13)
    kr = torch.tensor(k).repeat_interleave(Hq // Hkv, dim=1).numpy()
    vr = torch.tensor(v).repeat_interleave(Hq // Hkv, dim=1).numpy()
    out, lse = mod.forward(q, k, v, cu, cu, 0.5, causal)
    out2, lse2 = mod.forward(q, kr, vr, cu, cu, 0.5, causal)
    np.testing.assert_allclose(out, out2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    dq, dk, dv = mod.backward(q, k, v, cu, cu, 0.5, causal, do)
    dq2, dk2, dv2 = mod.backward(q, kr, vr, cu, cu, 0.5, causal, do)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(dk2.shape[0], Hkv, Hq // Hkv, -1).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(dv2.shape[0], Hkv, Hq // Hkv, -1).sum(2), atol=1e-13)


def check_empty_rows(mod):
    # Causal with Lq > Lk: queries i < Lq - Lk see no key -> O = 0, LSE = -inf, no gradient.
    q, k, v, do, cu_q, cu_k = rand_problem([5], 2, 1, 4, seed=14, seqlens_k=[2])
    out, lse = mod.forward(q, k, v, cu_q, cu_k, 1.0, True)
    assert np.all(out[:3] == 0) and np.all(np.isneginf(lse[:, :3]))
    assert np.all(np.isfinite(lse[:, 3:]))
    # query 3 sees exactly key 0 -> O = v_0, LSE = s_30
    np.testing.assert_allclose(out[3, :], np.broadcast_to(v[0, 0], (2, 4)), atol=1e-14)
    dq, dk, dv = mod.backward(q, k, v, cu_q, cu_k, 1.0, True, do)
    assert np.all(dq[:3] == 0)


# Local (sliding-window) attention. The band is built here with torch.tril /
# torch.triu diagonals, independently of the oracle's own mask code.
WINDOWS = [(3, 1), (0, 0), (2, -1), (-1, 2), (5, 0), (1, 3)]


def band_mask(Lq, Lk, causal, window):
    """Visible (query, key) pairs: diagonals relative to the bottom-right-aligned one."""
    off = Lk - Lq
    left, right = window
    ones = torch.ones(Lq, Lk, dtype=torch.bool)
    m = ones.clone()
    if causal:
        m &= torch.tril(ones, diagonal=off)
    if right >= 0:
        m &= torch.tril(ones, diagonal=off + right)
    if left >= 0:
        m &= torch.triu(ones, diagonal=off - left)
    return m


def check_window_against_sdpa(mod, causal, window):
    # torch float64 SDPA with the band as a boolean mask, per sequence; rows whose
    # band is empty must give O = 0 and LSE = -inf (SDPA itself gives NaN there).
    seqlens_q, seqlens_k = [9, 4, 12], [9, 7, 5]
    Hq, Hkv, scale = 4, 2, 0.45
    q, k, v, do, cu_q, cu_k = rand_problem(seqlens_q, Hq, Hkv, 8, seed=21, seqlens_k=seqlens_k)
    out, lse = mod.forward(q, k, v, cu_q, cu_k, scale, causal, window=window)
    dq, dk, dv = mod.backward(q, k, v, cu_q, cu_k, scale, causal, do, window=window)
    for b in range(3):
        sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        Lq, Lk = seqlens_q[b], seqlens_k[b]
        m = band_mask(Lq, Lk, causal, window)
        rows = m.any(dim=1).numpy()
        qb = torch.tensor(q[sq]).permute(1, 0, 2).contiguous().requires_grad_(True)
        kb = torch.tensor(k[sk]).permute(1, 0, 2).contiguous().requires_grad_(True)
        vb = torch.tensor(v[sk]).permute(1, 0, 2).contiguous().requires_grad_(True)
        kr, vr = kb.repeat_interleave(Hq // Hkv, dim=0), vb.repeat_interleave(Hq // Hkv, dim=0)
        ob = F.scaled_dot_product_attention(qb[None], kr[None], vr[None], attn_mask=m, scale=scale)[0]
        ob = torch.where(torch.tensor(rows)[None, :, None], ob, torch.zeros_like(ob))
        sc = (scale * (qb @ kr.transpose(1, 2))).masked_fill(~m, -math.inf)
        lref = torch.logsumexp(sc, dim=-1).detach().numpy()
        o_ref = ob.permute(1, 0, 2).detach().numpy()
        np.testing.assert_allclose(out[sq][rows], o_ref[rows], rtol=0, atol=1e-12)
        assert np.all(out[sq][~rows] == 0)
        np.testing.assert_allclose(lse[:, sq][:, rows], lref[:, rows], rtol=0, atol=1e-12)
        assert np.all(np.isneginf(lse[:, sq][:, ~rows]))
        (ob * torch.tensor(do[sq]).permute(1, 0, 2)).sum().backward()
        np.testing.assert_allclose(dq[sq], qb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[sk], kb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[sk], vb.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)


def check_window_zero_query(mod, causal, window):
    # Q = 0: O_i is the mean of v over the keys lo .. hi of row i's band, with
    # lo = i + off - left and hi = i + off + right clipped to the sequence; LSE_i is
    # log of the band's size; an empty band gives O = 0, LSE = -inf.
    seqlens_q, seqlens_k = [7, 10], [11, 4]
    q, k, v, do, cu_q, cu_k = rand_problem(seqlens_q, 2, 1, 4, seed=22, seqlens_k=seqlens_k)
    q[:] = 0.0
    out, lse = mod.forward(q, k, v, cu_q, cu_k, 0.8, causal, window=window)
    left, right = window
    if causal:
        right = 0 if right < 0 else min(right, 0)
    for b in range(2):
        Lq, Lk = seqlens_q[b], seqlens_k[b]
        off = Lk - Lq
        for i in range(Lq):
            lo = max(0, i + off - left) if left >= 0 else 0
            hi = min(Lk - 1, i + off + right) if right >= 0 else Lk - 1
            for h in range(2):
                if lo > hi:
                    assert np.all(out[cu_q[b] + i, h] == 0) and np.isneginf(lse[h, cu_q[b] + i])
                else:
                    exp_o = v[cu_k[b] + lo:cu_k[b] + hi + 1, 0].mean(axis=0)
                    np.testing.assert_allclose(out[cu_q[b] + i, h], exp_o, rtol=0, atol=1e-13)
                    assert abs(lse[h, cu_q[b] + i] - math.log(hi - lo + 1)) < 1e-13


def check_window_rows(mod, causal, window):
    # the row-sampled forms agree with the full oracle under a window
    seqlens = [13, 6]
    q, k, v, do, cu, _ = rand_problem(seqlens, 4, 2, 8, seed=23)
    out, lse = mod.forward(q, k, v, cu, cu, 0.5, causal, window=window)
    dq, dk, dv = mod.backward(q, k, v, cu, cu, 0.5, causal, do, window=window)
    rows = [0, 3, 7, 12, 13, 18]
    r, o, l = mod.forward_rows(q, k, v, cu, cu, 0.5, causal, rows, window=window)
    np.testing.assert_allclose(o, out[r], atol=1e-13)
    np.testing.assert_allclose(l, lse[:, r], atol=1e-13)
    r, g = mod.backward_dq_rows(q, k, v, cu, cu, 0.5, causal, do, rows, window=window)
    np.testing.assert_allclose(g, dq[r], atol=1e-12)
    r, gk, gv = mod.backward_dkdv_rows(q, k, v, cu, cu, 0.5, causal, do, [1, 5, 12, 14, 18], window=window)
    np.testing.assert_allclose(gk, dk[r], atol=1e-12)
    np.testing.assert_allclose(gv, dv[r], atol=1e-12)


# ---------------------------------------------------------------------------
# the tests
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    check_hand_worked(O)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(causal):
    check_zero_query_closed_form(O, causal)


def test_single_key():
    check_single_key(O)


def test_identical_keys():
    check_identical_keys(O)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    check_key_shift(O, causal)


def test_permutation_equivariance():
    check_permutation(O)


@pytest.mark.parametrize("causal", [False, True])
def test_row_sums(causal):
    check_row_sums(O, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [None, (3, 1), (0, -1), (-1, 2)])
def test_probabilities_against_torch_softmax(causal, window):
    check_probabilities(O, causal, window)


def test_mutation_probabilities_scale_and_grouping_are_caught():
    def unscaled(q, k, cu_q, cu_k, scale, causal, b, h, window=None):
        return O.probabilities(q, k, cu_q, cu_k, 1.0, causal, b, h, window=window)
    assert _fails(check_probabilities, _mutant(probabilities=unscaled), False)
    assert _fails(check_probabilities, _mutant(kv_head_of=lambda h, hq, hkv: h % hkv), True)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_f64(causal):
    check_against_sdpa(O, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    check_finite_differences(O, causal)


def test_finite_differences_unequal_lengths_causal():
    # Lq != Lk per sequence (bottom-right causal alignment), including a row-free prefix
    check_finite_differences(O, True, seqlens_q=(4, 2), seqlens_k=(2, 5))


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    check_gradient_invariants(O, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_dv(causal):
    check_zero_query_dv(O, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_separate(causal):
    check_varlen_equals_separate(O, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha(causal):
    check_gqa_equals_mha(O, causal)


def test_empty_rows():
    check_empty_rows(O)


def test_zero_length_sequences():
    q, k, v, do, cu, _ = rand_problem([0, 4, 0, 3], 2, 1, 4, seed=15)
    out, lse = O.forward(q, k, v, cu, cu, 0.5, True)
    o2, l2 = O.forward(q, k, v, [0, 4, 7], [0, 4, 7], 0.5, True)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_row_sampled_forms_match_full(causal):
    seqlens = [9, 17, 4]
    q, k, v, do, cu, _ = rand_problem(seqlens, 4, 2, 8, seed=16)
    out, lse = O.forward(q, k, v, cu, cu, 0.5, causal)
    dq, dk, dv = O.backward(q, k, v, cu, cu, 0.5, causal, do)
    rows = np.array([0, 3, 8, 9, 20, 25, 29])
    r, o_r, l_r = O.forward_rows(q, k, v, cu, cu, 0.5, causal, rows)
    np.testing.assert_array_equal(r, rows)
    np.testing.assert_allclose(o_r, out[rows], atol=1e-14)
    np.testing.assert_allclose(l_r, lse[:, rows], atol=1e-14)
    r, dq_r = O.backward_dq_rows(q, k, v, cu, cu, 0.5, causal, do, rows)
    np.testing.assert_allclose(dq_r, dq[rows], atol=1e-13)
    r, dk_r, dv_r = O.backward_dkdv_rows(q, k, v, cu, cu, 0.5, causal, do, rows, chunk=5)
    np.testing.assert_allclose(dk_r, dk[rows], atol=1e-13)
    np.testing.assert_allclose(dv_r, dv[rows], atol=1e-13)


def test_chunking_does_not_change_results():
    q, k, v, do, cu, _ = rand_problem([37], 2, 1, 8, seed=17)
    a = O.forward(q, k, v, cu, cu, 0.5, True, chunk=2048)
    b = O.forward(q, k, v, cu, cu, 0.5, True, chunk=5)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)
    ga = O.backward(q, k, v, cu, cu, 0.5, True, do, chunk=2048)
    gb = O.backward(q, k, v, cu, cu, 0.5, True, do, chunk=6)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, atol=1e-13)


# ---------------------------------------------------------------------------
# mutation tests: plausible mistakes planted in a copy of the oracle must be caught
# ---------------------------------------------------------------------------

def _mutant(**overrides):
    m = types.ModuleType("oracle_mutant")
    src_globals = dict(vars(O))
    m.__dict__.update(src_globals)
    # rebind the functions so that they look names up in the mutant's namespace
    for name, fn in list(src_globals.items()):
        if isinstance(fn, types.FunctionType) and fn.__module__ == O.__name__:
            m.__dict__[name] = types.FunctionType(fn.__code__, m.__dict__, fn.__name__, fn.__defaults__)
    m.__dict__.update(overrides)
    return m


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_against_torch_sdpa_f64(causal, window):
    check_window_against_sdpa(O, causal, window)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_zero_query_closed_form(causal, window):
    check_window_zero_query(O, causal, window)


@pytest.mark.parametrize("causal, window", [(False, (2, 1)), (True, (1, -1)), (False, (0, 0))])
def test_window_finite_differences(causal, window):
    check_finite_differences(O, causal, (5, 4), None, window)


@pytest.mark.parametrize("causal, window", [(False, (3, 2)), (True, (4, -1)), (False, (-1, 1))])
def test_window_row_sampled_forms(causal, window):
    check_window_rows(O, causal, window)


def test_window_unbounded_is_plain_attention():
    # (-1, -1) is full attention and (-1, 0) is causal: the same masks as the
    # causal flag, so the results are identical
    q, k, v, do, cu, _ = rand_problem([9, 5], 4, 2, 8, seed=24)
    for causal in (False, True):
        a = O.forward(q, k, v, cu, cu, 0.5, causal)
        b = O.forward(q, k, v, cu, cu, 0.5, causal, window=(-1, -1))
        np.testing.assert_array_equal(a[0], b[0])
    a = O.forward(q, k, v, cu, cu, 0.5, True)
    b = O.forward(q, k, v, cu, cu, 0.5, False, window=(-1, 0))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_mutation_window_off_by_one_is_caught():
    good = O.visible

    def vis(Lq, Lk, causal, rows=None, window=None):
        m = good(Lq, Lk, causal, rows, window)
        if window is not None and window[0] >= 0:
            m = m & good(Lq, Lk, causal, rows, (window[0] - 1 if window[0] > 0 else 0, window[1]))
        return m
    bad = _mutant(visible=vis)
    assert _fails(check_window_zero_query, bad, False, (3, 1))
    assert _fails(check_window_against_sdpa, bad, False, (3, 1))


def _fails(check, *args):
    try:
        check(*args)
    except AssertionError:
        return True
    return False


def test_mutation_wrong_gqa_grouping_is_caught():
    bad = _mutant(kv_head_of=lambda h, hq, hkv: h % hkv)
    assert _fails(check_gqa_equals_mha, bad, False)
    assert _fails(check_against_sdpa, bad, False)


def test_mutation_strict_causal_mask_is_caught():
    def vis(Lq, Lk, causal, rows=None, window=None):
        i = np.arange(Lq) if rows is None else np.asarray(rows)
        j = np.arange(Lk)
        if not causal:
            return np.ones((i.shape[0], Lk), dtype=bool)
        return j[None, :] < (i[:, None] + (Lk - Lq))
    bad = _mutant(visible=vis)
    assert _fails(check_zero_query_closed_form, bad, True)
    assert _fails(check_hand_worked, bad)


def test_mutation_top_left_causal_alignment_is_caught():
    def vis(Lq, Lk, causal, rows=None, window=None):
        i = np.arange(Lq) if rows is None else np.asarray(rows)
        j = np.arange(Lk)
        if not causal:
            return np.ones((i.shape[0], Lk), dtype=bool)
        return j[None, :] <= i[:, None]
    bad = _mutant(visible=vis)
    assert _fails(check_finite_differences, bad, True, (4, 2), (2, 5)) or _fails(check_empty_rows, bad)


def test_mutation_softmax_without_max_subtraction_in_lse_is_caught():
    def rs(s, vis):
        s_vis = np.where(vis, s, -np.inf)
        any_vis = vis.any(axis=1)
        m = np.where(any_vis, s_vis.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(s_vis - m[:, None]), 0.0)
        z = e.sum(axis=1)
        lse = np.where(any_vis, np.log(np.where(any_vis, z, 1.0)), -np.inf)  # dropped "+ m"
        p = np.where(any_vis[:, None], e / np.where(any_vis, z, 1.0)[:, None], 0.0)
        return p, lse
    bad = _mutant(_row_softmax=rs)
    assert _fails(check_single_key, bad)
    assert _fails(check_against_sdpa, bad, False)


def test_mutation_dropped_delta_term_is_caught():
    src = O.backward.__code__
    # Replace the backward with one that forgets Delta in dS (a dropped term).
    def bwd(q, k, v, cu_q, cu_k, scale, causal, dout, chunk=2048):
        q, k, v, cu_q, cu_k = O._check(q, k, v, cu_q, cu_k)
        dout = np.asarray(dout, dtype=np.float64)
        Tq, Hq, D = q.shape
        Hkv = k.shape[1]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(len(cu_q) - 1):
            cq, Lq = cu_q[b], cu_q[b + 1] - cu_q[b]
            ck, Lk = cu_k[b], cu_k[b + 1] - cu_k[b]
            for h in range(Hq):
                g = O.kv_head_of(h, Hq, Hkv)
                kb, vb = k[ck:ck + Lk, g], v[ck:ck + Lk, g]
                qr, dor = q[cq:cq + Lq, h], dout[cq:cq + Lq, h]
                p, _ = O._row_softmax(scale * qr @ kb.T, O.visible(Lq, Lk, causal))
                ds = p * (dor @ vb.T)
                dq[cq:cq + Lq, h] = scale * ds @ kb
                dk[ck:ck + Lk, g] += scale * ds.T @ qr
                dv[ck:ck + Lk, g] += p.T @ dor
        return dq, dk, dv
    assert src is not None
    bad = _mutant(backward=bwd)
    assert _fails(check_gradient_invariants, bad, False)
    assert _fails(check_hand_worked, bad)


def test_mutation_missing_scale_in_dk_is_caught():
    def bwd(q, k, v, cu_q, cu_k, scale, causal, dout, chunk=2048):
        dq, dk, dv = O.backward(q, k, v, cu_q, cu_k, scale, causal, dout, chunk)
        return dq, dk / scale, dv
    bad = _mutant(backward=bwd)
    assert _fails(check_finite_differences, bad, False)


def test_mutation_transposed_pv_operand_is_caught():
    def fwd(q, k, v, cu_q, cu_k, scale, causal, chunk=2048):
        out, lse = O.forward(q, k, v, cu_q, cu_k, scale, causal, chunk)
        # use V of the wrong KV head (transposed head index) for the output
        out2, _ = O.forward(q, k, v[:, ::-1].copy(), cu_q, cu_k, scale, causal, chunk)
        return out2, lse
    bad = _mutant(forward=fwd)
    assert _fails(check_zero_query_closed_form, bad, False)
