"""CPU checks of the parity helpers that carry numeric reasoning of their own:
the bf16 spacing used by the output check for sharply peaked attention."""
import numpy as np
import pytest
import torch

from parity import OUT_MAX_ABS, bf16_half_ulp, check_out, check_out_rounded


def test_bf16_half_ulp_values():
    # bf16 keeps 8 significant bits: spacing 2^(e-7) on [2^e, 2^(e+1))
    assert bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8
    assert bf16_half_ulp(np.array([3.99]))[0] == 2.0 ** -7
    assert bf16_half_ulp(np.array([4.0]))[0] == 2.0 ** -6
    assert bf16_half_ulp(np.array([-6.5]))[0] == 2.0 ** -6
    assert bf16_half_ulp(np.array([0.1]))[0] == 2.0 ** -12


def test_bf16_half_ulp_bounds_torch_rounding():
    rng = np.random.default_rng(0)
    # from float32, as the kernels round their fp32 results (float64 -> bf16
    # in torch goes through float32, a second rounding)
    x = (rng.standard_normal(200_000) * 3.0).astype(np.float32)
    r = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    ratio = np.abs(r - x.astype(np.float64)) / bf16_half_ulp(x)
    assert ratio.max() <= 1.0
    assert ratio.max() > 0.99  # the bound is attained, not loose


def test_check_out_rounded_accepts_rounding_and_rejects_more():
    rng = np.random.default_rng(1)
    ref = rng.uniform(-6.0, 6.0, size=(64, 4, 8))
    ref[0, 0, 0] = 4.0 + 2.0 ** -6 * 0.999  # just below a midpoint of the spacing at 4
    best = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert np.abs(best - ref).max() > OUT_MAX_ABS  # the plain bound cannot hold here
    check_out_rounded(best, ref)
    worse = best.copy()
    worse[3, 2, 1] += 0.04
    with pytest.raises(AssertionError):
        check_out_rounded(worse, ref)


def test_gradient_column_check_catches_a_few_bad_columns():
    """Errors confined to 4 of 256 head-dim columns (the footprint of a stale
    accumulator register) stay under the whole-tensor bound but fail the
    per-column one; spread-out rounding-sized errors pass both."""
    import pytest
    from parity import GRAD_REL_FRO, check_grad, rel_fro

    rng = np.random.default_rng(0)
    ref = rng.standard_normal((300, 2, 256))
    noisy = ref * (1 + 3e-3 * rng.standard_normal(ref.shape))
    check_grad(noisy, ref, "spread")
    bad = noisy.copy()
    bad[..., [250, 251, 254, 255]] *= 1.15
    assert rel_fro(bad, ref) <= GRAD_REL_FRO
    with pytest.raises(AssertionError, match="head-dim column 25"):
        check_grad(bad, ref, "columns")
    # an exactly-zero tensor must come out zero up to rounding
    with pytest.raises(AssertionError, match="exactly zero"):
        check_grad(np.full((3, 1, 64), 1e-3), np.zeros((3, 1, 64)), "zero tensor")
    check_grad(np.full((3, 1, 64), 1e-7), np.zeros((3, 1, 64)), "zero tensor, rounding only")


@pytest.mark.parametrize("causal,window", [(True, (9, -1)), (False, (6, 11)), (True, (0, -1))])
def test_band_subsequence_gives_the_full_problems_rows(causal, window):
    # the oracle on the sub-sequence against the oracle on the whole sequence
    import oracle.attention as O

    from parity import band_subsequence

    rng = np.random.default_rng(3)
    L, Hq, Hkv, D, scale = 90, 4, 2, 8, 0.4
    q, dout = rng.standard_normal((2, L, Hq, D))
    k, v = rng.standard_normal((2, L, Hkv, D))
    cu = [0, L]
    o, lse = O.forward(q, k, v, cu, cu, scale, causal, window=window)
    dq, dk, dv = O.backward(q, k, v, cu, cu, scale, causal, dout, window=window)
    right = 0 if causal else window[1]
    for s, n in [(0, 10), (37, 12), (80, 10), (0, 90)]:
        a, e = band_subsequence(L, s, n, window[0], right)
        cs = [0, e - a]
        o2, lse2 = O.forward(q[a:e], k[a:e], v[a:e], cs, cs, scale, causal, window=window)
        dq2, dk2, dv2 = O.backward(q[a:e], k[a:e], v[a:e], cs, cs, scale, causal, dout[a:e], window=window)
        r = slice(s - a, s - a + n)
        np.testing.assert_allclose(o2[r], o[s:s + n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2[:, r], lse[:, s:s + n], rtol=0, atol=1e-12)
        for x2, x in ((dq2, dq), (dk2, dk), (dv2, dv)):
            np.testing.assert_allclose(x2[r], x[s:s + n], rtol=0, atol=1e-12)
        if n < L and a > 0:
            # a narrower sub-sequence is not enough: the first compared rows lose keys
            a3 = a + 1
            cs3 = [0, e - a3]
            o3, _ = O.forward(q[a3:e], k[a3:e], v[a3:e], cs3, cs3, scale, causal, window=window)
            dq3, dk3, _ = O.backward(q[a3:e], k[a3:e], v[a3:e], cs3, cs3, scale, causal, dout[a3:e], window=window)
            r3 = slice(s - a3, s - a3 + n)
            assert (np.abs(o3[r3] - o[s:s + n]).max() > 1e-9 or np.abs(dk3[r3] - dk[s:s + n]).max() > 1e-9
                    or np.abs(dq3[r3] - dq[s:s + n]).max() > 1e-9)


def test_check_out_allows_bf16_rounding_only_where_it_exceeds_the_bound():
    rng = np.random.default_rng(4)
    ref = rng.uniform(-3.5, 3.5, size=(32, 4, 8))
    ref[1, 2, 3] = 4.0 + 2.0 ** -6 * 0.999  # rounds to 4: an error of almost 2^-6 > 1e-2
    best = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    check_out(best, ref)  # the correctly rounded result passes
    half = 2.0 ** -6  # half the bf16 spacing on [4, 8)
    near = best.copy()
    near[1, 2, 3] = ref[1, 2, 3] - (half + 0.009)  # within 1e-2 beyond the rounding where |O| >= 4
    check_out(near, ref)
    bad = best.copy()
    bad[1, 2, 3] = ref[1, 2, 3] - (half + 0.012)  # beyond it
    with pytest.raises(AssertionError):
        check_out(bad, ref)
    bad = best.copy()
    bad[5, 1, 0] = ref[5, 1, 0] + 0.0105  # past 1e-2 where |O| < 4: no allowance there
    with pytest.raises(AssertionError):
        check_out(bad, ref)
