"""CPU checks of the parity helpers that carry numeric reasoning of their own:
the bf16 spacing used by the output check for sharply peaked attention."""
import numpy as np
import pytest
import torch

from parity import OUT_MAX_ABS, bf16_half_ulp, check_out_rounded


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
