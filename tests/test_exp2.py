"""The forward's FMA-pipe exponential (av_exp2.h), evaluated through the host
export: against numpy's float64 2^x over the whole range the softmax feeds it
(scaled, max-subtracted scores: x <= 8 with the lazy rescale's slack, down to
-inf for masked keys)."""
import ctypes
import os

import numpy as np
import pytest

import exact_attention_varlen_amd._lib as L

FIT_REL = 7.5e-5  # the polynomial's minimax relative error (exp2_fit.py)


def exp2_fma(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    rc = L.lib().attn_varlen_exp2_fma_host(x.ctypes.data_as(ctypes.c_void_p), y.ctypes.data_as(ctypes.c_void_p),
                                           x.size)
    assert rc >= 0
    return y


def test_relative_error_over_the_softmax_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([np.linspace(-125, 8, 2_000_001, dtype=np.float32),
                        rng.uniform(-125, 8, 1_000_000).astype(np.float32),
                        np.arange(-125, 9, dtype=np.float32),                 # integers: f = 0
                        np.arange(-125, 8, dtype=np.float32) + np.float32(0.5),  # ties of rint
                        np.float32([-0.0, 0.0, 1e-30, -1e-30])])
    y = exp2_fma(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    assert rel.max() <= FIT_REL + 4 * 2.0 ** -24, rel.max()
    assert np.all(y > 0)


def test_underflow_and_masked_scores_give_exact_zero():
    x = np.float32([-np.inf, -1e30, -200.0, -126.0, -125.0001])
    assert np.all(exp2_fma(x) == 0.0)
    assert exp2_fma(np.float32([-125.0]))[0] > 0


def test_exponent_assembly_at_the_range_ends():
    # 2^n for every integer n in range comes out within the fit's error of the exact power
    n = np.arange(-125, 9)
    y = exp2_fma(n.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y / np.ldexp(1.0, n) - 1.0) <= FIT_REL)


def test_default_build_uses_the_hardware_exponential():
    # the return value is the build's AV_EXP2_EMU: 0 for the default library
    # (a variant build loaded through ATTN_VARLEN_LIBRARY reports its own K)
    if os.path.basename(L.LIB_PATH) != "libattn_varlen.so":
        pytest.skip("a variant build is loaded")
    x = np.zeros(1, dtype=np.float32)
    y = np.zeros(1, dtype=np.float32)
    assert L.lib().attn_varlen_exp2_fma_host(x.ctypes.data_as(ctypes.c_void_p), y.ctypes.data_as(ctypes.c_void_p),
                                             1) == 0
