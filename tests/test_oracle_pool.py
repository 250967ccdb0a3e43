"""The threaded piece-by-piece runner of the oracle (tests/oracle_pool.py) gives
the oracle's own results: same rows, same heads, KV gradients summed over each
group, empty sequences and rows without keys included."""
import numpy as np
import pytest

import oracle.attention as O
import oracle_pool as P
import workloads as W


def problem(seed=3):
    rng = np.random.default_rng(seed)
    lq, lk = [37, 0, 150, 9, 64], [40, 5, 150, 0, 100]
    cu_q, cu_k = W.cu_from_lengths(lq), W.cu_from_lengths(lk)
    Hq, Hkv, D = 6, 2, 16
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    do = rng.standard_normal((cu_q[-1], Hq, D))
    return q, k, v, do, cu_q, cu_k


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (False, (20, 7)), (True, (30, -1))])
def test_pool_matches_the_oracle(causal, window):
    q, k, v, do, cu_q, cu_k = problem()
    o, l = O.forward(q, k, v, cu_q, cu_k, 0.3, causal, window=window)
    po, pl = P.forward(q, k, v, cu_q, cu_k, 0.3, causal, window=window, nthreads=4)
    np.testing.assert_allclose(po, o, rtol=0, atol=1e-13)
    assert np.array_equal(np.isfinite(pl), np.isfinite(l))
    np.testing.assert_allclose(pl[np.isfinite(l)], l[np.isfinite(l)], rtol=0, atol=1e-13)
    dq, dk, dv = O.backward(q, k, v, cu_q, cu_k, 0.3, causal, do, window=window)
    pq, pk, pv = P.backward(q, k, v, cu_q, cu_k, 0.3, causal, do, window=window, nthreads=4)
    for a, b in ((pq, dq), (pk, dk), (pv, dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    keys = np.array([0, 39, 41, 44, 45, 100, 194, 195, 250, 294])
    r, rk, rv = P.backward_dkdv_rows(q, k, v, cu_q, cu_k, 0.3, causal, do, keys, window=window, nthreads=3)
    assert np.array_equal(r, keys)
    np.testing.assert_allclose(rk, dk[keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(rv, dv[keys], rtol=0, atol=1e-12)


def test_pool_chunking_of_long_rows():
    """Long key rows are taken in smaller row chunks (memory); results are unchanged."""
    assert P._chunk(1 << 17) == 256 and P._chunk(100) == 2048 and P._chunk(1 << 30) == 64
