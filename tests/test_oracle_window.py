"""Pins for the oracle's sliding-window attention: a scalar loop route,
reduction to causal attention when the window covers everything, the
one-key window, and equality with causal attention on each row's key slice."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import scalar


@pytest.mark.parametrize("nq,nk,w", [(6, 9, 3), (5, 5, 1), (4, 20, 7), (8, 8, 100)])
def test_window_vs_scalar_loops(nq, nk, w):
    rng = np.random.default_rng(nq * 31 + nk + w)
    q, k, v = rng.standard_normal((nq, 8)), rng.standard_normal((nk, 8)), rng.standard_normal((nk, 8))
    sigma = float(np.float32(0.4))
    o, lse = A.attention(q[None, None], k[None, None], v[None, None], 0.4, True, window=w)
    ro, rl = scalar.attention_rows_window(q.tolist(), k.tolist(), v.tolist(), sigma, w)
    assert np.allclose(o[0, 0], np.array(ro), rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], np.array(rl), rtol=0, atol=1e-12)


def test_large_window_is_causal_and_unit_window_copies_v():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((1, 2, 7, 16)), rng.standard_normal((1, 2, 12, 16)), rng.standard_normal((1, 2, 12, 16))
    o1, l1 = A.attention(q, k, v, 0.3, True, window=12)
    o2, l2 = A.attention(q, k, v, 0.3, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, _ = A.attention(q, k, v, 0.3, True, window=1)
    assert np.allclose(o3, v[:, :, 5:12], rtol=0, atol=1e-12)     # row i sees only key i + 5


def test_each_row_is_causal_attention_on_its_slice():
    rng = np.random.default_rng(2)
    nq, nk, w = 10, 30, 6
    q, k, v = rng.standard_normal((1, 1, nq, 8)), rng.standard_normal((1, 1, nk, 8)), rng.standard_normal((1, 1, nk, 8))
    o, lse = A.attention(q, k, v, 0.5, True, window=w)
    for i in range(nq):
        last = i + nk - nq
        sl = slice(last - w + 1, last + 1)
        oi, li = A.attention(q[:, :, i:i + 1], k[:, :, sl], v[:, :, sl], 0.5, False)
        assert np.allclose(o[0, 0, i], oi[0, 0, 0], rtol=0, atol=1e-12)
        assert np.allclose(lse[0, 0, i], li[0, 0, 0], rtol=0, atol=1e-12)
