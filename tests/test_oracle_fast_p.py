"""Pins for the oracle's single-term FP8 probability attention
(``attention.attention_fast_p``): an independent scalar route, weights that are
exact powers of two (then it equals exact attention), invariances, and the
E4M3 error bound against exact attention."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import scalar


@pytest.mark.parametrize("nq,nk,causal", [(5, 9, False), (4, 7, True), (3, 300, True), (2, 260, False)])
def test_fast_p_vs_scalar_brute_force(nq, nk, causal):
    rng = np.random.default_rng(nq * 100 + nk)
    d = 8
    q = rng.standard_normal((nq, d)) * 2.0
    k = rng.standard_normal((nk, d))
    v = rng.standard_normal((nk, d))
    sigma = float(np.float32(0.7))
    o, lse = A.attention_fast_p(q[None, None], k[None, None], v[None, None], 0.7, causal)
    ro, rl = scalar.attention_rows_fast_p(q.tolist(), k.tolist(), v.tolist(), sigma, causal)
    assert np.allclose(o[0, 0], np.array(ro), rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], np.array(rl), rtol=0, atol=1e-12)


def test_power_of_two_weights_give_exact_attention():
    # one-hot keys and log2-domain scores that are integers: every weight is a
    # power of two within E4M3's range, so the rounding is exact
    rng = np.random.default_rng(1)
    nk, nq = 20, 6
    k = np.eye(nk)
    n = rng.integers(-6, 1, size=(nq, nk)).astype(np.float64)
    q = n * math.log(2.0)
    v = rng.standard_normal((nk, nk))
    o, lse = A.attention_fast_p(q[None, None], k[None, None], v[None, None], 1.0, False)
    ro, rl = A.attention(q[None, None], k[None, None], v[None, None], 1.0, False)
    assert np.allclose(o, ro, rtol=0, atol=1e-12)
    assert np.allclose(lse, rl, rtol=0, atol=1e-12)


def test_constant_v_and_within_block_permutation():
    rng = np.random.default_rng(2)
    nk, d = 256, 16
    q = rng.standard_normal((1, 1, 3, d))
    k = rng.standard_normal((1, 1, nk, d))
    v = np.tile(rng.standard_normal(d), (nk, 1))[None, None]
    o, _ = A.attention_fast_p(q, k, v, 0.3, False)
    assert np.allclose(o, v[:, :, :3], rtol=0, atol=1e-12)
    # permuting keys inside each aligned 32-key block leaves the result unchanged
    v = rng.standard_normal((1, 1, nk, d))
    perm = np.concatenate([32 * b + rng.permutation(32) for b in range(nk // 32)])
    o1, l1 = A.attention_fast_p(q, k, v, 0.3, False)
    o2, l2 = A.attention_fast_p(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_range_exponent_is_per_32_key_block():
    # two 32-key blocks whose base-2 scores are 0 and -15.3: with one range
    # exponent per 32 keys the small block's weights keep 3 mantissa bits
    # (X = floor(-15.3) - 7 = -23, 2^(-15.3 + 23) = 207.9 -> E4M3 208), while a
    # range shared with the large block (X = -7) would put them in E4M3's
    # subnormals, 2^-8.3 -> 2 * 2^-9, an error of 23%.  Hand-worked values.
    from oracle.formats import e4m3_decode, e4m3_encode
    nk = 64
    k = np.zeros((nk, 2))
    k[32:, 0] = -15.3
    q = np.array([[math.log(2.0), 0.0]])   # t = s * log2(e) = k[:, 0]
    v = np.zeros((nk, 2))
    v[:32, 0] = 1.0
    v[32:, 1] = 1.0
    o, _ = A.attention_fast_p(q[None, None], k[None, None], v[None, None], 1.0, False)
    w1q = float(e4m3_decode(e4m3_encode(np.array([2.0 ** (-15.3 + 23)])))[0]) * 2.0 ** -23
    assert w1q == 208 * 2.0 ** -23
    want = np.array([32.0, 32 * w1q]) / (32 + 32 * w1q)
    assert np.allclose(o[0, 0, 0], want, rtol=0, atol=1e-15)
    shared = 2 * 2.0 ** -9 * 2.0 ** -7        # the same weight on a 64-key shared range
    assert abs(shared / 2.0 ** -15.3 - 1) > 0.2 and abs(w1q / 2.0 ** -15.3 - 1) <= 2.0 ** -4
