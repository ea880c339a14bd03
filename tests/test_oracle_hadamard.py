"""Pins for the oracle's Hadamard rotation of Q/K rows: the matrix
definition, involution up to d, the float32 butterfly order (a second scalar
route with per-operation float32 rounding), and the invariance of exact
attention under the rotation."""
import numpy as np
import pytest
from scipy.linalg import hadamard

from bit_quantized_attention_online_amd import synth
from oracle import attention as A
from oracle import quant, scalar
from oracle.formats import bf16_bits_to_float64


@pytest.mark.parametrize("d", [32, 64, 128])
def test_matches_the_hadamard_matrix_on_exact_inputs(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-8, 9, size=(5, d)).astype(np.float32)
    y = quant.hadamard_rows_f32(synth.bf16_bits(x))
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ hadamard(d).T)


def test_applied_twice_gives_d_times_x():
    rng = np.random.default_rng(1)
    x = rng.integers(-4, 5, size=(3, 128)).astype(np.float32)
    y = quant.hadamard_rows_f32(synth.bf16_bits(x))
    z = quant.hadamard_rows_f32(synth.bf16_bits(y))     # integers below 2^8 are exact in bf16
    assert np.array_equal(z, 128 * x)


def test_float32_rounding_matches_the_scalar_butterflies():
    rng = np.random.default_rng(2)
    bits = synth.bf16_bits((rng.standard_normal((4, 128)) * np.exp2(rng.integers(-20, 20, (4, 128)))).astype(np.float32))
    y = quant.hadamard_rows_f32(bits)
    for r in range(4):
        ref = scalar.hadamard_row_f32(bf16_bits_to_float64(bits[r]).tolist())
        assert np.array_equal(y[r], np.array(ref, dtype=np.float32))


def test_rotation_leaves_exact_attention_unchanged():
    # (H q).(H k) / d = q.k: exact attention on rotated, unquantized rows equals
    # exact attention on the original rows
    rng = np.random.default_rng(3)
    q = synth.bf16_bits(rng.standard_normal((1, 2, 16, 64)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((1, 2, 40, 64)).astype(np.float32))
    v = rng.standard_normal((1, 2, 40, 64))
    qr = quant.hadamard_rows_f32(q).astype(np.float64)
    kr = quant.hadamard_rows_f32(k).astype(np.float64)
    o1, l1 = A.attention(qr, kr, v, 0.125 / 64, True)
    o2, l2 = A.attention(bf16_bits_to_float64(q), bf16_bits_to_float64(k), v, 0.125, True)
    assert np.allclose(o1, o2, rtol=0, atol=1e-9) and np.allclose(l1, l2, rtol=0, atol=1e-9)


def test_rotation_reduces_error_with_outlier_channels():
    # the point of the rotation: with a few large K channels, quantizing the
    # rotated rows loses less than quantizing the raw rows
    rng = np.random.default_rng(4)
    qf = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    kf = rng.standard_normal((1, 1, 256, 128)).astype(np.float32)
    kf[..., [3, 50, 77, 100]] *= 20.0
    q, k = synth.bf16_bits(qf), synth.bf16_bits(kf)
    v = synth.bf16_bits(rng.standard_normal((1, 1, 256, 128)).astype(np.float32))
    exact, _ = A.attention(bf16_bits_to_float64(q), bf16_bits_to_float64(k), bf16_bits_to_float64(v), 0.088, True)
    plain, _ = A.qk4v8_prefill(q, k, v, 0.088, True, 64)
    rot, _ = A.qk4v8_prefill_hadamard(q, k, v, 0.088, True, 64)
    e_plain = np.linalg.norm(plain - exact) / np.linalg.norm(exact)
    e_rot = np.linalg.norm(rot - exact) / np.linalg.norm(exact)
    assert e_rot < 0.8 * e_plain, (e_rot, e_plain)   # 0.45 vs 0.64 here
