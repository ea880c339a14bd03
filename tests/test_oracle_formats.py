"""Pins for the oracle's element formats: spec tables, torch's E4M3FN cast
(an independent library routine), and the pure-Python brute force."""
import os

import numpy as np
import pytest
import torch

from oracle import formats, scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e2m1_table_matches_spec():
    for code, val in _rows("e2m1_values.txt"):
        got = formats.e2m1_decode(int(code))
        assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_points_match_spec():
    for code, val in _rows("e4m3fn_points.txt"):
        got = formats.e4m3_decode(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def _all_finite_bf16_as_float64():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32).astype(np.float64)
    return f[np.isfinite(f)]


def test_e4m3_encode_vs_torch_every_bf16_in_range():
    # Every finite bf16 value with |y| <= 448, plus the E4M3 midpoints (which
    # bf16 cannot all hold) - torch's cast is RNE and agrees below 464.
    y = _all_finite_bf16_as_float64()
    y = y[np.abs(y) <= 448.0]
    mags = formats.E4M3_MAGNITUDES
    mids = (mags[1:] + mags[:-1]) / 2
    y = np.concatenate([y, mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.e4m3_encode(y)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    y = np.array([448.0, 460.0, 463.9, 464.0, 500.0, 1e30, -1e30])
    assert list(formats.e4m3_encode(y)) == [0x7E] * 5 + [0x7E, 0xFE]


def test_rne_points():
    for fmt, x, code in _rows("rne_points.txt"):
        enc = formats.e2m1_encode if fmt == "e2m1" else formats.e4m3_encode
        assert int(enc(np.array([float(x)]))[0]) == int(code, 0), (fmt, x)


def test_e2m1_encode_vs_brute_force_grid():
    y = np.concatenate([np.arange(-8 * 64, 8 * 64 + 1) / 64.0, [-0.0, 0.0, 1e-30, -1e-30]])
    got = formats.e2m1_encode(y)
    for yi, gi in zip(y, got):
        yc = np.copysign(min(abs(yi), 6.0), yi)
        assert gi == scalar.nearest_code(float(yc), range(16), scalar.e2m1_value), yi


def test_e4m3_encode_vs_brute_force_sample():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.uniform(-448, 448, 300), np.ldexp(rng.uniform(-1, 1, 300), rng.integers(-14, 9, 300)),
                        formats.E4M3_MAGNITUDES[:20] * 1.5])
    got = formats.e4m3_encode(y)
    for yi, gi in zip(y, got):
        assert gi == scalar.nearest_code(float(yi), range(256), scalar.e4m3_value), yi


def test_decode_encode_roundtrip():
    c4 = np.arange(16, dtype=np.uint8)
    assert np.array_equal(formats.e2m1_encode(formats.e2m1_decode(c4)), c4)
    c8 = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(formats.e4m3_encode(formats.e4m3_decode(c8)), c8)


def test_bf16_decode_exact():
    assert formats.bf16_bits_to_float64(np.array([0x3F80, 0xC000, 0x0001, 0x8000])).tolist() == \
        [1.0, -2.0, 2.0 ** -133, -0.0]
