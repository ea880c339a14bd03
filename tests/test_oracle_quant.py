"""Pins for the oracle's quantizers: closed forms, brute force, torch's E4M3
cast, idempotence, losslessness on representable blocks, sign symmetry."""
import numpy as np
import torch

from bit_quantized_attention_online_amd.synth import bf16_bits, bits_to_f32
from oracle import formats, quant, scalar


def _bits(x):
    return bf16_bits(np.asarray(x, dtype=np.float32))


def test_worked_block_by_hand():
    # amax 6.5 -> floor(log2 6.5) = 2 -> X = 0 -> scale byte 127; elements
    # 1.0 -> code 2; -0.3 -> nearest 0.5 -> code 9; 6.5 -> saturates to 6 -> 7
    x = np.zeros(32, dtype=np.float32)
    x[:3] = [1.0, -0.3, 6.5]
    codes, scales = quant.quantize_qk(_bits(x)[None])
    assert scales.tolist() == [[127]]
    assert codes[0, 0] == (2 | (9 << 4)) and codes[0, 1] == 7 and not codes[0, 2:].any()
    # amax 0.02 -> floor(log2) = -6 -> X = -8 -> 0.02 * 256 = 5.12 > 5 -> code 7 (6.0)
    x = np.zeros(32, dtype=np.float32)
    x[5] = 0.02
    codes, scales = quant.quantize_qk(_bits(x)[None])
    assert scales.tolist() == [[127 - 8]] and (codes[0, 2] >> 4) == 7


def test_shared_exponent_vs_stepping():
    rng = np.random.default_rng(0)
    a = np.concatenate([np.ldexp(rng.uniform(1, 2, 200), rng.integers(-140, 128, 200)), [0.0, 2.0 ** -133, 3.0e38]])
    a = bits_to_f32(_bits(a)).astype(np.float64)
    for emax in (2, 8):
        got = quant.shared_exponent(a, emax)
        for ai, gi in zip(a, got):
            want = -127 if ai == 0 else max(-127, min(127, scalar.floor_log2(ai) - emax))
            assert gi == want, (ai, emax)


def test_quantize_qk_vs_brute_force():
    rng = np.random.default_rng(1)
    rows = []
    for e in (-130, -20, -3, 0, 2, 5, 60, 126):
        rows.append(np.ldexp(rng.standard_normal(64), e))
    rows.append(np.zeros(64))
    rows.append(np.r_[np.zeros(63), -1e-3])
    x_bits = _bits(np.array(rows))
    codes, scales = quant.quantize_qk(x_bits)
    xf = bits_to_f32(x_bits).astype(np.float64)
    for r in range(xf.shape[0]):
        for blk in range(2):
            bc, bs = scalar.quantize_block_e2m1([float(v) for v in xf[r, blk * 32:(blk + 1) * 32]])
            assert scales[r, blk] == bs
            packed = [bc[2 * i] | (bc[2 * i + 1] << 4) for i in range(16)]
            assert codes[r, blk * 16:(blk + 1) * 16].tolist() == packed


def test_quantize_qk_exhaustive_bf16_against_brute_force_per_scale_class():
    # Every finite bf16 value x, placed in a block whose amax A is fixed (one
    # scale class per A).  The element code must be the RNE E2M1 code of x/2^X.
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits_to_f32(bits).astype(np.float64)
    fin = np.isfinite(vals)
    for A in (1.0, 6.0, 2.0 ** -126, 3.0 * 2 ** 100):
        sel = bits[fin & (np.abs(vals) <= A)]
        blocks = np.zeros((len(sel), 32), dtype=np.uint16)
        blocks[:, 0] = sel
        blocks[:, 1] = _bits([A])[0]
        codes, scales = quant.quantize_qk(blocks)
        X = int(scales[0, 0]) - 127
        assert (scales == X + 127).all()
        y = bits_to_f32(sel).astype(np.float64) / 2.0 ** X
        # brute force on a strided subset (pure Python is slow), vectorised
        # encoder with torch-free closed form on all
        got = codes[:, 0] & 0xF
        want_all = formats.e2m1_encode(y)
        assert np.array_equal(got, want_all)
        for i in range(0, len(sel), 97):
            yc = np.copysign(min(abs(y[i]), 6.0), y[i])
            assert got[i] == scalar.nearest_code(float(yc), range(16), scalar.e2m1_value)


def test_quantize_v_vs_brute_force_and_torch():
    rng = np.random.default_rng(2)
    v = np.ldexp(rng.standard_normal((3, 20, 32)), rng.integers(-30, 30, (3, 1, 1)))
    v[1, 16:] = 0.0
    v_bits = _bits(v)
    codes, scales = quant.quantize_v(v_bits, tile_rows=8)       # tiles 8, 8, 4 rows
    vf = bits_to_f32(v_bits).astype(np.float64)
    for g in range(3):
        for t, (r0, r1) in enumerate([(0, 8), (8, 16), (16, 20)]):
            flat = [float(x) for x in vf[g, r0:r1].ravel()]
            bc, bs = scalar.quantize_tile_e4m3(flat)
            assert scales[g, t] == bs
            assert codes[g, r0:r1].ravel().tolist() == bc
            y = vf[g, r0:r1] / 2.0 ** (bs - 127)
            ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(ref, codes[g, r0:r1])


def test_idempotent_and_sign_symmetric():
    rng = np.random.default_rng(3)
    x_bits = _bits(rng.standard_normal((16, 128)) * 3)
    c, s = quant.quantize_qk(x_bits)
    deq = quant.dequantize_qk(c, s)
    c2, s2 = quant.quantize_qk(_bits(deq))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    cn, sn = quant.quantize_qk(x_bits ^ np.uint16(0x8000))
    assert np.array_equal(cn, c ^ np.uint8(0x88)) and np.array_equal(sn, s)
    v_bits = _bits(rng.standard_normal((2, 40, 64)))
    vc, vs = quant.quantize_v(v_bits, 16)
    vd = quant.dequantize_v(vc, vs, 16)
    vc2, vs2 = quant.quantize_v(_bits(vd), 16)
    assert np.array_equal(vc, vc2) and np.array_equal(vs, vs2)
    vcn, vsn = quant.quantize_v(v_bits ^ np.uint16(0x8000), 16)
    assert np.array_equal(vcn, vc ^ np.uint8(0x80)) and np.array_equal(vsn, vs)


def test_lossless_on_representable_blocks():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, (8, 128))
    codes[:, ::32] = 7                      # every block holds a +-6 -> X = k
    k = rng.integers(-20, 20, (8, 4))
    x = formats.e2m1_decode(codes) * np.repeat(np.ldexp(1.0, k), 32, axis=1)
    c, s = quant.quantize_qk(_bits(x))
    assert np.array_equal(quant.dequantize_qk(c, s), x)
    vcodes = rng.integers(0, 0x7F, (2, 16, 32)).astype(np.uint8) | (rng.integers(0, 2, (2, 16, 32)) << 7).astype(np.uint8)
    vcodes[:, 0, 0] = 0x7E                  # 448 present -> X = k
    v = formats.e4m3_decode(vcodes) * np.ldexp(1.0, rng.integers(-10, 10, (2, 1, 1)))
    vc, vs = quant.quantize_v(_bits(v), 16)
    assert np.array_equal(quant.dequantize_v(vc, vs, 16), v)
