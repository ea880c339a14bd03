"""Pins for the oracle's attention: scalar brute force, torch SDPA in float64
(an independent library routine) on exactly representable inputs, closed
forms and invariants."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from bit_quantized_attention_online_amd.synth import bf16_bits
from oracle import attention, formats, quant, scalar


def _bits(x):
    return bf16_bits(np.asarray(x, dtype=np.float32))


def _rand(shape, seed, scale=1.0):
    return _bits(np.random.default_rng(seed).standard_normal(shape) * scale)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", [
    (1, 1, 1, 7, 7, 32, False), (1, 2, 1, 5, 9, 32, True), (2, 4, 2, 3, 3, 64, True), (1, 2, 2, 1, 6, 32, True)])
def test_prefill_vs_scalar_brute_force(B, Hq, Hkv, Nq, Nk, d, causal):
    q, k, v = _rand((B, Hq, Nq, d), 1, 2), _rand((B, Hkv, Nk, d), 2, 2), _rand((B, Hkv, Nk, d), 3)
    sigma = 1.0 / np.sqrt(d)
    o, lse = attention.qk4v8_prefill(q, k, v, sigma, causal, v_tile_rows=4)
    G = Hq // Hkv
    qf, kf, vf = (formats.bf16_bits_to_float64(t) for t in (q, k, v))
    sig32 = float(np.float32(sigma))
    for b in range(B):
        kq, vq = [], []
        for g in range(Hkv):
            rows = []
            for j in range(Nk):
                blocks = [scalar.quantize_block_e2m1(list(kf[b, g, j, c:c + 32])) for c in range(0, d, 32)]
                rows.append([scalar.e2m1_value(cd) * 2.0 ** (s - 127) for cds, s in blocks for cd in cds])
            kq.append(rows)
            vrows = []
            for t0 in range(0, Nk, 4):
                tile = [float(x) for x in vf[b, g, t0:t0 + 4].ravel()]
                cds, s = scalar.quantize_tile_e4m3(tile)
                vals = [scalar.e4m3_value(c) * 2.0 ** (s - 127) for c in cds]
                vrows += [vals[i:i + d] for i in range(0, len(vals), d)]
            vq.append(vrows)
        for h in range(Hq):
            qrows = []
            for i in range(Nq):
                blocks = [scalar.quantize_block_e2m1(list(qf[b, h, i, c:c + 32])) for c in range(0, d, 32)]
                qrows.append([scalar.e2m1_value(cd) * 2.0 ** (s - 127) for cds, s in blocks for cd in cds])
            so, sl = scalar.attention_rows(qrows, kq[h // G], vq[h // G], sig32, causal)
            np.testing.assert_allclose(o[b, h], np.array(so), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], np.array(sl), rtol=1e-12, atol=1e-12)


def _representable(shape, seed, kind):
    """Values exactly representable after quantization (E2M1 * 2^k blocks with
    a +-6 present, or E4M3 * 2^k tiles with a 448 present)."""
    rng = np.random.default_rng(seed)
    if kind == "e2m1":
        c = rng.integers(0, 16, shape)
        c[..., ::32] = 7 + 8 * rng.integers(0, 2, c[..., ::32].shape)
        x = formats.e2m1_decode(c) * np.ldexp(1.0, rng.integers(-3, 1))
    else:
        c = rng.integers(0, 0x7F, shape) | (rng.integers(0, 2, shape) << 7)
        c[..., ::8, 0] = 0x7E
        x = formats.e4m3_decode(c) * 2.0 ** -8
    return x


@pytest.mark.parametrize("causal,Nq,Nk", [(False, 16, 16), (True, 16, 16), (True, 5, 24)])
def test_exactly_representable_inputs_give_exact_attention(causal, Nq, Nk):
    B, Hq, Hkv, d = 2, 4, 2, 64
    q = _representable((B, Hq, Nq, d), 10, "e2m1")
    k = _representable((B, Hkv, Nk, d), 11, "e2m1")
    v = _representable((B, Hkv, Nk, d), 12, "e4m3")
    o, _ = attention.qk4v8_prefill(_bits(q), _bits(k), _bits(v), 0.125, causal, v_tile_rows=8)
    G = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k, G, axis=1))
    vt = torch.from_numpy(np.repeat(v, G, axis=1))
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=mask, scale=0.125)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_constant_v_returns_v_and_rows_sum_to_one():
    q, k = _rand((1, 2, 9, 32), 20), _rand((1, 1, 9, 32), 21)
    v = np.full((1, 1, 9, 32), _bits([1.375])[0], dtype=np.uint16)
    for causal in (False, True):
        o, _ = attention.qk4v8_prefill(q, k, v, 0.3, causal, v_tile_rows=4)
        np.testing.assert_allclose(o, 1.375, rtol=0, atol=1e-14)
        qh = quant.dequantize_qk(*quant.quantize_qk(q))
        kh = quant.dequantize_qk(*quant.quantize_qk(k))
        p = attention.probabilities(qh, kh, 0.3, causal)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert (p[..., 0, 1:] == 0).all()


def test_causal_row0_dominant_key_permutation_gqa():
    B, Hq, Hkv, N, d = 1, 4, 2, 12, 64
    q, k, v = _rand((B, Hq, N, d), 30), _rand((B, Hkv, N, d), 31), _rand((B, Hkv, N, d), 32)
    o, lse = attention.qk4v8_prefill(q, k, v, 0.125, True, v_tile_rows=4)
    vh = quant.dequantize_v(*quant.quantize_v(v.reshape(B * Hkv, N, d), 4), 4).reshape(B, Hkv, N, d)
    for h in range(Hq):
        np.testing.assert_array_equal(o[0, h, 0], vh[0, h // 2, 0])          # row 0 sees only key 0
    # a dominant score picks out one V row: key 5 = 8 * q row 3 of head 0
    k2 = k.copy()
    k2[0, 0, 5] = _bits(formats.bf16_bits_to_float64(q[0, 0, 3]) * 8)
    o2, _ = attention.qk4v8_prefill(q, k2, v, 1.0, False, v_tile_rows=4)
    np.testing.assert_allclose(o2[0, 0, 3], vh[0, 0, 5], atol=1e-12)
    # non-causal output is invariant to permuting the keys with their values
    perm = np.random.default_rng(33).permutation(N)
    vq = quant.dequantize_v(*quant.quantize_v(v.reshape(B * Hkv, N, d), N), N).reshape(B, Hkv, N, d)
    qh = quant.dequantize_qk(*quant.quantize_qk(q))
    kh = quant.dequantize_qk(*quant.quantize_qk(k))
    oa, la = attention.attention(qh, kh, vq, 0.125, False)
    ob, lb = attention.attention(qh, kh[:, :, perm], vq[:, :, perm], 0.125, False)
    np.testing.assert_allclose(oa, ob, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)
    # identical Q across a GQA group -> identical outputs
    q3 = q.copy()
    q3[0, 1] = q3[0, 0]
    o3, _ = attention.qk4v8_prefill(q3, k, v, 0.125, True, v_tile_rows=4)
    np.testing.assert_array_equal(o3[0, 0], o3[0, 1])
    # lse is the log-sum-exp of the visible scores
    s = float(np.float32(0.125)) * (qh[0, 0] @ kh[0, 0].T)
    for i in range(N):
        assert abs(la[0, 0, i] - logsumexp(s[i])) < 1e-12


def test_rows_subset_matches_full():
    q, k, v = _rand((1, 2, 20, 32), 40), _rand((1, 1, 28, 32), 41), _rand((1, 1, 28, 32), 42)
    o, lse = attention.qk4v8_prefill(q, k, v, 0.2, True, v_tile_rows=8)
    rows = np.array([0, 7, 19])
    o2, lse2 = attention.qk4v8_prefill(q[:, :, rows], k, v, 0.2, True, v_tile_rows=8, rows=(rows, 20))
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


def test_decode_equals_prefill_rows():
    # decode over a quantized cache of length n equals the last q_len rows of
    # a bottom-right causal prefill with the same V tile size
    B, Hq, Hkv, d, q_len, n, cap, R = 2, 4, 2, 64, 3, 37, 48, 16
    rng = np.random.default_rng(50)
    k = _bits(rng.standard_normal((B, Hkv, cap, d)))
    v = _bits(rng.standard_normal((B, Hkv, cap, d)))
    q = _bits(rng.standard_normal((B, q_len, Hq, d)))
    lens = np.array([n, n - 5])
    for b in range(B):          # cache rows past the length are empty, so the
        v[b, :, lens[b]:] = 0   # partial last V tile has the prefill's scale
    kc, ks = quant.quantize_qk(k)
    vc, vs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    vc, vs = vc.reshape(B, Hkv, cap, d), vs.reshape(B, Hkv, -1)
    o, lse = attention.qk4v8_decode(q, kc, ks, vc, vs, lens, R, 0.125)
    for b in range(B):
        nb = lens[b]
        po, pl = attention.qk4v8_prefill(q[b:b + 1].transpose(0, 2, 1, 3), k[b:b + 1, :, :nb], v[b:b + 1, :, :nb],
                                         0.125, True, R)
        np.testing.assert_allclose(o[b], po[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(lse[b], pl[0].T, atol=1e-12)
