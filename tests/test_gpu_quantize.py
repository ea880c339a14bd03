"""GPU quantizers vs the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import quant
from tests._util import to_dev

pytestmark = pytest.mark.gpu


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = synth.bits_to_f32(bits)
    return bits[np.isfinite(vals)], vals[np.isfinite(vals)]


def test_quantize_qk_exhaustive_bf16(gpu):
    from bit_quantized_attention_online_amd import ops
    bits, vals = _all_finite_bf16()
    for A in (1.0, 6.0, 2.0 ** -126, 2.0 ** -130, 3.0 * 2 ** 100, 2.0 ** 127):
        a_bits = synth.bf16_bits(np.array([A], dtype=np.float32))[0]
        sel = bits[np.abs(vals) <= synth.bits_to_f32(np.array([a_bits]))[0]]
        blocks = np.zeros((len(sel), 32), dtype=np.uint16)
        blocks[:, 0] = sel
        blocks[:, 17] = a_bits
        c, s = ops.quantize_qk(to_dev(blocks))
        torch.cuda.synchronize()
        rc, rs = quant.quantize_qk(blocks)
        assert np.array_equal(c.cpu().numpy(), rc), A
        assert np.array_equal(s.cpu().numpy(), rs), A


@pytest.mark.parametrize("rows,d,ld", [(1, 32, 32), (37, 64, 64), (1000, 128, 128), (300, 128, 136),
                                       (5, 1024, 1024), (129, 96, 104)])
def test_quantize_qk_random_shapes(gpu, rows, d, ld):
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(rows * d)
    x = synth.bf16_bits((rng.standard_normal((rows, ld)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32))
    x[rows // 2, :] = 0
    xd = to_dev(x)[:, :d]
    c, s = ops.quantize_qk(xd)
    rc, rs = quant.quantize_qk(x[:, :d])
    assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)


def test_quantize_qk_empty(gpu):
    from bit_quantized_attention_online_amd import ops
    c, s = ops.quantize_qk(torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"))
    assert c.shape == (0, 64) and s.shape == (0, 4)


@pytest.mark.parametrize("g,n,d,R", [(1, 256, 64, 64), (3, 1000, 128, 256), (2, 77, 128, 32), (4, 300, 8, 128),
                                     (2, 513, 512, 256), (5, 64, 128, 64), (1, 1, 128, 256)])
def test_quantize_v_random_shapes(gpu, g, n, d, R):
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(g * n * d + R)
    v = synth.bf16_bits((rng.standard_normal((g, n, d)) * np.exp2(rng.integers(-30, 30, (g, 1, 1)))).astype(np.float32))
    v[0, : min(n, R)] = 0          # an all-zero tile
    c, s = ops.quantize_v(to_dev(v), R)
    rc, rs = quant.quantize_v(v, R)
    assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)


def test_quantize_v_exhaustive_bf16(gpu):
    from bit_quantized_attention_online_amd import ops
    bits, vals = _all_finite_bf16()
    for A in (1.0, 448.0, 2.0 ** -120, 2.0 ** 127):
        a_bits = synth.bf16_bits(np.array([A], dtype=np.float32))[0]
        sel = bits[np.abs(vals) <= synth.bits_to_f32(np.array([a_bits]))[0]]
        # tiles of 32 rows x 8 columns: element 0 of every tile carries the
        # amax, the other 255 slots hold the swept values
        nt = -(-len(sel) // 255)
        flat = np.zeros((nt, 256), dtype=np.uint16)
        flat[:, 0] = a_bits
        body = np.zeros(nt * 255, dtype=np.uint16)
        body[: len(sel)] = sel
        flat[:, 1:] = body.reshape(nt, 255)
        vv = flat.reshape(1, nt * 32, 8)
        c, s = ops.quantize_v(to_dev(vv), 32)
        rc, rs = quant.quantize_v(vv, 32)
        assert np.array_equal(s.cpu().numpy(), rs), A
        assert np.array_equal(c.cpu().numpy(), rc), A


def test_quantize_strided_views(gpu):
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(9)
    x = synth.bf16_bits(rng.standard_normal((2, 50, 4, 128)).astype(np.float32))   # [B, N, H, d]
    xd = to_dev(x)
    v_view = xd.permute(0, 2, 1, 3)[1]        # [H, N, d] with row stride 4*128
    c, s = ops.quantize_v(v_view, 64)
    rc, rs = quant.quantize_v(np.ascontiguousarray(x.transpose(0, 2, 1, 3)[1]), 64)
    assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)


def test_prepared_quantizers_match_the_plain_calls(gpu):
    """PreparedQuantizeQK / PreparedQuantizeV (arguments marshalled once, as
    the bench times them) write the same bytes as quantize_qk / quantize_v."""
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(123)
    x = synth.bf16_bits(rng.standard_normal((3, 5, 300, 96)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((6, 700, 128)).astype(np.float32))
    xd, vd = to_dev(x), to_dev(v)
    print("[case] prepared quantizers", flush=True)
    c0, s0 = ops.quantize_qk(xd)
    pq = ops.PreparedQuantizeQK(xd)
    c1, s1 = pq()
    c2, s2 = pq()        # a second call on the same prepared arguments
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(c1, c2) and torch.equal(s1, s2)
    for R in (64, 256):
        c0, s0 = ops.quantize_v(vd, R)
        c1, s1 = ops.PreparedQuantizeV(vd, R)()
        torch.cuda.synchronize()
        assert torch.equal(c0, c1) and torch.equal(s0, s1)
