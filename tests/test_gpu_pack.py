"""The prefill's own K/V quantization, bit for bit.

qk4v8_prefill_pack_kv writes MXFP4 K and per-tile FP8 V into the workspace as
one record per (batch x KV head, 128-key tile), in the order the attention
kernel's matrix instructions consume them.  This test reads the workspace
back, undoes that layout on the host and compares every code and scale with
the oracle's quantizers (``oracle.quant``), for the fused V path (V tiles of
at most 128 rows, whose scales the pack workgroup computes itself) and the
separate scale pass (256-row tiles), with and without the Hadamard rotation
of K, on ragged key counts and strided inputs.

Record layout (head_dim d, NS = d / 64 contraction steps):
  K codes  [kb 4][step NS][lane 64][16 B]   at 0; lane = rho + 32 * (g % 2)
           holds 32-element block g = 2 * step + lane // 32 of key
           block_key(kb, rho), in the row-major nibble order of quantize_qk
  K scales [lane 64][kb * NS + step]        at 4 * NS * 1024
  V scales u32, byte b = E8M0 of the V tile holding key 32 b (the last key's
           tile past the sequence)          at 4 * NS * 1024 + 512
  V codes  [db d/32][s2 2][half 2][lane 64][16 keys] at 4 * NS * 1024 + 1024:
           column 32 db + lane % 32, keys 64 s2 + 32 half + 16 (lane // 32) ..
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import quant
from tests._util import to_dev

pytestmark = pytest.mark.gpu


def block_key(kb, rho):
    return 32 * kb + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3)


def unpack_records(ws, bk, seq_k, d, bf16_v=False):
    """Workspace bytes -> (k_codes [bk, T*128, d/2], k_scales [bk, T*128, d/32],
    v_codes [bk, T*128, d] (bf16_v: V values as bf16 bits, uint16), v_scale_words
    [bk, T, 4])."""
    NS = d // 64
    K, SC = 4 * NS * 1024, 1024
    REC = K + SC + 128 * d * (2 if bf16_v else 1)
    T = -(-seq_k // 128)
    rec = ws[:bk * T * REC].reshape(bk, T, REC)
    kc = np.zeros((bk, T, 128, d // 2), np.uint8)
    ks = np.zeros((bk, T, 128, d // 32), np.uint8)
    for kb in range(4):
        for step in range(NS):
            for lane in range(64):
                rho, g = lane % 32, 2 * step + lane // 32
                kk = block_key(kb, rho)
                off = (kb * NS + step) * 1024 + lane * 16
                kc[:, :, kk, 16 * g:16 * g + 16] = rec[:, :, off:off + 16]
                ks[:, :, kk, g] = rec[:, :, K + lane * 4 * NS + kb * NS + step]
    if bf16_v:
        # [db][st][lane][8 bf16]: column 32 db + lane % 32, keys
        # 32 (st // 2) + 16 (lane // 32) + 8 (st % 2) .. +7
        vb = np.zeros((bk, T, 128, d), np.uint16)
        words = rec[:, :, K + SC:].copy().view(np.uint16).reshape(bk, T, d * 16, 8)
        for o in range(d * 16):
            lane, st, db = o & 63, (o >> 6) & 7, o >> 9
            col, k0 = db * 32 + (lane & 31), 32 * (st >> 1) + 16 * (lane >> 5) + 8 * (st & 1)
            vb[:, :, k0:k0 + 8, col] = words[:, :, o]
        vsw = rec[:, :, K + 512:K + 516]
        return kc.reshape(bk, T * 128, -1), ks.reshape(bk, T * 128, -1), vb.reshape(bk, T * 128, d), vsw
    vc = np.zeros((bk, T, 128, d), np.uint8)
    for o in range(d * 8):
        lane, half, s2, db = o & 63, (o >> 6) & 1, (o >> 7) & 1, o >> 8
        col, k0 = db * 32 + (lane & 31), 64 * s2 + 32 * half + 16 * (lane >> 5)
        vc[:, :, k0:k0 + 16, col] = rec[:, :, K + SC + 16 * o:K + SC + 16 * o + 16]
    vsw = rec[:, :, K + 512:K + 516]
    return kc.reshape(bk, T * 128, -1), ks.reshape(bk, T * 128, -1), vc.reshape(bk, T * 128, d), vsw


CASES = [
    # B, Hkv, seq_k, d, R, hadamard
    (2, 2, 300, 128, 64, False),
    (1, 3, 129, 128, 32, False),
    (2, 1, 1000, 128, 128, False),
    (1, 2, 700, 128, 256, False),
    (2, 2, 200, 64, 64, False),
    (1, 1, 513, 64, 256, False),
    (2, 2, 300, 128, 64, True),
    (1, 2, 257, 64, 32, True),
    (1, 1, 600, 128, 256, True),
]
# (B, Hkv, seq_k, d, R, hadamard) of the bf16-V records (QK4V8_P_BF16)
BF16_CASES = [(2, 2, 300, 128, 64, False), (1, 2, 700, 128, 256, False), (1, 3, 129, 64, 32, True)]


def _pack_inputs(B, Hkv, seq_k, d, R, had):
    rng = np.random.default_rng(seq_k * 7 + d + R + int(had))
    k = rng.standard_normal((B, Hkv, seq_k, d)).astype(np.float32)
    k[..., rng.choice(d, 3, replace=False)] *= 20.0
    k *= np.exp2(rng.integers(-6, 6, (B, Hkv, seq_k, 1))).astype(np.float32)
    v = (rng.standard_normal((B, Hkv, seq_k, d))
         * np.exp2(rng.integers(-8, 8, (B, Hkv, seq_k // 16 + 1, 1)).repeat(16, axis=2)[:, :, :seq_k])
         ).astype(np.float32)
    return synth.bf16_bits(k), synth.bf16_bits(v)


@pytest.mark.parametrize("B,Hkv,seq_k,d,R,had", BF16_CASES)
def test_pack_kv_bf16_values_are_the_fp8_quantization(gpu, B, Hkv, seq_k, d, R, had):
    """bf16 mode: the records' V values are exactly the E4M3 codes times the
    tile scale of the oracle's FP8 quantization, and the K codes are bit-exact."""
    from bit_quantized_attention_online_amd import ops
    kb, vb = _pack_inputs(B, Hkv, seq_k, d, R, had)
    print(f"[case] pack_kv bf16 V B{B} Hkv{Hkv} seq_k{seq_k} d{d} R{R} hadamard={had}", flush=True)
    q = torch.zeros((B, Hkv, 1, d), dtype=torch.bfloat16, device="cuda")
    pp = ops.PackedPrefill(q, to_dev(kb), to_dev(vb), causal=False, v_tile_rows=R, hadamard=had, p_mode=3)
    pp.workspace.fill_(0xA5)
    pp.pack()
    torch.cuda.synchronize()
    bk = B * Hkv
    kc, ks, vbits, _ = unpack_records(pp.workspace.cpu().numpy(), bk, seq_k, d, bf16_v=True)
    rkc, rks = (quant.quantize_qk_hadamard(kb) if had else quant.quantize_qk(kb))
    rvc, rvs = quant.quantize_v(vb.reshape(bk, seq_k, d), R)
    vhat = quant.dequantize_v(rvc, rvs, R).astype(np.float32)          # exact in float32
    vhat_bits = vhat.view(np.uint32)
    assert not (vhat_bits & 0xFFFF).any()                               # and in bf16
    assert np.array_equal(kc[:, :seq_k], rkc.reshape(bk, seq_k, -1))
    assert np.array_equal(ks[:, :seq_k], rks.reshape(bk, seq_k, -1))
    assert np.array_equal(vbits[:, :seq_k], (vhat_bits >> 16).astype(np.uint16))
    assert not vbits[:, seq_k:].any()


@pytest.mark.parametrize("B,Hkv,seq_k,d,R,had", CASES)
def test_pack_kv_codes_are_bit_exact(gpu, B, Hkv, seq_k, d, R, had):
    from bit_quantized_attention_online_amd import ops
    # K with outlier channels and a wide spread of row scales; V with tiles of
    # very different magnitudes (so neighbouring V tiles get different scales)
    kb, vb = _pack_inputs(B, Hkv, seq_k, d, R, had)
    print(f"[case] pack_kv B{B} Hkv{Hkv} seq_k{seq_k} d{d} R{R} hadamard={had}", flush=True)
    # K stored token-major ([B, N, H, d] viewed as [B, H, N, d]): strided rows
    kd = to_dev(np.ascontiguousarray(kb.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    vd = to_dev(vb)
    q = torch.zeros((B, Hkv, 1, d), dtype=torch.bfloat16, device="cuda")
    pp = ops.PackedPrefill(q, kd, vd, causal=False, v_tile_rows=R, hadamard=had, p_mode=ops.P_FP8_TWO_TERM)
    pp.workspace.fill_(0xA5)              # bytes the pack must overwrite
    pp.pack()
    torch.cuda.synchronize()
    ws = pp.workspace.cpu().numpy()
    bk = B * Hkv
    kc, ks, vc, vsw = unpack_records(ws, bk, seq_k, d)
    rkc, rks = (quant.quantize_qk_hadamard(kb) if had else quant.quantize_qk(kb))
    rvc, rvs = quant.quantize_v(vb.reshape(bk, seq_k, d), R)
    assert np.array_equal(kc[:, :seq_k], rkc.reshape(bk, seq_k, -1))
    assert np.array_equal(ks[:, :seq_k], rks.reshape(bk, seq_k, -1))
    assert np.array_equal(vc[:, :seq_k], rvc)
    # padding keys of the last tile: zero codes, so they add nothing
    assert not kc[:, seq_k:].any() and not vc[:, seq_k:].any()
    # the V scale of each 32-key group (the last key's tile past the sequence)
    T = -(-seq_k // 128)
    for t in range(T):
        for b in range(4):
            j = min(t * 128 + 32 * b, seq_k - 1)
            assert np.array_equal(vsw[:, t, b], rvs[:, j // R]), (t, b)
    if R > 128:
        # the separate scale pass keeps the per-tile scales after the records
        NS = d // 64
        rec_bytes = bk * T * (4 * NS * 1024 + 1024 + 128 * d)
        off = -(-rec_bytes // 256) * 256
        nvt = -(-seq_k // R)
        assert np.array_equal(ws[off:off + bk * nvt].reshape(bk, nvt), rvs)
