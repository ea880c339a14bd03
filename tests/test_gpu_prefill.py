"""GPU prefill attention vs the fp64 oracle (relative L2 <= 5e-3, max abs <= 2e-2)."""
import math

import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import attention as oatt
from tests._util import assert_attn_close, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed, k_scale=1.0):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits(rng.standard_normal((B, Hq, Nq, d)).astype(np.float32))
    k = synth.bf16_bits((rng.standard_normal((B, Hkv, Nk, d)) * k_scale).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, Nk, d)).astype(np.float32))
    return q, k, v


def _run(q, k, v, causal, R, scale=None, lse=True, p_mode=0):
    from bit_quantized_attention_online_amd import ops
    d = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    print(f"[case] prefill q{q.shape} k{k.shape} causal={causal} R={R} p_mode={p_mode}", flush=True)
    o, l = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal, softmax_scale=scale, v_tile_rows=R,
                            return_lse=True, p_mode=p_mode)
    torch.cuda.synchronize()
    ro, rl = oatt.qk4v8_prefill(q, k, v, scale, causal, R)
    return from_dev_bf16(o), l.cpu().numpy().astype(np.float64), ro, rl


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, R
    (1, 1, 1, 256, 256, 64, False, 64),       # the tiny full-attention workload
    (2, 4, 2, 300, 300, 128, True, 64),       # ragged tail, GQA 2
    (1, 8, 1, 77, 333, 128, True, 32),        # Nq < Nk, bottom-right, GQA 8
    (1, 2, 2, 1, 1, 64, True, 64),            # one token
    (3, 6, 3, 129, 129, 64, False, 128),
    (1, 4, 4, 513, 700, 128, False, 256),
    (1, 16, 2, 260, 260, 128, True, 64),      # GQA 8 with several head groups
]


# the probability formats of the default bar (5e-3 relative L2): two-term FP8
# and bf16 (QK4V8_P_FP8_TWO_TERM, QK4V8_P_BF16)
P_MODES = [2, 3]


@pytest.mark.parametrize("p_mode", P_MODES)
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,R", CASES)
def test_prefill_parity(gpu, B, Hq, Hkv, Nq, Nk, d, causal, R, p_mode):
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed=B * 1000 + Nq + Nk + d)
    o, l, ro, rl = _run(q, k, v, causal, R, p_mode=p_mode)
    assert_attn_close(o, ro, f"prefill {B},{Hq},{Hkv},{Nq},{Nk},{d},{causal},{R} p_mode={p_mode}")
    # normalizer = sum of the quantized weights (two-term FP8: rel. error <= 2^-8 each; bf16: <= 2^-9)
    assert np.abs(l - rl).max() < 5e-3


def test_prefill_tiny_workload(gpu):
    w = synth.WORKLOADS[1]
    q, k, v = synth.prefill_inputs(1)
    o, l, ro, rl = _run(q, k, v, w["causal"], w["v_tile_rows"], scale=1.0 / math.sqrt(w["d"]))
    assert_attn_close(o, ro, "workload 1 (B1 H1 N256 d64)")


def test_prefill_outlier_channels_small(gpu):
    # the 4-outlier-channel K structure of the causal GQA workload, at a small size
    w = dict(synth.WORKLOADS[2], B=1, Nq=512, Nk=512)
    q = synth.normal_tensor(2, synth.Q_ID, 1, 32, 512, 128)
    k = np.stack([synth.prefill_k_slice(2, w, 0, h) for h in range(8)])[None]
    v = synth.normal_tensor(2, synth.V_ID, 1, 8, 512, 128)
    o, l, ro, rl = _run(q, k, v, True, 64)
    assert_attn_close(o, ro, "outlier channels N512")


def test_prefill_strided_layouts_and_determinism(gpu):
    from bit_quantized_attention_online_amd import ops
    q, k, v = _inputs(2, 4, 2, 200, 200, 128, seed=5)
    # [B, N, H, d] storage viewed as [B, H, N, d]
    qd = to_dev(np.ascontiguousarray(q.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    kd = to_dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    vd = to_dev(v)
    out = torch.empty((2, 200, 4, 128), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    o1 = ops.attn_prefill(qd, kd, vd, causal=True, v_tile_rows=64, out=out)
    o2 = ops.attn_prefill(qd, kd, vd, causal=True, v_tile_rows=64)
    torch.cuda.synchronize()
    assert torch.equal(o1.contiguous().view(torch.int16), o2.view(torch.int16))
    ro, _ = oatt.qk4v8_prefill(q, k, v, 1 / math.sqrt(128), True, 64)
    assert_attn_close(from_dev_bf16(o2), ro, "strided")


@pytest.mark.timeout(600)
def test_prefill_causal_gqa_workload_full(gpu):
    """The causal GQA prefill workload at full size (B4 Hq32 Hkv8 N4096 d128,
    4 outlier K channels x20), every output of both default-bar probability
    formats compared with the oracle."""
    w = synth.WORKLOADS[2]
    q, k, v = synth.prefill_inputs(2)
    from bit_quantized_attention_online_amd import ops
    outs = {}
    for pm in P_MODES:
        print(f"[case] full causal GQA workload p_mode={pm}", flush=True)
        o = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=1 / math.sqrt(128),
                             v_tile_rows=w["v_tile_rows"], p_mode=pm)
        torch.cuda.synchronize()
        outs[pm] = from_dev_bf16(o)
    for b in range(w["B"]):
        ro, _ = oatt.qk4v8_prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], 1 / math.sqrt(128), True, 64)
        for pm in P_MODES:
            assert_attn_close(outs[pm][b:b + 1], ro, f"workload 2 batch {b} p_mode={pm}")


@pytest.mark.timeout(600)
def test_prefill_long_causal_workload_sampled_rows(gpu):
    """The 131072-token causal prefill (B1 Hq64 Hkv8 d128, 2% of K rows x10) at
    full size; sampled rows (first, last, tile edges, random) of every head are
    compared with the oracle."""
    w = synth.WORKLOADS[4]
    N = w["Nq"]
    from bit_quantized_attention_online_amd import ops
    q = synth.normal_tensor(4, synth.Q_ID, 1, 64, N, 128)
    k = np.stack([synth.prefill_k_slice(4, w, 0, h) for h in range(8)])[None]
    v = synth.normal_tensor(4, synth.V_ID, 1, 8, N, 128)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 65536, N - 1],
                                     np.random.default_rng(4).integers(0, N, 9)]))
    ro, _ = oatt.qk4v8_prefill(q[:, :, rows], k, v, 1 / math.sqrt(128), True, 64, rows=(rows, N))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    for pm in P_MODES:
        print(f"[case] long causal workload N=131072 p_mode={pm}", flush=True)
        o = ops.attn_prefill(qd, kd, vd, causal=True, softmax_scale=1 / math.sqrt(128), v_tile_rows=64, p_mode=pm)
        torch.cuda.synchronize()
        o_rows = from_dev_bf16(o[:, :, torch.from_numpy(rows).cuda()])
        del o
        assert_attn_close(o_rows, ro, f"workload 4 sampled rows p_mode={pm}")


FAST_CASES = [
    (1, 1, 1, 256, 256, 64, False, 64),
    (2, 4, 2, 300, 300, 128, True, 64),
    (1, 8, 1, 77, 333, 128, True, 32),
    (1, 16, 2, 260, 260, 128, True, 64),
    (1, 4, 4, 513, 700, 128, False, 256),
]


# Fast mode against exact attention of the quantized operands: every weight
# carries up to 2^-4 relative E4M3 rounding (3 mantissa bits), which averages
# down over a row to a measured 1.4e-2 .. 2.5e-2 relative L2; the gate is
# twice the largest of those.
FAST_VS_EXACT_REL_L2 = 5e-2


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,R", FAST_CASES)
def test_prefill_fast_mode(gpu, B, Hq, Hkv, Nq, Nk, d, causal, R):
    """Single-term FP8 probabilities against their own (tile-independent)
    oracle at the parity bar, and against exact attention within
    FAST_VS_EXACT_REL_L2."""
    from bit_quantized_attention_online_amd import ops
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed=B * 1000 + Nq + Nk + d + 7)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] prefill fast q{q.shape} k{k.shape} causal={causal} R={R}", flush=True)
    o, l = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal, softmax_scale=scale, v_tile_rows=R,
                            return_lse=True, p_mode=1)
    torch.cuda.synchronize()
    ro, rl = oatt.qk4v8_prefill_fast(q, k, v, scale, causal, R)
    got = from_dev_bf16(o)
    assert_attn_close(got, ro, f"fast {B},{Hq},{Hkv},{Nq},{Nk},{d},{causal},{R}")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3
    ex, _ = oatt.qk4v8_prefill(q, k, v, scale, causal, R)
    rel = np.linalg.norm(got - ex) / np.linalg.norm(ex)
    print(f"[report] fast mode vs exact attention of the quantized operands: rel_l2={rel:.3e}", flush=True)
    assert rel <= FAST_VS_EXACT_REL_L2


def test_prefill_fast_mode_workload_sample(gpu):
    """The causal GQA workload in fast mode, sampled rows of batch 0."""
    from bit_quantized_attention_online_amd import ops
    w = synth.WORKLOADS[2]
    q, k, v = synth.prefill_inputs(2)
    scale = 1.0 / math.sqrt(w["d"])
    o = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale,
                         v_tile_rows=w["v_tile_rows"], p_mode=1)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, w["Nq"], 97), [w["Nq"] - 1]]))
    ro, _ = oatt.qk4v8_prefill_fast(q[:1, :, rows], k[:1], v[:1], scale, True, w["v_tile_rows"],
                                    rows=(rows, w["Nq"]))
    sel = torch.from_numpy(rows).to(o.device)
    got = from_dev_bf16(o[:1].index_select(2, sel))
    assert_attn_close(got, ro, "fast workload 2 batch 0 sampled rows")
    ex, _ = oatt.qk4v8_prefill(q[:1, :, rows], k[:1], v[:1], scale, True, w["v_tile_rows"], rows=(rows, w["Nq"]))
    rel = np.linalg.norm(got - ex) / np.linalg.norm(ex)
    print(f"[report] fast mode (workload 2 sample) vs exact attention: rel_l2={rel:.3e}", flush=True)
    assert rel <= FAST_VS_EXACT_REL_L2


@pytest.mark.timeout(600)
def test_prefill_hadamard_causal_gqa_workload_sampled(gpu):
    """The causal GQA workload at full size with rotated Q and K (B4 Hq32 Hkv8
    N4096 d128, outlier K channels): sampled rows of batch 1 against the
    oracle's rotated path."""
    from bit_quantized_attention_online_amd import ops
    w = synth.WORKLOADS[2]
    q, k, v = synth.prefill_inputs(2)
    scale = 1.0 / math.sqrt(w["d"])
    print("[case] full causal GQA workload, hadamard", flush=True)
    o = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale,
                         v_tile_rows=w["v_tile_rows"], hadamard=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, 2047, w["Nq"] - 1],
                                     np.random.default_rng(6).integers(0, w["Nq"], 40)]))
    sel = torch.from_numpy(rows).to(o.device)
    got = from_dev_bf16(o[1:2].index_select(2, sel))
    ro, _ = oatt.qk4v8_prefill_hadamard(q[1:2, :, rows], k[1:2], v[1:2], scale, True, w["v_tile_rows"],
                                        rows=(rows, w["Nq"]))
    assert_attn_close(got, ro, "workload 2 hadamard, batch 1 sampled rows")


HAD_CASES = [
    (1, 1, 1, 256, 256, 64, False, 64),
    (2, 4, 2, 300, 300, 128, True, 64),
    (1, 8, 1, 77, 333, 128, True, 32),
    (1, 4, 4, 513, 700, 128, False, 256),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,R", HAD_CASES)
def test_prefill_hadamard(gpu, B, Hq, Hkv, Nq, Nk, d, causal, R):
    from bit_quantized_attention_online_amd import ops
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed=B * 1000 + Nq + Nk + d + 11)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] prefill hadamard q{q.shape} k{k.shape} causal={causal} R={R}", flush=True)
    o, l = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal, softmax_scale=scale, v_tile_rows=R,
                            return_lse=True, hadamard=True)
    torch.cuda.synchronize()
    ro, rl = oatt.qk4v8_prefill_hadamard(q, k, v, scale, causal, R)
    assert_attn_close(from_dev_bf16(o), ro, f"hadamard {B},{Hq},{Hkv},{Nq},{Nk},{d},{causal},{R}")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3


def test_prefill_hadamard_outlier_channels(gpu):
    """The causal GQA workload's outlier-channel K at N=512: rotated parity, and
    the distance of the plain and the rotated path to unquantized attention
    (reported)."""
    from bit_quantized_attention_online_amd import ops
    from oracle.formats import bf16_bits_to_float64
    w = dict(synth.WORKLOADS[2], B=1, Nq=512, Nk=512)
    q = synth.normal_tensor(2, synth.Q_ID, 1, 32, 512, 128)
    k = np.stack([synth.prefill_k_slice(2, w, 0, h) for h in range(8)])[None]
    v = synth.normal_tensor(2, synth.V_ID, 1, 8, 512, 128)
    scale = 1.0 / math.sqrt(128)
    outs = {}
    for had in (False, True):
        outs[had] = from_dev_bf16(ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True,
                                                   softmax_scale=scale, v_tile_rows=64, hadamard=had))
    ro, _ = oatt.qk4v8_prefill_hadamard(q, k, v, scale, True, 64)
    assert_attn_close(outs[True], ro, "hadamard outlier channels N512")
    exact, _ = oatt.attention(bf16_bits_to_float64(q), bf16_bits_to_float64(k), bf16_bits_to_float64(v), scale, True)
    for had in (False, True):
        rel = np.linalg.norm(outs[had] - exact) / np.linalg.norm(exact)
        print(f"[report] {'rotated' if had else 'plain'} QK4V8 vs unquantized attention: rel_l2={rel:.3e}", flush=True)


def _ramped(B, Hq, Hkv, Nq, Nk, d, seed, slope):
    """Q rows near one direction u and K rows along u with a weight growing
    with the key position, so the score of a row grows along the keys."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    q = u + 0.3 * rng.standard_normal((B, Hq, Nq, d))
    k = (np.arange(Nk) * slope)[None, None, :, None] * u + 0.3 * rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    return tuple(synth.bf16_bits(x.astype(np.float32)) for x in (q, k, v))


@pytest.mark.parametrize("p_mode", P_MODES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_growing_scores_rescale(gpu, causal, p_mode):
    """Row maxima that grow by several times the lazy-rescale headroom along
    the keys, so the accumulators and the row sums are rescaled during the
    walk (the online-softmax correction step)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 640, 128
    q, k, v = _ramped(B, Hq, Hkv, N, N, d, seed=21, slope=1 / 400)
    # the inputs do what the test needs: over the keys the log2-domain score
    # of a row grows by much more than the 8 units of headroom
    c = math.log2(math.e) / math.sqrt(d)
    s = np.einsum("hd,hkd->hk", synth.bits_to_f32(q[0, 0::Hq // Hkv, -1]).astype(np.float64),
                  synth.bits_to_f32(k[0]).astype(np.float64)) * c
    assert (s[:, -128:].max(axis=1) - s[:, :128].max(axis=1)).min() > 12
    o, l, ro, rl = _run(q, k, v, causal, 64, p_mode=p_mode)
    assert_attn_close(o, ro, f"growing scores causal={causal} p_mode={p_mode}")
    assert np.abs(l - rl).max() < 5e-3


@pytest.mark.parametrize("p_mode", P_MODES)
@pytest.mark.parametrize("case", ["zero_q", "zero_k", "const_v", "zero_v"])
def test_prefill_degenerate_inputs(gpu, case, p_mode):
    """Degenerate inputs of the method: all-zero Q or K blocks (E8M0 floor,
    every score 0, uniform weights over the visible keys), a constant V
    (every row of the output is that value) and an all-zero V."""
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 128
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, seed=31)
    if case == "zero_q":
        q[:] = 0
    elif case == "zero_k":
        k[:] = 0
    elif case == "const_v":
        v[:] = synth.bf16_bits(np.full(1, 1.375, np.float32))[0]
    else:
        v[:] = 0
    o, l, ro, rl = _run(q, k, v, True, 64, p_mode=p_mode)
    assert_attn_close(o, ro, f"degenerate {case} p_mode={p_mode}")
    assert np.abs(l - rl).max() < 5e-3
    if case == "const_v":
        # 1.375 is exact in E4M3 (times the tile's power of two) and in bf16,
        # and the output divides the weighted sum by the sum of the same
        # weights: every output element is 1.375 after the bf16 rounding
        assert (o == 1.375).all()
    if case == "zero_v":
        assert not o.any()
    if case in ("zero_q", "zero_k"):
        # every score 0, so every weight is exactly 1 (bf16, or hi = 2^7 and
        # lo = 0 in the two-term split): row i is the mean of the visible
        # rows of V-hat, up to the fp32 sums and the bf16 rounding
        assert (np.abs(o - ro) <= np.abs(ro) * 2.0 ** -8 + 1e-4).all()
