"""GPU sliding-window attention (prefill and decode / block verify) vs the
fp64 oracle's window definition (relative L2 <= 5e-3, max abs <= 2e-2)."""
import math

import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import attention as oatt
from oracle import quant
from tests._util import assert_attn_close, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits(rng.standard_normal((B, Hq, Nq, d)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, Nk, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, Nk, d)).astype(np.float32))
    return q, k, v


PREFILL_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, R, window, p_mode
    (1, 2, 2, 700, 700, 128, 64, 100, 2),      # MHA: 256-row workgroups, early waves see masked tiles first
    (2, 8, 1, 300, 520, 128, 32, 130, 2),      # GQA 8, bottom-right offset
    (1, 4, 2, 600, 600, 64, 64, 1, 2),         # one key per row
    (1, 16, 2, 1100, 1100, 128, 256, 1024, 2), # the drafter's window
    (1, 2, 1, 333, 333, 128, 64, 333, 2),      # window = seq_k: plain causal
    (1, 4, 4, 513, 513, 128, 128, 300, 1),     # fast mode
    (1, 16, 2, 900, 900, 128, 64, 256, 1),
    (1, 16, 2, 1100, 1100, 128, 256, 1024, 3), # bf16 probabilities
    (2, 8, 1, 300, 520, 128, 32, 130, 3),
    (1, 4, 4, 513, 513, 64, 64, 300, 3),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,R,W,pt", PREFILL_CASES)
def test_prefill_window(gpu, B, Hq, Hkv, Nq, Nk, d, R, W, pt):
    from bit_quantized_attention_online_amd import ops
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed=Nq * 3 + Nk + W + pt)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] prefill window={W} p_mode={pt} q{q.shape} k{k.shape} R={R}", flush=True)
    o, l = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale, v_tile_rows=R,
                            return_lse=True, p_mode=pt, window=W)
    torch.cuda.synchronize()
    ref = oatt.qk4v8_prefill_fast if pt == 1 else oatt.qk4v8_prefill
    ro, rl = ref(q, k, v, scale, True, R, window=W)
    assert_attn_close(from_dev_bf16(o), ro, f"prefill window {B},{Hq},{Hkv},{Nq},{Nk},{d},{R},{W},{pt}")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3


def test_prefill_window_hadamard(gpu):
    from bit_quantized_attention_online_amd import ops
    q, k, v = _inputs(1, 8, 2, 640, 640, 128, seed=99)
    scale = 1.0 / math.sqrt(128)
    print("[case] prefill window=200 hadamard", flush=True)
    o = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale, v_tile_rows=64,
                         hadamard=True, window=200)
    torch.cuda.synchronize()
    ro, _ = oatt.qk4v8_prefill_hadamard(q, k, v, scale, True, 64, window=200)
    assert_attn_close(from_dev_bf16(o), ro, "prefill window hadamard")


def test_prefill_window_causal_gqa_workload_sampled(gpu):
    """The causal GQA prefill workload (B4 Hq32 Hkv8 N4096 d128, outlier K
    channels) with the drafter's 1024-key window, sampled rows of batch 0."""
    from bit_quantized_attention_online_amd import ops
    w = synth.WORKLOADS[2]
    q, k, v = synth.prefill_inputs(2)
    scale = 1.0 / math.sqrt(w["d"])
    print("[case] prefill window=1024 causal GQA workload", flush=True)
    o = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale,
                         v_tile_rows=w["v_tile_rows"], window=1024)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, w["Nq"], 61), [1023, 1024, 1025, w["Nq"] - 1]]))
    ro, _ = oatt.qk4v8_prefill(q[:1, :, rows], k[:1], v[:1], scale, True, w["v_tile_rows"], rows=(rows, w["Nq"]),
                               window=1024)
    sel = torch.from_numpy(rows).to(o.device)
    assert_attn_close(from_dev_bf16(o[:1].index_select(2, sel)), ro, "window 1024 workload 2 batch 0 sampled rows")


DECODE_CASES = [
    # B, Hq, Hkv, q_len, kv_len, cap, d, R, splits, ragged, window
    (3, 8, 2, 1, 1000, 1100, 128, 256, 0, False, 100),
    (2, 16, 2, 4, 900, 1000, 128, 64, 0, True, 200),
    (1, 64, 8, 8, 3000, 3072, 128, 256, 0, False, 1024),   # drafted block, the drafter's window
    (2, 4, 4, 1, 300, 300, 64, 32, 3, False, 1),
    (2, 16, 2, 4, 300, 300, 128, 128, 0, False, 2),        # window shorter than the block
    (3, 8, 2, 2, 5000, 5000, 128, 128, 0, True, 1024),
    (2, 8, 2, 1, 640, 640, 128, 256, 2, False, 640),       # window = kv_len: plain decode
    (2, 64, 8, 8, 2000, 2100, 128, 64, 2, True, 500),      # ping-pong workgroup, two splits
]


@pytest.mark.parametrize("B,Hq,Hkv,q_len,kv_len,cap,d,R,splits,ragged,W", DECODE_CASES)
def test_decode_window(gpu, B, Hq, Hkv, q_len, kv_len, cap, d, R, splits, ragged, W):
    """Keys before the tile that holds query 0's first visible key are filled
    with NaN bytes (E4M3 NaN codes, E8M0 NaN scales): the result stays finite
    and equal to the oracle only if they are never read."""
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(B * 5 + kv_len + W + q_len)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    lens = np.full(B, kv_len, dtype=np.int32)
    if ragged:
        lens = rng.integers(q_len, kv_len + 1, B).astype(np.int32)
        lens[0] = kv_len
    print(f"[case] decode window={W} B{B} Hq{Hq} Hkv{Hkv} q_len{q_len} kv_len{kv_len} R{R} s{splits}", flush=True)
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    rvc, rvs = rvc.reshape(B, Hkv, cap, d), rvs.reshape(B, Hkv, -1)
    ro, rl = oatt.qk4v8_decode(q, rkc, rks, rvc, rvs, lens, R, 1 / math.sqrt(d), window=W)
    kc, ks, vc = rkc.copy(), rks.copy(), rvc.copy()
    for b in range(B):
        base = max(0, int(lens[b]) - q_len + 1 - W) // 128 * 128
        kc[b, :, :base] = 0xFF
        ks[b, :, :base] = 0xFF
        vc[b, :, :base] = 0xFF
    dev = torch.device("cuda:0")
    kl = torch.from_numpy(lens).to(dev) if ragged else None
    o, l = ops.attn_decode(to_dev(q), torch.from_numpy(kc).to(dev), torch.from_numpy(ks).to(dev),
                           torch.from_numpy(vc).to(dev), torch.from_numpy(rvs).to(dev), kv_len, v_tile_rows=R,
                           kv_lens=kl, num_splits=splits, return_lse=True, window=W)
    torch.cuda.synchronize()
    assert_attn_close(from_dev_bf16(o), ro, "decode window")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3


def test_decode_window_matches_prefill_window(gpu):
    """The windowed decode of the last q_len queries equals the windowed GPU
    prefill's last rows (same quantized operands, both bottom-right aligned)."""
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, d, q_len, n, R, W = 2, 8, 2, 128, 4, 900, 64, 300
    q, k, v = _inputs(B, Hq, Hkv, n, n, d, seed=21)
    scale = 1 / math.sqrt(d)
    po = ops.attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True, softmax_scale=scale, v_tile_rows=R,
                          window=W)
    kc, ks = ops.quantize_qk(to_dev(k))
    vc, vs = ops.quantize_v(to_dev(v).reshape(B * Hkv, n, d), R)
    qd = to_dev(np.ascontiguousarray(q[:, :, n - q_len:].transpose(0, 2, 1, 3)))
    do = ops.attn_decode(qd, kc, ks, vc.reshape(B, Hkv, n, d), vs.reshape(B, Hkv, -1), n, v_tile_rows=R,
                         softmax_scale=scale, window=W)
    torch.cuda.synchronize()
    a = from_dev_bf16(po)[:, :, n - q_len:]
    b = from_dev_bf16(do).transpose(0, 2, 1, 3)
    assert np.abs(a - b).max() < 2e-2
