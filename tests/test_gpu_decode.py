"""GPU decode / block-verify attention over a quantized cache vs the oracle."""
import math

import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import attention as oatt
from oracle import quant
from tests._util import assert_attn_close, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu


def _cache_from(k_bits, v_bits, R):
    """Quantize bf16 K/V [B, Hkv, cap, d] into a cache with the GPU quantizers."""
    from bit_quantized_attention_online_amd import ops
    B, Hkv, cap, d = k_bits.shape
    kc, ks = ops.quantize_qk(to_dev(k_bits))
    vc, vs = ops.quantize_v(to_dev(v_bits).reshape(B * Hkv, cap, d), R)
    return kc, ks, vc.reshape(B, Hkv, cap, d), vs.reshape(B, Hkv, -1)


DEC_CASES = [
    # B, Hq, Hkv, q_len, kv_len, cap, d, R, splits, ragged lens
    (3, 8, 2, 1, 1000, 1100, 128, 256, 0, False),
    (2, 8, 2, 1, 1000, 1000, 128, 256, 1, False),
    (2, 8, 2, 1, 777, 800, 128, 64, 5, True),
    (2, 16, 2, 4, 600, 700, 128, 256, 3, True),     # block verify, 32 rows
    (1, 64, 8, 8, 1500, 1536, 128, 256, 0, False),  # 64 rows per KV head
    (2, 12, 2, 7, 500, 520, 128, 64, 0, True),      # 42 rows: three 16-row blocks
    (1, 10, 2, 8, 300, 300, 64, 32, 2, False),      # 40 rows at head_dim 64
    (2, 4, 4, 1, 300, 300, 64, 32, 0, False),
    (1, 6, 2, 3, 130, 140, 64, 128, 2, True),
    (2, 8, 8, 1, 1, 1, 128, 256, 0, False),         # a single cached token
    (1, 8, 2, 2, 1300, 1300, 128, 256, 9, True),    # nine splits, three of them empty
    # four 16-row blocks at head_dim 128: the ping-pong workgroup
    (2, 64, 8, 8, 700, 760, 128, 32, 0, True),      # ragged lengths, 32-row V tiles
    (1, 56, 8, 8, 2100, 2200, 128, 64, 3, True),    # 56 rows, three splits
    (2, 32, 4, 8, 100, 128, 128, 256, 0, True),     # one partial tile per sequence
    (1, 64, 8, 8, 1300, 1300, 128, 128, 9, True),   # nine splits, some of them empty
]


@pytest.mark.parametrize("B,Hq,Hkv,q_len,kv_len,cap,d,R,splits,ragged", DEC_CASES)
def test_decode_parity(gpu, B, Hq, Hkv, q_len, kv_len, cap, d, R, splits, ragged):
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(B * 7 + kv_len + d + q_len)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    lens = np.full(B, kv_len, dtype=np.int32)
    if ragged:
        lens = rng.integers(q_len, kv_len + 1, B).astype(np.int32)
        lens[0] = kv_len
    print(f"[case] decode B{B} Hq{Hq} Hkv{Hkv} q_len{q_len} kv_len{kv_len} cap{cap} d{d} R{R} s{splits}", flush=True)
    kc, ks, vc, vs = _cache_from(k, v, R)
    kl = torch.from_numpy(lens).cuda() if ragged else None
    o, l = ops.attn_decode(to_dev(q), kc, ks, vc, vs, kv_len, v_tile_rows=R, kv_lens=kl, num_splits=splits,
                           return_lse=True)
    torch.cuda.synchronize()
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    assert np.array_equal(kc.cpu().numpy(), rkc) and np.array_equal(ks.cpu().numpy(), rks)
    assert np.array_equal(vc.cpu().numpy().reshape(B * Hkv, cap, d), rvc)
    ro, rl = oatt.qk4v8_decode(q, rkc, rks, rvc.reshape(B, Hkv, cap, d), rvs.reshape(B, Hkv, -1), lens, R,
                               1 / math.sqrt(d))
    assert_attn_close(from_dev_bf16(o), ro, "decode")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3    # normalizer from the FP8 weights (rel. error <= 2^-8)


def test_decode_split_count_and_prefill_agree(gpu):
    """Different split counts give the same result within rounding, and the
    decode of the last q_len queries matches the GPU prefill's last rows."""
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, d, q_len, n, R = 2, 8, 2, 128, 4, 640, 64
    rng = np.random.default_rng(11)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    kc, ks, vc, vs = _cache_from(k, v, R)
    outs = [from_dev_bf16(ops.attn_decode(to_dev(q), kc, ks, vc, vs, n, v_tile_rows=R, num_splits=s))
            for s in (1, 2, 5)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-2
    po = ops.attn_prefill(to_dev(q).permute(0, 2, 1, 3), to_dev(k), to_dev(v), causal=True, v_tile_rows=R)
    po = from_dev_bf16(po).transpose(0, 2, 1, 3)
    assert np.abs(po - outs[0]).max() < 2e-2


def _full_cache_workload(cfg, sample_b):
    """Build the full quantized cache of a decode workload on the GPU, batch by
    batch; return the GPU cache and the host K/V of the sampled batches."""
    from bit_quantized_attention_online_amd import ops
    w = synth.WORKLOADS[cfg]
    B, Hkv, n, d, R = w["B"], w["Hkv"], w["kv_len"], w["d"], w["v_tile_rows"]
    kc = torch.empty((B, Hkv, n, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, n, d // 32), dtype=torch.uint8, device="cuda")
    vc = torch.empty((B, Hkv, n, d), dtype=torch.uint8, device="cuda")
    vs = torch.empty((B, Hkv, -(-n // R)), dtype=torch.uint8, device="cuda")
    kept = {}
    for b in range(B):
        kb = synth.normal_batch(cfg, synth.K_ID, b, Hkv, n, d)
        vb = synth.normal_batch(cfg, synth.V_ID, b, Hkv, n, d)
        if b % 16 == 0:
            print(f"[progress] cache batch {b}/{B}", flush=True)
        c, s = ops.quantize_qk(to_dev(kb))
        kc[b], ks[b] = c, s
        c, s = ops.quantize_v(to_dev(vb), R)
        vc[b], vs[b] = c, s
        if b in sample_b:
            kept[b] = (kb, vb)
    torch.cuda.synchronize()
    return w, (kc, ks, vc, vs), kept


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [3, 5])
def test_decode_workloads_full_size_sampled(gpu, cfg):
    """Decode (B64 Hq64 Hkv8 kv32768) and block verify (B32, 8 queries over
    16384 + 8 keys) at full size; sampled batches are checked bit-exact for the
    cache and within tolerance for the outputs."""
    from bit_quantized_attention_online_amd import ops
    sample_b = [0, 13, 31] if cfg == 5 else [0, 29, 63]
    print(f"[case] full decode workload {cfg}", flush=True)
    w, (kc, ks, vc, vs), kept = _full_cache_workload(cfg, sample_b)
    q = synth.normal_tensor(cfg, synth.Q_ID, w["B"], w["Hq"], w["q_len"], w["d"]).transpose(0, 2, 1, 3).copy()
    o = ops.attn_decode(to_dev(q), kc, ks, vc, vs, w["kv_len"], v_tile_rows=w["v_tile_rows"])
    torch.cuda.synchronize()
    o = from_dev_bf16(o)
    for b in sample_b:
        kb, vb = kept[b]
        rkc, rks = quant.quantize_qk(kb)
        rvc, rvs = quant.quantize_v(vb, w["v_tile_rows"])
        assert np.array_equal(kc[b].cpu().numpy(), rkc) and np.array_equal(ks[b].cpu().numpy(), rks)
        assert np.array_equal(vc[b].cpu().numpy(), rvc) and np.array_equal(vs[b].cpu().numpy(), rvs)
        ro, _ = oatt.qk4v8_decode(q[b:b + 1], rkc[None], rks[None], rvc[None], rvs[None],
                                  np.array([w["kv_len"]]), w["v_tile_rows"], 1 / math.sqrt(w["d"]))
        assert_attn_close(o[b:b + 1], ro, f"workload {cfg} batch {b}")
    # the same cache with the drafter's 1024-key sliding window
    ow = from_dev_bf16(ops.attn_decode(to_dev(q), kc, ks, vc, vs, w["kv_len"], v_tile_rows=w["v_tile_rows"],
                                       window=1024))
    for b in sample_b:
        kb, vb = kept[b]
        rkc, rks = quant.quantize_qk(kb)
        rvc, rvs = quant.quantize_v(vb, w["v_tile_rows"])
        ro, _ = oatt.qk4v8_decode(q[b:b + 1], rkc[None], rks[None], rvc[None], rvs[None],
                                  np.array([w["kv_len"]]), w["v_tile_rows"], 1 / math.sqrt(w["d"]), window=1024)
        assert_attn_close(ow[b:b + 1], ro, f"workload {cfg} window 1024 batch {b}")
    if cfg == 3:
        # the same cache as 256-token pages in a shuffled order (the paged
        # launch the bench times): the same bits as the contiguous cache, so
        # the sampled batches above also pin the paged result to the oracle
        from tests.test_gpu_paged import _table, _to_pages
        P, R = 256, w["v_tile_rows"]
        table = _table(w["B"], w["kv_len"] // P, 0, seed=w["kv_len"])
        pages = (_to_pages(kc, table, P, P), _to_pages(ks, table, P, P), _to_pages(vc, table, P, P),
                 _to_pages(vs, table, P, P // R))
        del kc, ks, vc, vs
        op = ops.attn_decode(to_dev(q), *pages, w["kv_len"], v_tile_rows=R,
                             block_table=torch.from_numpy(table).cuda(), page_size=P)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bf16(op), o), "paged decode differs from the contiguous cache"


@pytest.mark.parametrize("q_len,d", [(1, 128), (4, 128), (16, 128), (2, 64)])
def test_decode_hadamard(gpu, q_len, d):
    """Decode over a cache written with rotated K rows, queries rotated in the
    kernel, against the oracle's rotated definition."""
    from bit_quantized_attention_online_amd import ops
    from oracle import cache as ocache
    B, Hq, Hkv, n, R = 2, 8, 2, 700, 256
    rng = np.random.default_rng(q_len * 10 + d)
    k = synth.bf16_bits(rng.standard_normal((B, n, Hkv, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, n, Hkv, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    dev = torch.device("cuda:0")
    kc = torch.zeros((B, Hkv, n, d // 2), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B, Hkv, n, d // 32), dtype=torch.uint8, device=dev)
    vc = torch.zeros((B, Hkv, n, d), dtype=torch.uint8, device=dev)
    vs = torch.zeros((B, Hkv, -(-n // R)), dtype=torch.uint8, device=dev)
    tail = torch.zeros((B, Hkv, R, d), dtype=torch.bfloat16, device=dev)
    ops.kv_append(to_dev(k), to_dev(v), kc, ks, vc, vs, tail, 0, v_tile_rows=R, hadamard=True)
    o, l = ops.attn_decode(to_dev(q), kc, ks, vc, vs, n, v_tile_rows=R, return_lse=True, hadamard=True)
    torch.cuda.synchronize()
    rk = np.zeros((B, Hkv, n, d // 2), np.uint8)
    rks = np.zeros((B, Hkv, n, d // 32), np.uint8)
    rv = np.zeros((B, Hkv, n, d), np.uint8)
    rvs = np.zeros((B, Hkv, -(-n // R)), np.uint8)
    for b in range(B):
        for h in range(Hkv):
            rk[b, h], rks[b, h], rv[b, h], rvs[b, h] = ocache.cache_of_sequence(k[b, :, h], v[b, :, h], R, hadamard=True)
    assert np.array_equal(kc.cpu().numpy(), rk) and np.array_equal(ks.cpu().numpy(), rks)
    ro, rl = oatt.qk4v8_decode_hadamard(q, rk, rks, rv, rvs, np.array([n] * B), R, 1 / math.sqrt(d))
    assert_attn_close(from_dev_bf16(o), ro, f"decode hadamard q_len{q_len} d{d}")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3


def test_decode_single_split_direct_and_merged_agree(gpu):
    """With one split the kernel writes the final output itself when the
    output is 8-byte aligned with strides in multiples of 4 elements;
    otherwise the merge pass writes it.  Both must give the same bits."""
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, d, q_len, n, R = 2, 8, 2, 128, 2, 900, 256
    rng = np.random.default_rng(17)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    kc, ks, vc, vs = _cache_from(k, v, R)
    qd = to_dev(q)
    print("[case] decode one split, direct and merged output", flush=True)
    o1, l1 = ops.attn_decode(qd, kc, ks, vc, vs, n, v_tile_rows=R, num_splits=1, return_lse=True)
    wide = torch.zeros((B, q_len, Hq, d + 2), dtype=torch.bfloat16, device=qd.device)
    o2, l2 = ops.attn_decode(qd, kc, ks, vc, vs, n, v_tile_rows=R, num_splits=1, return_lse=True,
                             out=wide[..., :d])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.count_nonzero(wide[..., d:]) == 0
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, n, d), R)
    ro, _ = oatt.qk4v8_decode(q, rkc, rks, rvc.reshape(B, Hkv, n, d), rvs.reshape(B, Hkv, -1), np.array([n] * B), R,
                              1 / math.sqrt(d))
    assert_attn_close(from_dev_bf16(o1), ro, "decode one split")


@pytest.mark.parametrize("q_len,d,R", [(1, 128, 64), (8, 128, 256), (3, 64, 32)])
def test_decode_ignores_cache_bytes_past_each_length(gpu, q_len, d, R):
    """Rows at or past a sequence's length hold NaN bytes (E4M3 NaN codes,
    E8M0 NaN scales) in a contiguous cache; the loads stop at the length, so
    the result is finite and matches the oracle over the valid rows.  The
    lengths end inside 128-key tiles and inside V tiles."""
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, cap = 3, 16, 2, 700
    rng = np.random.default_rng(91 + q_len + d + R)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    lens = np.array([700, 333, 129], dtype=np.int32)
    print(f"[case] decode past-length NaN bytes q_len{q_len} d{d} R{R}", flush=True)
    kc, ks, vc, vs = _cache_from(k, v, R)
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    for b, n in enumerate(lens):
        kc[b, :, n:] = 0xFF
        ks[b, :, n:] = 0xFF
        vc[b, :, n:] = 0xFF
        vs[b, :, -(-int(n) // R):] = 0xFF          # V tiles that start past the length
    o = ops.attn_decode(to_dev(q), kc, ks, vc, vs, cap, v_tile_rows=R, kv_lens=torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    out = from_dev_bf16(o)
    assert np.isfinite(out).all()
    ro, _ = oatt.qk4v8_decode(q, rkc, rks, rvc.reshape(B, Hkv, cap, d), rvs.reshape(B, Hkv, -1), lens, R,
                              1 / math.sqrt(d))
    assert_attn_close(out, ro, "decode past-length NaN bytes")


@pytest.mark.parametrize("splits,paged,Hq", [(0, False, 8), (3, False, 8), (1, False, 8), (2, True, 8),
                                             (0, False, 32), (3, False, 32), (2, True, 32)])
def test_decode_out_of_contract_lengths_stay_in_bounds(gpu, splits, paged, Hq):
    """kv_lens above kv_len are read as kv_len, below q_len as an empty
    sequence (zero rows, lse -inf).  The cache bytes past kv_len are E4M3 NaN
    patterns, and cap is larger than every length, so a read past kv_len
    would show as NaN in the output while staying inside the allocation.
    Hq 32 gives 64 query rows per KV head, the block-verify kernel."""
    from bit_quantized_attention_online_amd import ops
    B, Hkv, q_len, kv_len, cap, d, R = 4, 2, 4, 600, 1024, 128, 256
    lens = np.array([900, 0, 3, 450], dtype=np.int32)
    clamped = np.array([600, 0, 0, 450])
    rng = np.random.default_rng(77)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    print(f"[case] decode out-of-contract lengths {lens.tolist()} splits={splits} paged={paged} Hq={Hq}", flush=True)
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    rvc, rvs = rvc.reshape(B, Hkv, cap, d), rvs.reshape(B, Hkv, -1)
    kc, ks, vc, vs = (rkc.copy(), rks.copy(), rvc.copy(), rvs.copy())
    kc[:, :, kv_len:] = 0xFF
    ks[:, :, kv_len:] = 0xFF
    vc[:, :, kv_len:] = 0x7F                      # E4M3 NaN
    vs[:, :, -(-kv_len // R):] = 0xFF             # E8M0 NaN
    dev = torch.device("cuda:0")
    cache = [torch.from_numpy(x).to(dev) for x in (kc, ks, vc, vs)]
    kw = {}
    if paged:
        P = 256
        npp = cap // P
        table = np.arange(B * npp, dtype=np.int32)[::-1].copy().reshape(B, npp)

        def pages(t, per):
            src = t.reshape((B, Hkv, npp, per) + tuple(t.shape[3:])).transpose(1, 2)
            pool = torch.empty((B * npp, Hkv, per) + tuple(t.shape[3:]), dtype=t.dtype, device=dev)
            pool[torch.from_numpy(table.reshape(-1)).long().to(dev)] = src.reshape((B * npp, Hkv, per)
                                                                                  + tuple(t.shape[3:]))
            return pool

        cache = [pages(cache[0], P), pages(cache[1], P), pages(cache[2], P), pages(cache[3], P // R)]
        kw = dict(block_table=torch.from_numpy(table).to(dev), page_size=P)
    o, l = ops.attn_decode(to_dev(q), *cache, kv_len, v_tile_rows=R, kv_lens=torch.from_numpy(lens).to(dev),
                           num_splits=splits, return_lse=True, **kw)
    torch.cuda.synchronize()
    o, l = from_dev_bf16(o), l.cpu().numpy()
    assert np.isfinite(o).all()
    live = clamped > 0
    ro, rl = oatt.qk4v8_decode(q[live], rkc[live], rks[live], rvc[live], rvs[live], clamped[live], R,
                               1 / math.sqrt(d))
    assert_attn_close(o[live], ro, "clamped lengths")
    assert np.abs(l[live] - rl).max() < 5e-3
    assert (o[~live] == 0).all() and np.isneginf(l[~live]).all()


def test_decode_auto_split_count_on_mi355x(gpu):
    """num_splits = 0 derives the count from the CU count and the split
    kernel's occupancy; on MI355X (256 CUs) that gives 2 splits for the
    decode workload and 1 for block verify (one ping-pong workgroup per CU)."""
    from bit_quantized_attention_online_amd import ops
    for cfg, want in ((3, 2), (5, 1)):
        w = synth.WORKLOADS[cfg]
        q = torch.empty((w["B"], w["q_len"], w["Hq"], w["d"]), dtype=torch.bfloat16, device="cuda")
        kc = torch.empty((w["B"], w["Hkv"], w["kv_len"], w["d"] // 2), dtype=torch.uint8, device="cuda")
        auto = ops.decode_workspace_bytes(q, kc, w["kv_len"], w["v_tile_rows"])
        forced = ops.decode_workspace_bytes(q, kc, w["kv_len"], w["v_tile_rows"], num_splits=want)
        print(f"[case] auto splits {w['name']}: {auto} vs {forced} bytes", flush=True)
        assert auto == forced > 0


@pytest.mark.parametrize("Hq,Hkv,q_len,R,splits", [(8, 2, 1, 256, 1), (64, 8, 8, 64, 0)])
def test_decode_growing_scores_rescale(gpu, Hq, Hkv, q_len, R, splits):
    """Decode (one split, one row per query head) and block verify (the
    64-row ping-pong workgroup) over keys whose scores grow along the cache
    by several times the lazy-rescale headroom: the running maximum moves
    during the walk and the accumulators and row sums are rescaled."""
    from bit_quantized_attention_online_amd import ops
    B, d, n = 1, 128, 1000
    rng = np.random.default_rng(Hq + q_len)
    u = rng.standard_normal(d)
    q = synth.bf16_bits((u + 0.3 * rng.standard_normal((B, q_len, Hq, d))).astype(np.float32))
    k = synth.bf16_bits(((np.arange(n) / 600)[None, None, :, None] * u
                         + 0.3 * rng.standard_normal((B, Hkv, n, d))).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    c = math.log2(math.e) / math.sqrt(d)
    s = synth.bits_to_f32(k[0, 0]).astype(np.float64) @ synth.bits_to_f32(q[0, 0, 0]).astype(np.float64) * c
    assert s[-128:].max() - s[:128].max() > 16       # the inputs move the maximum far enough
    print(f"[case] decode growing scores Hq{Hq} Hkv{Hkv} q_len{q_len} R{R} s{splits}", flush=True)
    kc, ks, vc, vs = _cache_from(k, v, R)
    o, l = ops.attn_decode(to_dev(q), kc, ks, vc, vs, n, v_tile_rows=R, num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, n, d), R)
    ro, rl = oatt.qk4v8_decode(q, rkc, rks, rvc.reshape(B, Hkv, n, d), rvs.reshape(B, Hkv, -1),
                               np.full(B, n, dtype=np.int32), R, 1 / math.sqrt(d))
    assert_attn_close(from_dev_bf16(o), ro, "decode growing scores")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3


@pytest.mark.parametrize("Hq,Hkv,q_len,R", [(8, 2, 1, 256), (64, 8, 8, 64)])
@pytest.mark.parametrize("case", ["zero_q", "const_v"])
def test_decode_degenerate_inputs(gpu, Hq, Hkv, q_len, R, case):
    """All-zero queries (exact uniform weights over the visible keys) and a
    constant V cache (every output element is that value), for decode and
    for the 64-row block-verify workgroup."""
    from bit_quantized_attention_online_amd import ops
    B, d, n = 2, 128, 700
    rng = np.random.default_rng(q_len + 3)
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))
    if case == "zero_q":
        q[:] = 0
    else:
        v[:] = synth.bf16_bits(np.full(1, -0.8125, np.float32))[0]
    print(f"[case] decode degenerate {case} Hq{Hq} q_len{q_len} R{R}", flush=True)
    kc, ks, vc, vs = _cache_from(k, v, R)
    o, l = ops.attn_decode(to_dev(q), kc, ks, vc, vs, n, v_tile_rows=R, return_lse=True)
    torch.cuda.synchronize()
    o = from_dev_bf16(o)
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, n, d), R)
    ro, rl = oatt.qk4v8_decode(q, rkc, rks, rvc.reshape(B, Hkv, n, d), rvs.reshape(B, Hkv, -1),
                               np.full(B, n, dtype=np.int32), R, 1 / math.sqrt(d))
    assert_attn_close(o, ro, f"decode degenerate {case}")
    assert np.abs(l.cpu().numpy() - rl).max() < 5e-3
    if case == "const_v":
        assert (o == -0.8125).all()      # exact in E4M3 (times the tile's power of two) and in bf16
    else:
        assert (np.abs(o - ro) <= np.abs(ro) * 2.0 ** -8 + 1e-4).all()
