"""Paged KV cache (pages of whole 128-key tiles named by a block table):
decode and the cache writer over a paged cache give the same bits as over the
contiguous cache holding the same rows, and match the oracle on the gathered
cache.  Pages outside the table are filled with NaN bytes (E4M3 NaN codes,
E8M0 NaN scales) so a stray read would show."""
import math

import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import quant
from tests._util import assert_attn_close, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu


def _table(B, npp, extra, seed):
    rng = np.random.default_rng(seed)
    return rng.permutation(B * npp + extra)[:B * npp].reshape(B, npp).astype(np.int32)


def _to_pages(t, table, P, per):
    """Scatter a contiguous cache array [B, Hkv, npp*per, ...] into a page pool
    [pages, Hkv, per, ...] (per = P rows, or P / R scale entries)."""
    B, npp = table.shape
    pages = int(table.max()) + 1 + 3
    pool = torch.full((pages,) + (t.shape[1], per) + tuple(t.shape[3:]), 0xFF, dtype=t.dtype, device=t.device)
    src = t.reshape((B, t.shape[1], npp, per) + tuple(t.shape[3:])).transpose(1, 2)
    pool[torch.from_numpy(table.reshape(-1)).long().to(t.device)] = src.reshape((B * npp, t.shape[1], per)
                                                                                   + tuple(t.shape[3:]))
    return pool


DEC_CASES = [
    # B, Hq, Hkv, q_len, d, R, P, pages per sequence, ragged, window
    (3, 8, 2, 1, 128, 256, 256, 5, True, 0),
    (2, 16, 2, 4, 128, 64, 128, 8, True, 200),
    (2, 64, 8, 8, 128, 256, 512, 3, False, 0),
    (2, 4, 4, 1, 64, 32, 128, 6, True, 0),
    (2, 64, 8, 8, 128, 64, 128, 9, True, 300),       # ping-pong workgroup, 128-key pages
]


@pytest.mark.parametrize("B,Hq,Hkv,q_len,d,R,P,npp,ragged,W", DEC_CASES)
def test_paged_decode_equals_contiguous(gpu, B, Hq, Hkv, q_len, d, R, P, npp, ragged, W):
    from bit_quantized_attention_online_amd import ops
    cap = npp * P
    rng = np.random.default_rng(cap + q_len + d + W)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, cap, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    lens = rng.integers(q_len, cap + 1, B).astype(np.int32) if ragged else np.full(B, cap, np.int32)
    lens[0] = cap
    print(f"[case] paged decode B{B} Hq{Hq} Hkv{Hkv} q_len{q_len} d{d} R{R} P{P} pages{npp} W{W}", flush=True)
    kc, ks = ops.quantize_qk(to_dev(k))
    vc, vs = ops.quantize_v(to_dev(v).reshape(B * Hkv, cap, d), R)
    vc, vs = vc.reshape(B, Hkv, cap, d), vs.reshape(B, Hkv, -1)
    # the cache codes are the oracle's own quantization, bit for bit
    rkc, rks = quant.quantize_qk(k)
    rvc, rvs = quant.quantize_v(v.reshape(B * Hkv, cap, d), R)
    rvc, rvs = rvc.reshape(B, Hkv, cap, d), rvs.reshape(B, Hkv, -1)
    assert np.array_equal(kc.cpu().numpy(), rkc) and np.array_equal(ks.cpu().numpy(), rks)
    assert np.array_equal(vc.cpu().numpy(), rvc) and np.array_equal(vs.cpu().numpy(), rvs)
    table = _table(B, npp, 5, seed=cap)
    pk, pks, pv = _to_pages(kc, table, P, P), _to_pages(ks, table, P, P), _to_pages(vc, table, P, P)
    pvs = _to_pages(vs, table, P, P // R)
    kl = torch.from_numpy(lens).cuda()
    bt = torch.from_numpy(table).cuda()
    qd = to_dev(q)
    o1, l1 = ops.attn_decode(qd, kc, ks, vc, vs, cap, v_tile_rows=R, kv_lens=kl, return_lse=True, window=W)
    o2, l2 = ops.attn_decode(qd, pk, pks, pv, pvs, cap, v_tile_rows=R, kv_lens=kl, return_lse=True, window=W,
                             block_table=bt, page_size=P)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the pages gather back into the oracle's cache, and the oracle on its
    # own codes gives the reference
    g = [ocache.gather_pages(t.cpu().numpy(), table, P) for t in (pk, pks, pv)]
    gvs = ocache.gather_pages(pvs.cpu().numpy(), table, P, rows_per_page=P // R)
    assert np.array_equal(g[0], rkc) and np.array_equal(g[1], rks) and np.array_equal(g[2], rvc)
    assert np.array_equal(gvs, rvs)
    ro, rl = oatt.qk4v8_decode(q, rkc, rks, rvc, rvs, lens, R, 1 / math.sqrt(d), window=W)
    assert_attn_close(from_dev_bf16(o2), ro, "paged decode")
    assert np.abs(l2.cpu().numpy() - rl).max() < 5e-3


APP_CASES = [
    # B, Hkv, d, R, P, pages per sequence, initial lengths, append sizes
    (2, 2, 128, 64, 128, 6, [0, 70], [1, 64, 3, 130, 1, 200]),
    (3, 2, 128, 256, 256, 3, [0, 5, 256], [1, 7, 255, 2, 100]),
    (2, 3, 64, 32, 128, 4, [31, 0], [1, 33, 64, 200]),
]


@pytest.mark.parametrize("B,Hkv,d,R,P,npp,init,chunks", APP_CASES)
def test_paged_append_equals_contiguous(gpu, B, Hkv, d, R, P, npp, init, chunks):
    """The same appends into a contiguous and a paged cache; the gathered pages
    equal the contiguous cache bit for bit, and equal the oracle's quantization
    of each whole sequence."""
    from bit_quantized_attention_online_amd import ops
    cap = npp * P
    total = max(init) + sum(chunks)
    assert total <= cap
    rng = np.random.default_rng(cap + R + d)
    k = synth.bf16_bits(rng.standard_normal((B, total, Hkv, d)).astype(np.float32))
    v = synth.bf16_bits((rng.standard_normal((B, total, Hkv, d)) * np.exp(rng.standard_normal((B, total, 1, 1))))
                        .astype(np.float32))
    print(f"[case] paged append B{B} Hkv{Hkv} d{d} R{R} P{P} pages{npp} init{init} chunks{chunks}", flush=True)
    dev = torch.device("cuda:0")
    table = _table(B, npp, 4, seed=cap + 1)
    bt = torch.from_numpy(table).to(dev)
    pages = int(table.max()) + 1 + 2
    cont = [torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device=dev),
            torch.zeros((B, Hkv, cap, d // 32), dtype=torch.uint8, device=dev),
            torch.zeros((B, Hkv, cap, d), dtype=torch.uint8, device=dev),
            torch.zeros((B, Hkv, cap // R), dtype=torch.uint8, device=dev)]
    pool = [torch.full((pages, Hkv, P, d // 2), 0xFF, dtype=torch.uint8, device=dev),
            torch.full((pages, Hkv, P, d // 32), 0xFF, dtype=torch.uint8, device=dev),
            torch.full((pages, Hkv, P, d), 0xFF, dtype=torch.uint8, device=dev),
            torch.full((pages, Hkv, P // R), 0xFF, dtype=torch.uint8, device=dev)]
    tails = [torch.zeros((B, Hkv, R, d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    lens = np.array(init, np.int32)
    kd, vd = to_dev(k), to_dev(v)
    # the initial rows, one sequence at a time (batch slices of the contiguous
    # cache; the whole pool with that sequence's table row), then the chunks
    for b in range(B):
        if lens[b]:
            kb, vb = kd[b:b + 1, :lens[b]], vd[b:b + 1, :lens[b]]
            ops.kv_append(kb, vb, *(x[b:b + 1] for x in cont), tails[0][b:b + 1], 0, v_tile_rows=R)
            ops.kv_append(kb, vb, *pool, tails[1][b:b + 1], 0, v_tile_rows=R, block_table=bt[b:b + 1], page_size=P)
    pos = lens.copy()
    for n in chunks:
        idx = torch.from_numpy(np.stack([np.arange(p, p + n) for p in pos])).to(dev)
        kn = torch.stack([kd[b, idx[b]] for b in range(B)])
        vn = torch.stack([vd[b, idx[b]] for b in range(B)])
        kl = torch.from_numpy(pos).to(dev)
        ops.kv_append(kn, vn, *cont, tails[0], 0, v_tile_rows=R, kv_lens=kl)
        ops.kv_append(kn, vn, *pool, tails[1], 0, v_tile_rows=R, kv_lens=kl, block_table=bt, page_size=P)
        pos += n
    torch.cuda.synchronize()
    assert torch.equal(tails[0], tails[1])
    got = [ocache.gather_pages(t.cpu().numpy(), table, P) for t in pool[:3]]
    got.append(ocache.gather_pages(pool[3].cpu().numpy(), table, P, rows_per_page=P // R))
    ref = [t.cpu().numpy() for t in cont]
    for b in range(B):
        n = pos[b]
        for h in range(Hkv):
            assert np.array_equal(got[0][b, h, :n], ref[0][b, h, :n]) and np.array_equal(got[1][b, h, :n], ref[1][b, h, :n])
            assert np.array_equal(got[2][b, h, :n], ref[2][b, h, :n])
            nt = -(-n // R)
            assert np.array_equal(got[3][b, h, :nt], ref[3][b, h, :nt])
            rkc, rks, rvc, rvs = ocache.cache_of_sequence(k[b, :n, h], v[b, :n, h], R)
            assert np.array_equal(got[0][b, h, :n], rkc) and np.array_equal(got[2][b, h, :n], rvc)
            assert np.array_equal(got[3][b, h, :nt], rvs)
