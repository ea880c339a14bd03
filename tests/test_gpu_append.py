"""GPU KV-cache append vs the oracle.  After every append the cache is
bit-identical to the quantization of each whole sequence so far (K rows MXFP4,
V tiles FP8 with the scale of all their rows), the tail buffer holds the
source rows of each sequence's partial V tile, and sequences that do not fit
the capacity are left untouched."""
import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from oracle import cache as ocache
from tests._util import to_dev

pytestmark = pytest.mark.gpu


def _sequences(B, n, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    # scale changes inside tiles: a few large rows (the tile's scale grows after
    # smaller rows were encoded), a few small ones, and all-zero rows
    for b in range(B):
        for pos, f in ((3, 0.01), (40, 30.0), (97, 1e-3), (300, 50.0), (301, 0.0), (450, 200.0)):
            if pos < n:
                v[b, pos] *= f
                k[b, pos] *= f
        v[b, 5:9] = 0.0
    return synth.bf16_bits(k), synth.bf16_bits(v)


def _check(kc, ks, vc, vs, tail, k_bits, v_bits, lens, R):
    kc, ks, vc, vs = (t.cpu().numpy() for t in (kc, ks, vc, vs))
    tail = tail.view(torch.int16).cpu().numpy().view(np.uint16)
    B, Hkv = kc.shape[:2]
    for b in range(B):
        n = lens[b]
        for h in range(Hkv):
            rkc, rks, rvc, rvs = ocache.cache_of_sequence(k_bits[b, :n, h], v_bits[b, :n, h], R)
            assert np.array_equal(kc[b, h, :n], rkc), (b, h, n, "K codes")
            assert np.array_equal(ks[b, h, :n], rks), (b, h, n, "K scales")
            assert np.array_equal(vc[b, h, :n], rvc), (b, h, n, "V codes")
            assert np.array_equal(vs[b, h, :len(rvs)], rvs), (b, h, n, "V scales")
            t0 = (n // R) * R
            assert np.array_equal(tail[b, h, :n - t0], v_bits[b, t0:n, h]), (b, h, n, "tail")


CASES = [
    # B, Hkv, d, R, cap, initial lengths, append sizes (one per call, all sequences)
    (3, 2, 128, 256, 700, [0, 5, 256], [1, 7, 1, 64, 130, 3, 200, 1, 300]),
    (2, 2, 128, 64, 520, [63, 64], [1, 1, 65, 8, 128, 0, 256]),
    (2, 3, 64, 32, 300, [0, 31], [33, 1, 2, 64, 31, 1]),
    (1, 8, 128, 128, 1000, [0], [1] * 5 + [8] * 3 + [127, 129]),
]


@pytest.mark.parametrize("B,Hkv,d,R,cap,init,chunks", CASES)
def test_append_matches_whole_sequence_quantization(gpu, B, Hkv, d, R, cap, init, chunks):
    from bit_quantized_attention_online_amd import ops
    print(f"[case] append B{B} Hkv{Hkv} d{d} R{R} cap{cap} init{init} chunks{chunks}", flush=True)
    k_bits, v_bits = _sequences(B, cap, Hkv, d, seed=B * 100 + d + R)
    dev = torch.device("cuda:0")
    kc = torch.full((B, Hkv, cap, d // 2), 0xAB, dtype=torch.uint8, device=dev)
    ks = torch.full((B, Hkv, cap, d // 32), 0xAB, dtype=torch.uint8, device=dev)
    vc = torch.full((B, Hkv, cap, d), 0xAB, dtype=torch.uint8, device=dev)
    vs = torch.full((B, Hkv, -(-cap // R)), 0xAB, dtype=torch.uint8, device=dev)
    tail = torch.zeros((B, Hkv, R, d), dtype=torch.bfloat16, device=dev)
    lens = [0] * B
    # ragged starting lengths: append each sequence's prefix on its own batch slice
    for b, n0 in enumerate(init):
        if n0:
            ops.kv_append(to_dev(k_bits[b:b + 1, :n0]), to_dev(v_bits[b:b + 1, :n0]), kc[b:b + 1], ks[b:b + 1],
                          vc[b:b + 1], vs[b:b + 1], tail[b:b + 1], 0, v_tile_rows=R)
            lens[b] = n0
    torch.cuda.synchronize()
    _check(kc, ks, vc, vs, tail, k_bits, v_bits, lens, R)
    for c in chunks:
        knew = np.zeros((B, c, Hkv, d), dtype=np.uint16)
        vnew = np.zeros((B, c, Hkv, d), dtype=np.uint16)
        for b in range(B):
            m = min(c, cap - lens[b])
            knew[b, :m] = k_bits[b, lens[b]:lens[b] + m]
            vnew[b, :m] = v_bits[b, lens[b]:lens[b] + m]
        kl = torch.tensor(lens, dtype=torch.int32, device=dev)
        before = [t.clone() for t in (kc, ks, vc, vs, tail)]
        ops.kv_append(to_dev(knew), to_dev(vnew), kc, ks, vc, vs, tail, 0, v_tile_rows=R, kv_lens=kl)
        torch.cuda.synchronize()
        for b in range(B):
            if lens[b] + c <= cap:
                lens[b] += c
            else:   # does not fit: the sequence must be untouched
                for t0, t1 in zip(before, (kc, ks, vc, vs, tail)):
                    assert torch.equal(t0[b], t1[b]), ("overflowing sequence modified", b, c)
        _check(kc, ks, vc, vs, tail, k_bits, v_bits, lens, R)
    print(f"[parity] append: final lengths {lens} bit-exact", flush=True)


def test_append_strided_inputs_and_decode(gpu):
    """Token-major new K/V taken as strided views, then decode over the appended
    cache equals decode over a cache quantized in one go."""
    from bit_quantized_attention_online_amd import ops
    B, Hkv, Hq, d, R, cap = 2, 2, 8, 128, 256, 600
    k_bits, v_bits = _sequences(B, cap, Hkv, d, seed=7)
    dev = torch.device("cuda:0")
    # the unused part of the cache holds NaN patterns (E4M3 0xFF, E8M0 0xFF):
    # decode must not let them reach the output
    kc = torch.full((B, Hkv, cap, d // 2), 0xFF, dtype=torch.uint8, device=dev)
    ks = torch.full((B, Hkv, cap, d // 32), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full((B, Hkv, cap, d), 0xFF, dtype=torch.uint8, device=dev)
    vs = torch.full((B, Hkv, -(-cap // R)), 0xFF, dtype=torch.uint8, device=dev)
    tail = torch.zeros((B, Hkv, R, d), dtype=torch.bfloat16, device=dev)
    # [B, n, Hkv, 2d] storage, the first d columns used: head stride 2d
    big_k = torch.zeros((B, cap, Hkv, 2 * d), dtype=torch.bfloat16, device=dev)
    big_v = torch.zeros((B, cap, Hkv, 2 * d), dtype=torch.bfloat16, device=dev)
    big_k[..., :d] = to_dev(k_bits)
    big_v[..., :d] = to_dev(v_bits)
    n = 0
    for c in (100, 1, 250, 49, 8):
        ops.kv_append(big_k[:, n:n + c, :, :d], big_v[:, n:n + c, :, :d], kc, ks, vc, vs, tail, n, v_tile_rows=R)
        n += c
    torch.cuda.synchronize()
    _check(kc, ks, vc, vs, tail, k_bits, v_bits, [n] * B, R)
    rng = np.random.default_rng(3)
    q = to_dev(synth.bf16_bits(rng.standard_normal((B, 1, Hq, d)).astype(np.float32)))
    o1 = ops.attn_decode(q, kc, ks, vc, vs, n, v_tile_rows=R)
    kc2, ks2 = ops.quantize_qk(to_dev(np.ascontiguousarray(k_bits[:, :n].transpose(0, 2, 1, 3))))
    vc2, vs2 = ops.quantize_v(to_dev(np.ascontiguousarray(v_bits[:, :n].transpose(0, 2, 1, 3))).reshape(B * Hkv, n, d), R)
    o2 = ops.attn_decode(q, kc2, ks2, vc2.reshape(B, Hkv, n, d), vs2.reshape(B, Hkv, -1), n, v_tile_rows=R)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2)
    print("[parity] append + decode equals one-shot quantization + decode", flush=True)


@pytest.mark.parametrize("d,R", [(128, 256), (64, 64)])
def test_append_hadamard_rotated_k_is_bit_exact(gpu, d, R):
    """K rows rotated by H_d in fp32 (fixed butterfly order) before MXFP4: the
    cache codes equal the oracle's to the bit."""
    from bit_quantized_attention_online_amd import ops
    B, Hkv, cap = 2, 3, 300
    k_bits, v_bits = _sequences(B, cap, Hkv, d, seed=d + 5)
    dev = torch.device("cuda:0")
    kc = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B, Hkv, cap, d // 32), dtype=torch.uint8, device=dev)
    vc = torch.zeros((B, Hkv, cap, d), dtype=torch.uint8, device=dev)
    vs = torch.zeros((B, Hkv, -(-cap // R)), dtype=torch.uint8, device=dev)
    tail = torch.zeros((B, Hkv, R, d), dtype=torch.bfloat16, device=dev)
    n = 0
    for c in (1, 77, 150, 2):
        ops.kv_append(to_dev(k_bits[:, n:n + c]), to_dev(v_bits[:, n:n + c]), kc, ks, vc, vs, tail, n,
                      v_tile_rows=R, hadamard=True)
        n += c
    torch.cuda.synchronize()
    kcn, ksn, vcn, vsn = (t.cpu().numpy() for t in (kc, ks, vc, vs))
    for b in range(B):
        for h in range(Hkv):
            rkc, rks, rvc, rvs = ocache.cache_of_sequence(k_bits[b, :n, h], v_bits[b, :n, h], R, hadamard=True)
            assert np.array_equal(kcn[b, h, :n], rkc) and np.array_equal(ksn[b, h, :n], rks), (b, h)
            assert np.array_equal(vcn[b, h, :n], rvc) and np.array_equal(vsn[b, h, :len(rvs)], rvs), (b, h)
    print(f"[parity] rotated K append d{d}: bit-exact", flush=True)
