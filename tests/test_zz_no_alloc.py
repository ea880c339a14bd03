"""qk4v8_attn_decode_noalloc (split partials in the library's fixed per-GPU
array, no allocation) against qk4v8_attn_decode with a caller workspace: the
same kernels, so the same bits, on two calls in a row (the second smaller)."""
import math

import numpy as np
import pytest
import torch

from bit_quantized_attention_online_amd import synth
from tests._util import to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, q_len, kv_len, d, R, seed):
    from bit_quantized_attention_online_amd import ops
    rng = np.random.default_rng(seed)
    k = synth.bf16_bits(rng.standard_normal((B, Hkv, kv_len, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((B, Hkv, kv_len, d)).astype(np.float32))
    q = synth.bf16_bits(rng.standard_normal((B, q_len, Hq, d)).astype(np.float32))
    kc, ks = ops.quantize_qk(to_dev(k))
    vc, vs = ops.quantize_v(to_dev(v).reshape(B * Hkv, kv_len, d), R)
    lens = torch.from_numpy(rng.integers(q_len, kv_len + 1, B).astype(np.int32)).cuda()
    return to_dev(q), kc, ks, vc.reshape(B, Hkv, kv_len, d), vs.reshape(B, Hkv, -1), lens


def _both(args, kv_len, R, splits):
    from bit_quantized_attention_online_amd import ops
    q, kc, ks, vc, vs, lens = args
    ref, ref_l = ops.attn_decode(q, kc, ks, vc, vs, kv_len, v_tile_rows=R, kv_lens=lens, num_splits=splits,
                                 return_lse=True, softmax_scale=1 / math.sqrt(q.shape[-1]))
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    ops.attn_decode_noalloc(q, kc, ks, vc, vs, kv_len, out, lse=lse, v_tile_rows=R, kv_lens=lens,
                            num_splits=splits, softmax_scale=1 / math.sqrt(q.shape[-1]))
    torch.cuda.synchronize()
    return ref, ref_l, out, lse


@pytest.mark.parametrize("splits", [0, 4])
def test_noalloc_decode_matches_workspace_decode(gpu, splits):
    big = (8, 64, 8, 8, 4096, 128, 256)          # block verify shape: 64 rows per KV head
    small = (2, 8, 2, 1, 700, 128, 64)           # decode shape, fewer partial rows
    for i, (B, Hq, Hkv, q_len, kv_len, d, R) in enumerate((big, small)):
        print(f"[case] noalloc call {i}: B{B} Hq{Hq} Hkv{Hkv} q_len{q_len} kv_len{kv_len} splits={splits}",
              flush=True)
        args = _case(B, Hq, Hkv, q_len, kv_len, d, R, seed=100 + i)
        ref, ref_l, out, lse = _both(args, kv_len, R, splits)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, ref_l)


def test_noalloc_rejects_partials_beyond_the_array(gpu):
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, q_len, kv_len, d = 64, 64, 8, 8, 4096, 128
    q = torch.zeros((B, q_len, Hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, kv_len, d // 2), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Hkv, kv_len, d // 32), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((B, Hkv, kv_len, d), dtype=torch.uint8, device="cuda")
    vs = torch.zeros((B, Hkv, kv_len // 256), dtype=torch.uint8, device="cuda")
    need = ops.decode_workspace_bytes(q, kc, kv_len, 256, num_splits=16)
    assert need > ops.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ops.QK4V8Error) as e:
        ops.attn_decode_noalloc(q, kc, ks, vc, vs, kv_len, torch.empty_like(q), num_splits=16)
    assert e.value.status == 5


@pytest.mark.parametrize("shape", [(8, 64, 8, 1, 4096, 128, 256),    # decode: 2 splits, partials and the merge
                                   (4, 64, 8, 8, 3000, 128, 256)])   # block verify: one split, direct output
def test_noalloc_decode_replays_under_graph_capture(gpu, shape):
    """The allocation-free call captured into a HIP graph, as a serving loop
    that cannot allocate would run it: every replay, with eager work and a
    synchronization before each, writes the eager call's bits."""
    from bit_quantized_attention_online_amd import ops
    B, Hq, Hkv, q_len, kv_len, d, R = shape
    print(f"[case] noalloc graph capture B{B} Hq{Hq} Hkv{Hkv} q_len{q_len} kv_len{kv_len}", flush=True)
    q, kc, ks, vc, vs, lens = _case(B, Hq, Hkv, q_len, kv_len, d, R, seed=300 + q_len)
    kw = dict(v_tile_rows=R, kv_lens=lens, softmax_scale=1 / math.sqrt(d))
    ref = torch.empty_like(q)
    ops.attn_decode_noalloc(q, kc, ks, vc, vs, kv_len, ref, **kw)
    out = torch.full_like(q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.attn_decode_noalloc(q, kc, ks, vc, vs, kv_len, out, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.attn_decode_noalloc(q, kc, ks, vc, vs, kv_len, out, **kw)
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
