"""Seeded synthetic inputs for the QK4V8 workloads.

This module holds no arithmetic of the method: it only draws standard normal
numbers, rounds them to bfloat16 bit patterns, and applies the fixed input
structures of the workloads (outlier K channels, outlier K rows).  Both the
tests/bench (which feed the HIP path) and the CPU oracle consume its arrays.

The pages evaluate on long-context summarisation / QA at 4K-16K tokens and
beyond (MpFA page §4.3) and on 8-token block verification (MiMo page, section
"DFlash块扩散推测解码"); no dataset or model is available here, so seeded
normal tensors with those shapes stand in for them.

Every slice is drawn from ``numpy.random.default_rng([20261203, cfg,
tensor_id, b, h])`` so that one (batch, head) slice can be regenerated alone.
tensor_id: 0 = Q, 1 = K, 2 = V, 3 = outlier selection.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT_SEED = 20261203
Q_ID, K_ID, V_ID, OUTLIER_ID = 0, 1, 2, 3


def bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    one, half = np.uint32(1), np.uint32(0x7FFF)      # finite inputs: no uint32 overflow
    return ((u + half + ((u >> np.uint32(16)) & one)) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(cfg, tensor_id, b, h):
    return np.random.default_rng([ROOT_SEED, cfg, tensor_id, b, h])


def normal_bits(cfg, tensor_id, b, h, shape, scale=1.0):
    """One seeded slice of N(0, scale^2) values as bf16 bit patterns."""
    x = rng_for(cfg, tensor_id, b, h).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return bf16_bits(x)


def normal_tensor(cfg, tensor_id, B, H, n, d, scale=1.0, threads=8):
    """[B, H, n, d] bf16 bits, one independent seeded stream per (b, h)
    (slices are drawn in parallel threads; the result does not depend on it)."""
    out = np.empty((B, H, n, d), dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = normal_bits(cfg, tensor_id, b, h, (n, d), scale)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def normal_batch(cfg, tensor_id, b, H, n, d, threads=8):
    """[H, n, d] bf16 bits: the slices (b, 0..H-1) of ``normal_tensor``."""
    out = np.empty((H, n, d), dtype=np.uint16)

    def fill(h):
        out[h] = normal_bits(cfg, tensor_id, b, h, (n, d))

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(H)))
    return out


def scale_bits(bits, factor):
    """Multiply bf16 values by ``factor`` in float32 and re-round to bf16."""
    return bf16_bits(bits_to_f32(bits) * np.float32(factor))


def outlier_channels(cfg, b, h, d, count=4):
    """Distinct K channels (per KV head) that carry outliers."""
    return np.sort(rng_for(cfg, OUTLIER_ID, b, h).choice(d, count, replace=False))


def outlier_rows(cfg, b, h, n, frac=0.02):
    """Distinct K rows (per KV head) that carry outliers: round(frac * n)."""
    return np.sort(rng_for(cfg, OUTLIER_ID, b, h).choice(n, int(round(frac * n)), replace=False))


# ----------------------------------------------------------------------------
# The five workloads.  Shapes follow the configurations the pages' use cases
# imply (tiny correctness case, 4K causal GQA prefill with outlier channels,
# 32K decode over a quantized cache, 128K causal prefill with outlier rows,
# 8-token block verification over a 16K prefix).
# ----------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="tiny_full_b1_h1_n256_d64", kind="prefill", B=1, Hq=1, Hkv=1, Nq=256, Nk=256, d=64,
            causal=False, v_tile_rows=64),
    2: dict(name="causal_gqa_prefill_b4_hq32_hkv8_n4096_d128", kind="prefill", B=4, Hq=32, Hkv=8,
            Nq=4096, Nk=4096, d=128, causal=True, v_tile_rows=64, k_outlier_channels=4,
            k_outlier_factor=20.0),
    3: dict(name="decode_b64_hq64_hkv8_kv32768_d128", kind="decode", B=64, Hq=64, Hkv=8, q_len=1,
            kv_len=32768, d=128, v_tile_rows=256),
    4: dict(name="long_causal_prefill_b1_hq64_hkv8_n131072_d128", kind="prefill", B=1, Hq=64, Hkv=8,
            Nq=131072, Nk=131072, d=128, causal=True, v_tile_rows=64, k_outlier_row_frac=0.02,
            k_outlier_factor=10.0),
    5: dict(name="block_verify_b32_q8_prefix16384_hq64_hkv8_d128", kind="decode", B=32, Hq=64, Hkv=8,
            q_len=8, kv_len=16384 + 8, d=128, v_tile_rows=256),
}


def prefill_k_slice(cfg, w, b, h):
    """K for one (b, kv-head) with the workload's outlier structure."""
    k = normal_bits(cfg, K_ID, b, h, (w["Nk"], w["d"]))
    if "k_outlier_channels" in w:
        ch = outlier_channels(cfg, b, h, w["d"], w["k_outlier_channels"])
        k[:, ch] = scale_bits(k[:, ch], w["k_outlier_factor"])
    if "k_outlier_row_frac" in w:
        rows = outlier_rows(cfg, b, h, w["Nk"], w["k_outlier_row_frac"])
        k[rows, :] = scale_bits(k[rows, :], w["k_outlier_factor"])
    return k


def prefill_inputs(cfg, w=None):
    """(q [B,Hq,Nq,d], k [B,Hkv,Nk,d], v [B,Hkv,Nk,d]) bf16 bits."""
    w = w or WORKLOADS[cfg]
    q = normal_tensor(cfg, Q_ID, w["B"], w["Hq"], w["Nq"], w["d"])
    k = np.empty((w["B"], w["Hkv"], w["Nk"], w["d"]), dtype=np.uint16)
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            k[b, h] = prefill_k_slice(cfg, w, b, h)
    v = normal_tensor(cfg, V_ID, w["B"], w["Hkv"], w["Nk"], w["d"])
    return q, k, v


def decode_inputs(cfg, w=None):
    """(q [B, q_len, Hq, d], k [B,Hkv,kv_len,d], v [B,Hkv,kv_len,d]) bf16 bits;
    K and V are quantized into the cache by whoever consumes them."""
    w = w or WORKLOADS[cfg]
    q = normal_tensor(cfg, Q_ID, w["B"], w["Hq"], w["q_len"], w["d"]).transpose(0, 2, 1, 3).copy()
    k = normal_tensor(cfg, K_ID, w["B"], w["Hkv"], w["kv_len"], w["d"])
    v = normal_tensor(cfg, V_ID, w["B"], w["Hkv"], w["kv_len"], w["d"])
    return q, k, v
