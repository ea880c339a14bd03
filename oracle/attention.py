"""Attention on dequantized operands, exactly in float64 (oracle; test
infrastructure only).

MpFA page §2.3/§3.3: attention on 4-bit Q/K and 8-bit V with an FP32
accumulator and an online softmax whose result is, up to rounding, the plain
softmax attention of the dequantized operands.  The oracle therefore evaluates
that plain definition exactly in float64 and does not model any kernel-side
rounding of the probabilities:

    s_ij = sigma * sum_c q_ic k_jc          (sigma: the call's fp32 scale)
    mask (causal): keep j <= i + (Nk - Nq)  (bottom-right alignment)
    p_ij = exp(s_ij - max_j s_ij)
    o_i  = sum_j p_ij v_j / sum_j p_ij
    lse_i = max_j s_ij + ln(sum_j p_ij)     (natural log)

GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
Sliding window (MiMo page, section "DFlash块扩散推测解码": the drafter attends
only to the most recent 1024 tokens): with a window W > 0, row i additionally
drops keys j <= i + (Nk - Nq) - W, i.e. it sees at most the W most recent keys
up to and including its own position.
Decode / block verify (MiMo page, section "DFlash块扩散推测解码": the backbone
checks a drafted block of q_len tokens in one pass) is the same definition with
Nq = q_len queries placed at the end of an Nk-long sequence, i.e. the causal
bottom-right mask.
"""

import numpy as np

from .formats import e4m3_decode, e4m3_encode
from .quant import dequantize_qk, dequantize_v, quantize_qk, quantize_qk_hadamard, quantize_v

_CHUNK_ELEMS = 1 << 25


def _visible(cols, limits, lows):
    return (cols[None, :] <= limits[:, None]) & (cols[None, :] >= lows[:, None])


def _rows_attention(q, k, v, sigma, limits, lows):
    """q [R, d], k/v [Nk, d] float64; row r sees keys lows[r] <= j <= limits[r].
    Returns (o [R, d], lse [R])."""
    s = sigma * (q @ k.T)
    cols = np.arange(k.shape[0])
    s = np.where(_visible(cols, limits, lows), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    return o, m + np.log(l)


def _limits(pos, Nq, Nk, causal, window):
    limits = pos + (Nk - Nq) if causal else np.full(len(pos), Nk - 1)
    lows = limits - window + 1 if window else np.zeros(len(pos), dtype=np.int64)
    return limits, lows


def attention(q, k, v, softmax_scale, causal, rows=None, window=0):
    """Exact float64 attention (``window`` > 0: sliding window, causal only).

    q: [B, Hq, Nq, d]  (or [B, Hq, R, d] when ``rows`` selects R query
       positions out of Nq = rows_total, see below)
    k, v: [B, Hkv, Nk, d]
    rows: optional (positions int array [R], Nq) - evaluate only those query
       positions of an Nq-long query sequence; q then holds just those rows.
    Returns (o [B, Hq, R, d], lse [B, Hq, R]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, R, d = q.shape
    _, Hkv, Nk, _ = k.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if rows is None:
        pos, Nq = np.arange(R), R
    else:
        pos, Nq = np.asarray(rows[0]), rows[1]
    sigma = float(np.float32(softmax_scale))
    assert not window or causal
    limits, lows = _limits(pos, Nq, Nk, causal, window)
    o = np.zeros((B, Hq, R, d))
    lse = np.zeros((B, Hq, R))
    step = max(1, _CHUNK_ELEMS // max(Nk, 1))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, R, step):
                sl = slice(r0, min(R, r0 + step))
                o[b, h, sl], lse[b, h, sl] = _rows_attention(q[b, h, sl], k[b, g], v[b, g], sigma, limits[sl],
                                                             lows[sl])
    return o, lse


def probabilities(q, k, softmax_scale, causal):
    """Softmax matrix P [B, Hq, Nq, Nk] of the same definition (for tests)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sigma = float(np.float32(softmax_scale))
    out = np.zeros((B, Hq, Nq, Nk))
    limits = np.arange(Nq) + (Nk - Nq) if causal else np.full(Nq, Nk - 1)
    cols = np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            s = sigma * (q[b, h] @ k[b, h // G].T)
            s = np.where(cols[None, :] <= limits[:, None], s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h] = p / p.sum(axis=1, keepdims=True)
    return out


def qk4v8_prefill(q_bits, k_bits, v_bits, softmax_scale, causal, v_tile_rows, rows=None, window=0):
    """The whole QK4V8 prefill on the CPU: MXFP4 Q and K, per-tile FP8 V,
    then exact attention of the dequantized operands.

    q_bits [B, Hq, Nq, d] (or the selected rows, see ``attention``),
    k_bits / v_bits [B, Hkv, Nk, d]: uint16 bf16 patterns.
    Returns (o, lse) float64.
    """
    qh = dequantize_qk(*quantize_qk(q_bits))
    kh = dequantize_qk(*quantize_qk(k_bits))
    B, Hkv, Nk, d = v_bits.shape
    vc, vs = quantize_v(v_bits.reshape(B * Hkv, Nk, d), v_tile_rows)
    vh = dequantize_v(vc, vs, v_tile_rows).reshape(B, Hkv, Nk, d)
    return attention(qh, kh, vh, softmax_scale, causal, rows=rows, window=window)


def qk4v8_decode(q_bits, k_codes, k_scales, v_codes, v_scales, kv_lens, v_tile_rows, softmax_scale, window=0):
    """QK4V8 decode / block verify over a quantized cache.

    q_bits: uint16 [B, q_len, Hq, d]; caches: k_codes [B, Hkv, cap, d/2],
    k_scales [B, Hkv, cap, d/32], v_codes [B, Hkv, cap, d],
    v_scales [B, Hkv, ceil(cap / v_tile_rows)]; kv_lens: int [B].
    Query t of a block sees keys j <= kv_len - q_len + t.
    Returns (o [B, q_len, Hq, d], lse [B, q_len, Hq]) float64.
    """
    B, q_len, Hq, d = q_bits.shape
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    qh = dequantize_qk(*quantize_qk(q_bits)).transpose(0, 2, 1, 3)   # [B, Hq, q_len, d]
    o = np.zeros((B, q_len, Hq, d))
    lse = np.zeros((B, q_len, Hq))
    for b in range(B):
        n = int(kv_lens[b])
        kh = dequantize_qk(k_codes[b, :, :n], k_scales[b, :, :n])
        vh = dequantize_v(v_codes[b, :, :n], v_scales[b], v_tile_rows)
        ob, lb = attention(qh[b:b + 1], kh[None], vh[None], softmax_scale, causal=True, window=window)
        o[b] = ob[0].transpose(1, 0, 2)
        lse[b] = lb[0].T
    return o, lse


# ---------------------------------------------------------------------------
# Single-term FP8 probabilities (the library's fast mode).
#
# P·V on FP8 (E4M3) with one term per probability.  Its definition does not
# depend on how keys are tiled: with base-2 scores t_ij = s_ij * log2(e), the
# keys of a row are grouped in aligned blocks of 32 (key indices [32a, 32a +
# 32), the MX block size of the MiMo page's section "MXFP4专家量化"), each block
# gets the range exponent X = floor(max_j t_ij) - 7 over its visible keys (an
# E8M0 scale, as in MX), and each weight is rounded to E4M3 on that range:
#     p~_ij = 2^X * E4M3_RNE(2^(t_ij - X))       (2^(t - X) < 256, no saturation)
#     o_i   = sum_j p~_ij v_j / sum_j p~_ij,   lse_i = ln(sum_j p~_ij)
# A common factor 2^M per row (M any integer) cancels in o and is added back
# in lse.  The two-term FP8 split of the default path is a kernel rounding
# detail below the gate and is not modelled here (see ``attention``).
# ---------------------------------------------------------------------------

FAST_P_BLOCK = 32
FAST_P_HEADROOM = 7
_LOG2E = 1.4426950408889634


def _rows_attention_fast(q, k, v, sigma, limits, lows):
    s = sigma * (q @ k.T)
    Nk = k.shape[0]
    cols = np.arange(Nk)
    t = np.where(_visible(cols, limits, lows), s * _LOG2E, -np.inf)
    M = np.floor(t.max(axis=1))                                  # common integer shift per row
    t = t - M[:, None]
    nb = -(-Nk // FAST_P_BLOCK)
    tp = np.full((t.shape[0], nb * FAST_P_BLOCK), -np.inf)
    tp[:, :Nk] = t
    tb = tp.reshape(t.shape[0], nb, FAST_P_BLOCK)
    bmax = tb.max(axis=2)
    X = np.where(np.isfinite(bmax), np.floor(bmax) - FAST_P_HEADROOM, 0.0)
    y = np.exp2(tb - X[:, :, None])                              # 0 for masked keys
    p = e4m3_decode(e4m3_encode(y)) * np.exp2(X)[:, :, None]
    p = p.reshape(t.shape[0], nb * FAST_P_BLOCK)[:, :Nk]
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    return o, (M + np.log2(l)) * np.log(2.0)


def attention_fast_p(q, k, v, softmax_scale, causal, rows=None, window=0):
    """Attention with single-term E4M3 probabilities (definition above);
    same arguments and returns as ``attention``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, R, d = q.shape
    _, Hkv, Nk, _ = k.shape
    G = Hq // Hkv
    if rows is None:
        pos, Nq = np.arange(R), R
    else:
        pos, Nq = np.asarray(rows[0]), rows[1]
    sigma = float(np.float32(softmax_scale))
    assert not window or causal
    limits, lows = _limits(pos, Nq, Nk, causal, window)
    o = np.zeros((B, Hq, R, d))
    lse = np.zeros((B, Hq, R))
    step = max(1, _CHUNK_ELEMS // max(Nk, 1))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, R, step):
                sl = slice(r0, min(R, r0 + step))
                o[b, h, sl], lse[b, h, sl] = _rows_attention_fast(q[b, h, sl], k[b, h // G], v[b, h // G], sigma,
                                                                  limits[sl], lows[sl])
    return o, lse


def qk4v8_prefill_fast(q_bits, k_bits, v_bits, softmax_scale, causal, v_tile_rows, rows=None, window=0):
    """``qk4v8_prefill`` with single-term FP8 probabilities."""
    qh = dequantize_qk(*quantize_qk(q_bits))
    kh = dequantize_qk(*quantize_qk(k_bits))
    B, Hkv, Nk, d = v_bits.shape
    vc, vs = quantize_v(v_bits.reshape(B * Hkv, Nk, d), v_tile_rows)
    vh = dequantize_v(vc, vs, v_tile_rows).reshape(B, Hkv, Nk, d)
    return attention_fast_p(qh, kh, vh, softmax_scale, causal, rows=rows, window=window)


# ---------------------------------------------------------------------------
# Hadamard-rotated Q and K (MpFA page §3.1).  Q and K rows are rotated by the
# Sylvester-Hadamard matrix H_d (``quant.hadamard_rows_f32``) before MXFP4;
# since (H q).(H k) = d (q.k), the scores are scaled by softmax_scale / d
# (exact: d is a power of two).  V is unchanged.
# ---------------------------------------------------------------------------

def qk4v8_prefill_hadamard(q_bits, k_bits, v_bits, softmax_scale, causal, v_tile_rows, rows=None, window=0):
    """``qk4v8_prefill`` with rotated Q and K."""
    d = q_bits.shape[-1]
    qh = dequantize_qk(*quantize_qk_hadamard(q_bits))
    kh = dequantize_qk(*quantize_qk_hadamard(k_bits))
    B, Hkv, Nk, _ = v_bits.shape
    vc, vs = quantize_v(v_bits.reshape(B * Hkv, Nk, d), v_tile_rows)
    vh = dequantize_v(vc, vs, v_tile_rows).reshape(B, Hkv, Nk, d)
    return attention(qh, kh, vh, float(np.float32(softmax_scale)) / d, causal, rows=rows, window=window)


def qk4v8_decode_hadamard(q_bits, k_codes, k_scales, v_codes, v_scales, kv_lens, v_tile_rows, softmax_scale,
                          window=0):
    """``qk4v8_decode`` over a cache whose K rows were rotated before
    quantization; the queries are rotated the same way."""
    B, q_len, Hq, d = q_bits.shape
    qh = dequantize_qk(*quantize_qk_hadamard(q_bits)).transpose(0, 2, 1, 3)
    o = np.zeros((B, q_len, Hq, d))
    lse = np.zeros((B, q_len, Hq))
    for b in range(B):
        n = int(kv_lens[b])
        kh = dequantize_qk(k_codes[b, :, :n], k_scales[b, :, :n])
        vh = dequantize_v(v_codes[b, :, :n], v_scales[b], v_tile_rows)
        ob, lb = attention(qh[b:b + 1], kh[None], vh[None], float(np.float32(softmax_scale)) / d, causal=True,
                           window=window)
        o[b] = ob[0].transpose(1, 0, 2)
        lse[b] = lb[0].T
    return o, lse
