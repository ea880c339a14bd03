"""Quantized KV cache of a token sequence (oracle; test infrastructure only).

MpFA page §6.1: the KV cache is kept quantized; §3.2: each block's scale is
computed from the block itself.  A cache filled by successive appends is
therefore defined as the quantization of the whole sequence so far: each K row
MXFP4-quantized on its own, and each V tile of R rows (the last one possibly
partial) FP8-quantized with the scale of all the rows it holds.

A paged cache holds the same rows in fixed-size pages named by a block table
(the common serving layout); ``gather_pages`` spells out its addressing.
"""

import numpy as np

from .quant import quantize_qk, quantize_qk_hadamard, quantize_v


def cache_of_sequence(k_bits, v_bits, tile_rows, hadamard=False):
    """k_bits, v_bits: uint16 bf16 patterns [n, d] of one (batch, kv-head).
    Returns (k_codes [n, d/2], k_scales [n, d/32], v_codes [n, d],
    v_scales [ceil(n / tile_rows)]).  With ``hadamard`` the K rows are
    rotated before quantization (``quant.quantize_qk_hadamard``)."""
    kc, ks = quantize_qk_hadamard(k_bits) if hadamard else quantize_qk(k_bits)
    vc, vs = quantize_v(v_bits[None], tile_rows)
    return kc, ks, vc[0], vs[0]


def gather_pages(pool, block_table, page_size, rows_per_page=None):
    """The contiguous cache a paged cache stands for: key j of sequence b lives
    in slot j % P of page block_table[b, j // P] (P = page_size keys per page,
    or rows_per_page entries per page for per-tile arrays such as the V
    scales).  pool: [pages, kv_heads, P, ...] -> [batch, kv_heads, pages_per_seq * P, ...]."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    B, npp = bt.shape
    per = rows_per_page if rows_per_page is not None else page_size
    out = np.empty((B, pool.shape[1], npp * per) + pool.shape[3:], dtype=pool.dtype)
    for b in range(B):
        for i in range(npp):
            out[b, :, i * per:(i + 1) * per] = pool[bt[b, i]]
    return out
