"""Quantized KV cache of a token sequence (oracle; test infrastructure only).

MpFA page §6.1: the KV cache is kept quantized; §3.2: each block's scale is
computed from the block itself.  A cache filled by successive appends is
therefore defined as the quantization of the whole sequence so far: each K row
MXFP4-quantized on its own, and each V tile of R rows (the last one possibly
partial) FP8-quantized with the scale of all the rows it holds.
"""

from .quant import quantize_qk, quantize_qk_hadamard, quantize_v


def cache_of_sequence(k_bits, v_bits, tile_rows, hadamard=False):
    """k_bits, v_bits: uint16 bf16 patterns [n, d] of one (batch, kv-head).
    Returns (k_codes [n, d/2], k_scales [n, d/32], v_codes [n, d],
    v_scales [ceil(n / tile_rows)]).  With ``hadamard`` the K rows are
    rotated before quantization (``quant.quantize_qk_hadamard``)."""
    kc, ks = quantize_qk_hadamard(k_bits) if hadamard else quantize_qk(k_bits)
    vc, vs = quantize_v(v_bits[None], tile_rows)
    return kc, ks, vc[0], vs[0]
