"""Online per-block quantizers (oracle; test infrastructure only).

MpFA page §3.2: the scale is not calibrated ahead of time; it is computed at
run time from each block's extreme values as the block is loaded, and it holds
for that block only.  Read as the block's absolute maximum, because E2M1 and
E4M3 are sign-symmetric with no zero point.  MpFA page §2.1/§2.2: Q and K at 4
bits, V at 8 bits.  MiMo page, section "MXFP4专家量化": one scale per 32
elements.

Scale rule (OCP MX v1.0): X = floor(log2(amax)) - emax_elem, with emax = 2 for
E2M1 (largest magnitude 6 = 1.5 * 2**2) and emax = 8 for E4M3 (448 = 1.75 *
2**8); X is clamped to [-127, 127]; an all-zero block takes X = -127.  Elements
are divided by 2**X (exact: a power of two) and rounded RNE with saturation.
"""

import numpy as np

from .formats import (bf16_bits_to_float64, e2m1_decode, e2m1_encode,
                      e4m3_decode, e4m3_encode, e8m0_decode)

MX_BLOCK = 32
E2M1_EMAX = 2
E4M3_EMAX = 8


def shared_exponent(amax, emax_elem):
    """OCP MX shared exponent X for blocks with absolute maxima ``amax``
    (float64 array).  floor(log2(a)) is read exactly off frexp: a = f * 2**e
    with f in [0.5, 1) gives floor(log2(a)) = e - 1."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    x = (e.astype(np.int64) - 1) - emax_elem
    x = np.clip(x, -127, 127)
    return np.where(amax == 0.0, -127, x).astype(np.int64)


def quantize_qk(x_bits):
    """MXFP4-quantize bf16 rows along the last axis.

    x_bits: uint16 bf16 patterns, shape [..., d] with d % 32 == 0.
    Returns (codes uint8 [..., d/2], scales uint8 [..., d/32]); byte k of a
    row holds element 2k in its low nibble and element 2k+1 in its high
    nibble; a scale byte is X + 127.
    """
    return quantize_qk_values(bf16_bits_to_float64(x_bits))


def quantize_qk_values(x):
    """``quantize_qk`` of rows given as float64 values (here: exact float32
    values, e.g. rotated rows)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    X = shared_exponent(amax, E2M1_EMAX)
    y = np.ldexp(blocks, -X[..., None])
    codes = e2m1_encode(y).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def dequantize_qk(codes, scales):
    """MXFP4 codes/scales from ``quantize_qk`` -> float64 [..., d]."""
    codes = np.asarray(codes)
    lo = e2m1_decode(codes & 0xF)
    hi = e2m1_decode(codes >> 4)
    vals = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    d = vals.shape[-1]
    blocks = vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    return (blocks * e8m0_decode(scales)[..., None]).reshape(vals.shape)


def quantize_v(v_bits, tile_rows):
    """FP8 E4M3FN quantization with one E8M0 scale per tile of rows.

    v_bits: uint16 bf16 patterns [groups, n, d] (a group is one
    (batch, kv-head) pair).  Tiles are rows [t*R, min((t+1)*R, n)); the last
    tile may be shorter.  Returns (codes uint8 [groups, n, d],
    scales uint8 [groups, ceil(n / R)]).
    """
    v = bf16_bits_to_float64(v_bits)
    g, n, d = v.shape
    n_tiles = -(-n // tile_rows)
    codes = np.zeros((g, n, d), dtype=np.uint8)
    scales = np.zeros((g, n_tiles), dtype=np.uint8)
    for t in range(n_tiles):
        rows = slice(t * tile_rows, min((t + 1) * tile_rows, n))
        tile = v[:, rows, :]
        amax = np.abs(tile).reshape(g, -1).max(axis=1)
        X = shared_exponent(amax, E4M3_EMAX)
        codes[:, rows, :] = e4m3_encode(np.ldexp(tile, -X[:, None, None]))
        scales[:, t] = (X + 127).astype(np.uint8)
    return codes, scales


def dequantize_v(codes, scales, tile_rows):
    """FP8 codes [groups, n, d] + per-tile scales -> float64 [groups, n, d]."""
    codes = np.asarray(codes)
    g, n, d = codes.shape
    row_scale = e8m0_decode(scales)[:, np.arange(n) // tile_rows]   # [g, n]
    return e4m3_decode(codes) * row_scale[:, :, None]


def hadamard_rows_f32(x_bits):
    """Sylvester-Hadamard transform y = H_d x of bf16 rows along the last axis
    (d a power of two; H has +-1 entries, H_2n = [[H_n, H_n], [H_n, -H_n]]),
    evaluated in float32 with the butterfly stages in the order h = 1, 2, 4,
    ..., d/2: (x_i, x_{i+h}) -> (x_i + x_{i+h}, x_i - x_{i+h}) for i & h == 0.
    Every float32 operation is fixed by this order, so the result is exact to
    the bit.  MpFA page §3.1: a rotation spreads the energy of outlier
    channels over all channels before the 4-bit quantization; H H^T = d I, so
    (H q).(H k) = d (q.k) and only the quantization error changes."""
    x = bf16_bits_to_float64(x_bits).astype(np.float32)
    d = x.shape[-1]
    assert d > 0 and d & (d - 1) == 0
    h = 1
    while h < d:
        y = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :], y[..., 1, :]
        x = np.stack([a + b, a - b], axis=-2).reshape(x.shape)
        h *= 2
    return x


def quantize_qk_hadamard(x_bits):
    """MXFP4 of the rotated rows H_d x (``hadamard_rows_f32``)."""
    return quantize_qk_values(hadamard_rows_f32(x_bits).astype(np.float64))
