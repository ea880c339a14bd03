"""Element and scale formats (oracle; test infrastructure only).

MXFP4 as the MiMo page's section "MXFP4专家量化" names it: FP4 elements, one
shared scale per 32 elements.  The bit layouts are the OCP MX v1.0 ones:

* E2M1 element: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
  Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  No Inf/NaN.
* E8M0 scale: an unsigned byte b meaning 2**(b - 127); 0xFF is NaN and is
  never produced here.
* E4M3FN element (OCP OFP8, the "FP8 E4M3" that keeps V at 8 bits per the MpFA
  page §2.2): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN; no Inf;
  largest finite magnitude 448.

Encoding = round to nearest, ties to the even code, after clamping the
magnitude to the largest finite value (saturation).  Written as a nearest-value
search over the table of representable magnitudes, which is the definition of
round-to-nearest.
"""

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_decode(codes):
    """E2M1 4-bit codes (any integer array, values 0..15) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def _e4m3_magnitude_table():
    # codes 0x00..0x7E are the finite non-negative values, increasing with code
    vals = np.zeros(127)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_MAGNITUDES = _e4m3_magnitude_table()


def e4m3_decode(codes):
    """E4M3FN byte codes -> float64 (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(codes).astype(np.int64)
    mag_code = c & 0x7F
    mag = np.where(mag_code == 0x7F, np.nan, E4M3_MAGNITUDES[np.minimum(mag_code, 126)])
    return np.where((c & 0x80) != 0, -mag, mag)


def e8m0_decode(scales):
    """E8M0 scale bytes -> float64 powers of two."""
    b = np.asarray(scales).astype(np.int64)
    return np.ldexp(1.0, b - 127)


def _rne_index(mag, table):
    """Index of the nearest entry of the increasing ``table`` to each value of
    ``mag`` (0 <= mag <= table[-1]); an exact tie picks the even index."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(table, mag, side="left")          # table[hi-1] < mag <= table[hi]
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e2m1_encode(y):
    """Round float64 ``y`` to E2M1 (RNE, saturating at 6).  The sign bit
    follows the sign of ``y``, including -0.0 and values that round to zero."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), E2M1_MAX)
    code = _rne_index(mag, E2M1_MAGNITUDES).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x8, code).astype(np.uint8)


def e4m3_encode(y):
    """Round float64 ``y`` to E4M3FN (RNE incl. subnormals, saturating at
    448).  The sign bit follows the sign of ``y``."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), E4M3_MAX)
    code = _rne_index(mag, E4M3_MAGNITUDES).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def bf16_bits_to_float64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)

