"""Pure-Python scalar brute force for tiny shapes (oracle; test
infrastructure only).

A second, independent route to the same definitions as ``quant`` and
``attention``: no NumPy, no frexp and no sorted-table search.  The shared
exponent is found by stepping a power of two, each element is rounded by
scanning every code of the format, and attention is written as explicit loops
with math.exp / math.fsum.  Used only to cross-check the vectorised oracle on
inputs small enough for loops.
"""

import math
import struct

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def e4m3_value(code):
    if code & 0x7F == 0x7F:
        return math.nan
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


def e2m1_value(code):
    return (-1.0 if code & 8 else 1.0) * _E2M1[code & 7]


def floor_log2(a):
    """Largest integer e with 2**e <= a (a > 0), by stepping."""
    e = 0
    while 2.0 ** e > a:
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    return e


def nearest_code(y, codes, value_of):
    """Code whose value is nearest to y; ties go to the code with an even
    mantissa LSB (even code).  Only codes with the sign of y are scanned, so a
    negative y that rounds to zero keeps its sign bit."""
    neg = math.copysign(1.0, y) < 0
    best = None
    for c in codes:
        v = value_of(c)
        if math.isnan(v) or (math.copysign(1.0, v) < 0) != neg:
            continue
        dist = abs(v - y)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1]


def quantize_block_e2m1(values):
    """One 32-element MXFP4 block of float values -> (codes, scale byte)."""
    a = max(abs(x) for x in values)
    X = -127 if a == 0.0 else max(-127, min(127, floor_log2(a) - 2))
    codes = []
    for x in values:
        y = x / 2.0 ** X
        y = math.copysign(min(abs(y), 6.0), y)
        codes.append(nearest_code(y, range(16), e2m1_value))
    return codes, X + 127


def quantize_tile_e4m3(values):
    """A flat list of tile values -> (E4M3 codes, E8M0 scale byte)."""
    a = max(abs(x) for x in values)
    X = -127 if a == 0.0 else max(-127, min(127, floor_log2(a) - 8))
    codes = []
    for x in values:
        y = x / 2.0 ** X
        y = math.copysign(min(abs(y), 448.0), y)
        codes.append(nearest_code(y, range(256), e4m3_value))
    return codes, X + 127


def attention_rows(q, k, v, sigma, causal):
    """q: list of Nq rows, k/v: lists of Nk rows (floats).  Bottom-right
    causal mask when ``causal``.  Returns (o rows, lse list)."""
    nq, nk = len(q), len(k)
    out, lses = [], []
    for i in range(nq):
        last = i + (nk - nq) if causal else nk - 1
        s = [sigma * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in range(last + 1)]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        l = math.fsum(p)
        out.append([math.fsum(p[j] * v[j][c] for j in range(len(p))) / l for c in range(len(v[0]))])
        lses.append(m + math.log(l))
    return out, lses


def attention_rows_fast_p(q, k, v, sigma, causal, block=32, headroom=7):
    """Single-term E4M3 probabilities by loops: base-2 scores t = s*log2(e),
    keys in blocks [block*a, block*a + block), each block's range exponent
    X = floor(max t) - headroom (floor found by stepping), each weight rounded
    by scanning every E4M3 code.  Returns (o rows, lse list)."""
    nq, nk = len(q), len(k)
    log2e = 1.0 / math.log(2.0)
    out, lses = [], []
    for i in range(nq):
        last = i + (nk - nq) if causal else nk - 1
        t = [sigma * math.fsum(a * b for a, b in zip(q[i], k[j])) * log2e for j in range(last + 1)]
        M = max(t)
        Mi = math.floor(M)
        p = []
        for j in range(last + 1):
            a = j // block
            bmax = max(t[a * block:min((a + 1) * block, last + 1)]) - Mi
            X = floor_log2(2.0 ** bmax) - headroom
            y = 2.0 ** (t[j] - Mi - X)
            p.append(e4m3_value(nearest_code(y, range(128), e4m3_value)) * 2.0 ** X)
        l = math.fsum(p)
        out.append([math.fsum(p[j] * v[j][c] for j in range(len(p))) / l for c in range(len(v[0]))])
        lses.append((Mi + math.log2(l)) * math.log(2.0))
    return out, lses


def _f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def hadamard_row_f32(values):
    """One row through the Sylvester-Hadamard butterflies h = 1, 2, ..., d/2,
    each sum and difference rounded to float32 by packing (a second route to
    ``quant.hadamard_rows_f32``)."""
    x = [_f32(v) for v in values]
    d = len(x)
    h = 1
    while h < d:
        for i in range(d):
            if i & h == 0:
                a, b = x[i], x[i + h]
                x[i], x[i + h] = _f32(a + b), _f32(a - b)
        h *= 2
    return x


def attention_rows_window(q, k, v, sigma, window):
    """Bottom-right causal attention where row i sees only the ``window`` most
    recent keys up to its position, by loops (second route for the window
    mask)."""
    nq, nk = len(q), len(k)
    out, lses = [], []
    for i in range(nq):
        last = i + (nk - nq)
        first = max(0, last - window + 1)
        s = [sigma * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in range(first, last + 1)]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        l = math.fsum(p)
        out.append([math.fsum(p[j] * v[first + j][c] for j in range(len(p))) / l for c in range(len(v[0]))])
        lses.append(m + math.log(l))
    return out, lses
