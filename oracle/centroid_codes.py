"""fp8 (E4M3) codes of the centroids with one power-of-two scale per 32
values -- the reduced-precision centroid copies the decode may read.

TEST INFRASTRUCTURE ONLY (part of the oracle package; see its header).

The pages do not describe this format: it is a bandwidth option of this
implementation.  The element format is E4M3 of the OCP 8-bit floating point
specification (OFP8): sign, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals at exponent field 0, no infinities, S.1111.111 is NaN, largest
finite magnitude 448.  As in the OCP Microscaling (MX) formats, 32
consecutive values share a scale 2^E stored as an 8-bit biased exponent
(E + 127); unlike MX's rule (E from the exponent of the largest magnitude,
which clamps values above 448), E here is the least integer with
max|x| * 2^-E <= 448, floored at -126, so no value is clamped.

Written as plain definitions: a table of the 127 finite non-negative E4M3
values, the scale by search, and each code by nearest table value with ties
to the even code (round to nearest even).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 32          # values per shared scale
E_MIN = -126        # smallest scale exponent (biased 1)
MAX_FINITE = 448.0


def _value(code: int) -> float:
    """Magnitude of a non-negative E4M3 code (0 .. 126), from the definition."""
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return m * 2.0 ** -9            # subnormal: 0.m x 2^(1 - 7)
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


VALUES = np.array([_value(c) for c in range(127)])  # code 127 is NaN


def scale_exponent(amax: float) -> int:
    """Least integer E >= E_MIN with amax * 2^-E <= 448."""
    if amax == 0.0:
        return E_MIN
    E = math.frexp(amax)[1] - 10        # amax * 2^-E >= 2^9 > 448: too small
    while math.ldexp(amax, -E) > MAX_FINITE:
        E += 1
    return max(E, E_MIN)


def encode_magnitudes(a) -> np.ndarray:
    """Codes of the table values nearest to magnitudes a <= 448; ties go to
    the even code."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    if np.any(a > MAX_FINITE):
        raise ValueError("magnitude above 448")
    i = np.clip(np.searchsorted(VALUES, a), 1, len(VALUES) - 1)  # VALUES[i - 1] < a <= VALUES[i] (a > 0)
    lo, hi = VALUES[i - 1], VALUES[i]
    below, above = a - lo, hi - a
    pick_hi = (above < below) | ((above == below) & (i % 2 == 0))
    return np.where(a == 0, 0, np.where(pick_hi, i, i - 1)).astype(np.uint8)


def encode_magnitude(y: float) -> int:
    return int(encode_magnitudes([y])[0])


def encode_block(x) -> tuple:
    """(codes uint8[n], E) of up to 32 values sharing one scale."""
    x = np.asarray(x, dtype=np.float64)
    E = scale_exponent(float(np.abs(x).max()) if x.size else 0.0)
    codes = encode_magnitudes(np.ldexp(x, -E)) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return codes.astype(np.uint8), E


def encode_rows(X) -> tuple:
    """codes uint8 [n][d] and biased scale exponents uint8 [n][d / 32]."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    codes = np.zeros((n, d), np.uint8)
    scales = np.zeros((n, d // BLOCK), np.uint8)
    for i in range(n):
        for b in range(d // BLOCK):
            c, E = encode_block(X[i, b * BLOCK:(b + 1) * BLOCK])
            codes[i, b * BLOCK:(b + 1) * BLOCK] = c
            scales[i, b] = E + 127
    return codes, scales


def decode_rows(codes, scales) -> np.ndarray:
    """float64 values of codes [n][d] with biased exponents [n][d / 32]."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = VALUES[np.minimum(codes & 0x7F, 126)]
    if np.any((codes & 0x7F) == 127):
        raise ValueError("NaN code")
    sign = np.where(codes & 0x80, -1.0, 1.0)
    E = np.repeat(np.asarray(scales, dtype=np.int64) - 127, BLOCK, axis=1)
    return sign * mag * np.exp2(E.astype(np.float64))


def coded_state(st):
    """A copy of a unit state whose key and value centroids are their fp8
    round trips: the decode of such a state is the decode that reads the
    codes."""
    import copy
    out = copy.copy(st)
    C = st.n_clusters
    out.kbar = st.kbar.copy()
    out.vbar = st.vbar.copy()
    if C:
        out.kbar[:C] = decode_rows(*encode_rows(st.kbar[:C]))
        out.vbar[:C] = decode_rows(*encode_rows(st.vbar[:C]))
    return out
