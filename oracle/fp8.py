"""8-bit floating-point key/value storage (oracle side).

«The KV Cache and PagedAttention» › "What Came After": the cache can be kept in
8-bit floating point, one byte a number, fitting about twice the tokens. The
page names no format or scaling, so these readings are taken:
  * the format is OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias
    7, 3 mantissa bits; no infinities; exponent and mantissa all ones is NaN;
    the largest finite magnitude is 448 and subnormals go down to 2^-9;
  * each pool has one scale: a stored code c stands for decode(c) * scale, and a
    value x is stored as encode(x / scale);
  * encode rounds to the nearest representable value, ties to the even code
    (last mantissa bit 0), saturates magnitudes beyond 448 to 448, keeps NaN,
    and keeps the sign of values that round to zero.
Written from the format definition: decode by the formula, encode by searching
all finite codes (brute force, obviously correct).
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0


def decode_code(c: int) -> float:
    """Value of one E4M3 code (0..255)."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# finite non-negative codes sorted by value (0x00 .. 0x7E are increasing)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def encode_value(x: float) -> int:
    """E4M3 code of x: round to nearest, ties to even code, saturating, NaN kept."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = abs(x)
    if a >= MAX_FINITE:
        return sign | 0x7E
    # the two neighbouring representable magnitudes
    hi = int(np.searchsorted(_POS_VALUES, a, side="left"))
    if _POS_VALUES[hi] == a:
        return sign | hi
    lo = hi - 1
    d_lo, d_hi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
    if d_lo < d_hi:
        code = lo
    elif d_hi < d_lo:
        code = hi
    else:
        code = lo if lo % 2 == 0 else hi
    return sign | code


def encode(x) -> np.ndarray:
    """encode_value over an array, vectorized: the same nearest-value search (neighbours
    by a sorted search over the finite codes, ties to the even code, saturation, NaN)."""
    a = np.asarray(x, dtype=np.float64)
    flat = a.reshape(-1)
    sign = (np.signbit(flat).astype(np.int64)) << 7
    mag = np.abs(flat)
    mag_c = np.where(np.isnan(mag), 0.0, np.minimum(mag, MAX_FINITE))
    hi = np.minimum(np.searchsorted(_POS_VALUES, mag_c, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag_c - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag_c
    tie = np.where(lo % 2 == 0, lo, hi)
    code = np.where(_POS_VALUES[hi] == mag_c, hi,
                    np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, tie)))
    code = np.where(mag >= MAX_FINITE, 0x7E, code) | sign
    code = np.where(np.isnan(flat), 0x7F, code)
    return code.astype(np.uint8).reshape(a.shape)


def decode(codes) -> np.ndarray:
    """Element-wise decode of uint8 codes to float64."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize(x, scale: float) -> np.ndarray:
    """Stored codes of values x in a pool with the given scale."""
    return encode(np.asarray(x, dtype=np.float64) / scale)


def dequantize(codes, scale: float) -> np.ndarray:
    return decode(codes) * scale
