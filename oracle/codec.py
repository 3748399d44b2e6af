"""Stored number formats: fp32, bf16 and OCP E4M3 (e4m3fn), CPU oracle side.

Test infrastructure.  Decoding is exact (every bf16 and E4M3 value is an fp32
value).  Encoding is round-to-nearest, ties-to-even, done here by searching the
table of representable values, which is the definition rather than a bit
trick.  E4M3 follows the OCP 8-bit floating point specification: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, the
single NaN pattern S.1111.111, no infinities, largest finite value 448.
Values beyond 448 saturate to 448 (the method never needs NaN or infinity).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_value_table()
# non-negative finite magnitudes, ascending with the code (codes 0..126)
_E4M3_POS = _E4M3[:127].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float32 values (exact)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes, nearest value, ties to the even code, saturating.

    The sign of the result is the sign bit of the input, so -0.0 and small
    negative values give 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    a = np.abs(x).astype(np.float64)
    hi = np.searchsorted(_E4M3_POS, a, side="left")       # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)
    code = np.where(a <= _E4M3_POS[0], 0, code)
    return (code.astype(np.uint8) | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, nearest value with ties to the even pattern."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lo = bits & np.uint32(0xFFFF0000)                  # toward zero
    hi = lo + np.uint32(0x10000)                       # next away from zero
    v = np.abs(x.astype(np.float64))
    v_lo = np.abs(lo.view(np.float32).astype(np.float64))
    v_hi = np.abs(hi.view(np.float32).astype(np.float64))
    d_lo = v - v_lo
    d_hi = v_hi - v
    lo_even = ((lo >> 16) & 1) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    chosen = np.where(pick_hi, hi, lo).astype(np.uint32)
    return (chosen >> 16).astype(np.uint16)


def dequantize(raw: np.ndarray, scale, dtype: str) -> np.ndarray:
    """Stored rows -> float32 values; E4M3 rows are decoded then multiplied by
    their fp32 scale (one fp32 rounding), as the key is defined."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return bf16_decode(raw)
    if dtype == "e4m3":
        v = e4m3_decode(raw)
        s = np.asarray(scale, dtype=np.float32)
        return (v * s[..., None]).astype(np.float32)
    raise ValueError(dtype)


def decode_codes(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored rows -> float32 values without the per-row scale."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return bf16_decode(raw)
    if dtype == "e4m3":
        return e4m3_decode(raw)
    raise ValueError(dtype)


def quantize_rep(c: np.ndarray, dtype: str):
    """Cluster representative in the key format, from an fp32 centroid.

    fp32: the centroid itself.  bf16: nearest-even rounding.  E4M3: scale
    sr = amax|c| / 448 (fp32 division; 1.0 if the centroid is all zero), codes
    = E4M3(c_i / sr) with an fp32 division per element.
    Returns (raw, scale) with scale a python float32 (1.0 except E4M3).
    """
    c = np.asarray(c, dtype=np.float32)
    if dtype == "f32":
        return c.copy(), np.float32(1.0)
    if dtype == "bf16":
        return bf16_encode(c), np.float32(1.0)
    if dtype == "e4m3":
        amax = np.float32(np.max(np.abs(c))) if c.size else np.float32(0.0)
        if amax == 0:
            return np.zeros(c.shape, dtype=np.uint8), np.float32(1.0)
        sr = np.float32(amax / np.float32(E4M3_MAX))
        return e4m3_encode((c / sr).astype(np.float32)), sr
    raise ValueError(dtype)
