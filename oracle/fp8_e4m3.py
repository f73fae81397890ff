"""OCP 8-bit floating point, E4M3 ("FN") encoding, written from the OCP OFP8
specification: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, a single NaN mantissa pattern (S.1111.111), largest finite
magnitude 448.

The pages name the format only ("KV Cache优化实战" §2.1: FP8 takes one byte per
element; §3.3: vLLM's ``kv_cache_dtype`` accepts ``fp8_e4m3``) and ask for a
scale per token or per head rather than one per matrix (§3.2).  How the scale
is chosen and how values round are readings, stated with the functions below.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def decode_code(code: int) -> float:
    """Value of one e4m3 byte, straight from the field definitions."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                       # subnormal: 0.m * 2^(1-bias)
        return sign * (m / 8.0) * 2.0 ** (1 - _BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - _BIAS)


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E are ordered by value (exponent field
# above mantissa field), so the table slice is sorted ascending.
_POS = _TABLE[:0x7F].copy()


def encode_rne(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each finite ``y`` with |y| <= 448, ties to the even
    code (the code with even mantissa; adjacent codes alternate parity, and the
    largest subnormal 0x07 sits next to the smallest normal 0x08).  The sign bit
    follows the sign of ``y`` (so -0.0 encodes as 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("encode_rne expects finite inputs already clamped to +-448")
    hi = np.searchsorted(_POS, a, side="left")        # first code with value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[hi], hi, code).astype(np.uint8)   # exact hits
    neg = np.signbit(y)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def quantise_rows(x: np.ndarray):
    """Quantise rows of float32 values (last axis = one (token, head) row of
    head_dim values) with one scale per row.

    Reading of "per-token, per-head scale" ("KV Cache优化实战" §3.2, §7.3):
      a = max |x| over the row (float32, exact)
      s = a / 448 in float32 (correctly rounded); s = 1 when a == 0
      c = e4m3_rne(clamp(x / s, -448, 448)) with x / s a float32 division.
    Returns (codes uint8 with the shape of x, scales float32 with the leading shape).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(a == 0, np.float32(1.0), s).astype(np.float32)
    y = (x / s[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_rne(y), s


def dequantise(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 value of each code times its row's scale."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[..., None]
