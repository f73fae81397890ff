"""Quantised KV cache formats beyond fp8 e4m3: fp8 e5m2, and INT8 keys with
INT4 values, in plain numpy.

What the pages fix ("KV Cache优化实战" §3.2-3.4): K and V tolerate
quantisation differently, so the usual choice is mixed precision, K at INT8
or FP8 and V at INT4; a scale per token or per head restores values better
than one scale per matrix; vLLM's cache dtype accepts fp8_e5m2 as well as
fp8_e4m3, and llama.cpp pairs an 8-bit K cache with a 4-bit V cache.

Readings (the pages leave these open), kept parallel to the e4m3 path:
  * every format scales each (token, head) row of head_dim values by its own
    float32 scale s = max|x| / Q, with Q the format's largest code magnitude
    (57344 for e5m2, 127 for INT8, 7 for INT4) and s = 1 for an all-zero row;
  * codes come from x / s (a float32 division) clamped to [-Q, Q] and rounded
    to the nearest code with ties to even: the even mantissa for e5m2, the
    even integer for INT8 / INT4;
  * INT8 codes are stored as two's-complement bytes; INT4 codes as
    two's-complement nibbles, two per byte, element 2i in the low nibble of
    byte i and element 2i+1 in the high nibble;
  * e5m2 is OCP E5M2: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa
    bits, infinities at exponent 31 with mantissa 0 and NaN otherwise; the
    clamp keeps every stored code finite.

Test infrastructure: only tests, the smoke check and the CPU baseline leg of
the benchmark use this module.
"""
from __future__ import annotations

import numpy as np

from . import fp8_e4m3

E5M2_MAX = 57344.0
_E5M2_BIAS = 15
INT8_MAX = 127
INT4_MAX = 7


# ---- fp8 e5m2 -------------------------------------------------------------------------

def e5m2_decode_code(code: int) -> float:
    """Value of one e5m2 byte from the field definitions."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:                        # subnormal: 0.m * 2^(1-bias)
        return sign * (m / 4.0) * 2.0 ** (1 - _E5M2_BIAS)
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - _E5M2_BIAS)


def e5m2_table() -> np.ndarray:
    return np.array([e5m2_decode_code(c) for c in range(256)], dtype=np.float64)


_E5M2 = e5m2_table()
_E5M2_POS = _E5M2[:0x7C].copy()          # finite non-negative codes, ascending


def e5m2_encode_rne(y: np.ndarray) -> np.ndarray:
    """Nearest finite e5m2 code to each |y| <= 57344, ties to the code with
    the even mantissa (adjacent codes alternate parity); the sign bit follows
    y's sign."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(~np.isfinite(a)) or np.any(a > E5M2_MAX):
        raise ValueError("e5m2_encode_rne expects finite inputs already clamped to +-57344")
    hi = np.minimum(np.searchsorted(_E5M2_POS, a, side="left"), len(_E5M2_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E5M2_POS[lo]
    d_hi = _E5M2_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E5M2_POS[hi], hi, code).astype(np.uint8)
    return (code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def _row_scales(x: np.ndarray, qmax: float) -> np.ndarray:
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(qmax)).astype(np.float32)
    return np.where(a == 0, np.float32(1.0), s).astype(np.float32)


def quantise_e5m2_rows(x: np.ndarray):
    """(codes uint8 like x, scales float32 per row) with s = max|x| / 57344."""
    x = np.asarray(x, dtype=np.float32)
    s = _row_scales(x, E5M2_MAX)
    y = np.clip((x / s[..., None]).astype(np.float32), np.float32(-E5M2_MAX), np.float32(E5M2_MAX))
    return e5m2_encode_rne(y), s


def dequantise_e5m2(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return _E5M2[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[..., None]


# ---- symmetric integers -----------------------------------------------------------------

def quantise_int_rows(x: np.ndarray, qmax: int):
    """(codes int8 like x in [-qmax, qmax], scales float32 per row):
    s = max|x| / qmax, code = the integer nearest x / s (ties to even)."""
    x = np.asarray(x, dtype=np.float32)
    s = _row_scales(x, qmax)
    y = np.clip((x / s[..., None]).astype(np.float32), np.float32(-qmax), np.float32(qmax))
    return np.rint(y).astype(np.int8), s


def dequantise_int(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int4 codes [..., D] (values -8..7) -> bytes [..., D/2]: element 2i in
    the low nibble of byte i, element 2i+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.int16)
    if c.shape[-1] % 2 or np.any(c < -8) or np.any(c > 7):
        raise ValueError("int4 codes must be -8..7 with an even last dimension")
    u = (c & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---- cache formats ------------------------------------------------------------------------
# name -> (K element format, V element format); element formats:
#   "f32" / "f16" / "bf16": values kept as written
#   "e4m3", "e5m2", "i8", "i4": codes plus a float32 scale per (token, head)

FORMATS = {
    "f32": ("f32", "f32"),
    "f16": ("f16", "f16"),
    "bf16": ("bf16", "bf16"),
    "fp8_e4m3": ("e4m3", "e4m3"),
    "fp8_e5m2": ("e5m2", "e5m2"),
    "int8_int4": ("i8", "i4"),
}


def is_quantised(elem: str) -> bool:
    return elem in ("e4m3", "e5m2", "i8", "i4")


def quantise(x: np.ndarray, elem: str):
    """Stored (codes, scales) of rows x for a quantised element format; codes
    are what the pool holds (int4: packed bytes [..., D/2])."""
    if elem == "e4m3":
        return fp8_e4m3.quantise_rows(x)
    if elem == "e5m2":
        return quantise_e5m2_rows(x)
    if elem == "i8":
        c, s = quantise_int_rows(x, INT8_MAX)
        return c.view(np.uint8), s
    if elem == "i4":
        c, s = quantise_int_rows(x, INT4_MAX)
        return pack_int4(c), s
    raise ValueError(elem)


def dequantise(codes: np.ndarray, scales: np.ndarray, elem: str) -> np.ndarray:
    """float64 values of stored codes (as ``quantise`` returns them)."""
    if elem == "e4m3":
        return fp8_e4m3.dequantise(codes, scales)
    if elem == "e5m2":
        return dequantise_e5m2(codes, scales)
    if elem == "i8":
        return dequantise_int(np.asarray(codes, dtype=np.uint8).view(np.int8), scales)
    if elem == "i4":
        return dequantise_int(unpack_int4(codes), scales)
    raise ValueError(elem)


def values_as_cached(x: np.ndarray, elem: str) -> np.ndarray:
    """float64 values a pool of element format ``elem`` holds for rows x."""
    if not is_quantised(elem):
        return np.asarray(x, dtype=np.float64)
    c, s = quantise(x, elem)
    return dequantise(c, s, elem)
