"""FP8 E4M3 (OCP 8-bit floating point, "E4M3FN") codec for the FP8 KV-cache
variant -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages name a smaller KV data type only as a setting ("LLM serving from
scratch" (ta-paperlens), "in practice": a KV-cache dtype or quantisation
shrinks K/V so the pool holds more tokens; sns.style overview, "deep dive":
FP8 among the supported formats); they fix no format or scale.  Readings:
  * format: the OCP FP8 E4M3 encoding (sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no
    infinities; largest finite 448);
  * one scale per pool (K, V): a value x is stored as
    e4m3(clamp(f32(x) * f32(1 / scale), -448, 448)) rounded to nearest, ties
    to even mantissa; NaN stays NaN; a stored code c stands for
    decode(c) * scale.
The encoder is the definition written out: the nearest of the finite codes,
found by searching the sorted table of their values.
"""
from __future__ import annotations

import numpy as np

MAX_E4M3 = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (uint8 array); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def _finite_table():
    codes = np.arange(128, dtype=np.uint8)               # non-negative codes
    vals = decode_e4m3(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]                        # ascending in value


_CODES, _VALS = _finite_table()


def encode_e4m3(x) -> np.ndarray:
    """E4M3 codes of fp64-exact values x (already scaled): clamp to +-448,
    round to nearest, ties to the even mantissa; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), MAX_E4M3)
    a = np.where(np.isnan(x), 0.0, a)
    hi = np.clip(np.searchsorted(_VALS, a, side="left"), 0, len(_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_VALS) - 1)
    d_hi = _VALS[hi] - a
    d_lo = a - _VALS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((_CODES[lo] & 1) == 0))
    code = np.where(pick_lo, _CODES[lo], _CODES[hi]).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_table(scale: float) -> np.ndarray:
    """Code of every fp16 bit pattern under a per-pool scale: f32(x) *
    f32(1/scale) (both fp32 roundings), then ``encode_e4m3``; entry i is the
    code of the fp16 value whose bits are i."""
    inv = np.float32(1.0) / np.float32(scale)
    x = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):   # NaN and inf patterns
        y = x * inv
    return encode_e4m3(y.astype(np.float64))


def quantize(x16, scale: float) -> np.ndarray:
    """Codes of fp16 values x16: the code depends only on the value's bits and
    the scale, so it is looked up in ``quantize_table(scale)``."""
    bits = np.ascontiguousarray(np.asarray(x16, dtype=np.float16)).view(np.uint16)
    return quantize_table(scale)[bits]


def dequantize(codes, scale: float) -> np.ndarray:
    return decode_e4m3(codes) * float(np.float32(scale))
