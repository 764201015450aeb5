"""Oracle: 8-bit floating-point KV storage (E4M3) and its per-head scaling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
(pwwt.cn/news/3010209), section "工程边界与架构取舍", names FP8 storage of the
KV cache as the way to halve its memory, at the cost of quantisation error.
It fixes no format and no scaling rule; the readings taken here are:

* format: E4M3 as in the OCP 8-bit floating-point specification (1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
  subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448);
* scaling: one float32 scale per KV head for K and one for V; a stored code
  c represents scale * value(c);
* quantisation: x -> fp32(x) * fp32(1 / scale), the product rounded in
  float32, then to the nearest E4M3 value with ties to the even code,
  magnitudes above 448 saturating to 448, NaN to the NaN code.

Everything is written from that definition: values by the formula, encoding
by an exhaustive nearest-value search over the finite codes.
"""
from __future__ import annotations

import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0


def e4m3_value(code: int) -> float:
    """Real value of one E4M3 code (float64; NaN for the NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# finite non-negative magnitudes, indexed by code 0x00 .. 0x7E
_MAGNITUDES = E4M3_TABLE[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of an array of uint8 codes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_one(x: float) -> int:
    """Nearest E4M3 code of a float32 value, ties to the even code,
    saturating at 448."""
    x = float(np.float32(x))
    if np.isnan(x):
        return NAN_CODE
    sign = 0x80 if np.signbit(x) else 0
    a = abs(x)
    if a >= MAX_FINITE:
        return sign | 0x7E
    d = np.abs(_MAGNITUDES - a)
    best = np.flatnonzero(d == d.min())
    if best.size == 1:
        code = int(best[0])
    else:  # a tie between two neighbours: the code with an even mantissa
        code = int(best[0]) if int(best[0]) % 2 == 0 else int(best[1])
    return sign | code


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Array form of ``e4m3_encode_one``: the two finite magnitudes around
    |x| (the table is sorted), the nearer one, ties to the even code."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    hi = np.clip(np.searchsorted(_MAGNITUDES, a, side="left"), 0, 0x7E)  # first magnitude >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(a - _MAGNITUDES[lo])
    d_hi = np.abs(_MAGNITUDES[hi] - a)
    code = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(a >= MAX_FINITE, 0x7E, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), NAN_CODE, code)
    return code.astype(np.uint8)


def inverse_scale(scale: np.ndarray) -> np.ndarray:
    """fp32(1 / scale), the factor quantisation multiplies by."""
    s = np.asarray(scale, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)


def quantize_rows(rows_f32: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Codes of rows [..., Hkv, D] (float32 values) with per-head scales [Hkv]."""
    rows = np.asarray(rows_f32, dtype=np.float32)
    prod = (rows * inverse_scale(scale)[:, None]).astype(np.float32)  # one float32 product
    return e4m3_encode(prod)


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Float64 values scale[h] * value(code) of codes [..., Hkv, D]."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return e4m3_decode(codes) * s[:, None]
