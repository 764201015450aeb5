"""Oracle: 8-bit floating-point KV storage (E4M3 or E5M2) and its per-head scaling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
(pwwt.cn/news/3010209), section "工程边界与架构取舍", names FP8 storage of the
KV cache as the way to halve its memory, at the cost of quantisation error.
It fixes no format and no scaling rule; the readings taken here are:

* format: E4M3 as in the OCP 8-bit floating-point specification (1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
  subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448); or E5M2 from the same
  specification (1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits;
  exponent field 0 holds subnormals m/4 * 2^-14; exponent field 31 holds
  infinity (mantissa 0) and NaN (mantissa != 0), so the largest finite
  magnitude is 1.75 * 2^15 = 57344);
* scaling: one float32 scale per KV head for K and one for V; a stored code
  c represents scale * value(c);
* quantisation: x -> fp32(x) * fp32(1 / scale), the product rounded in
  float32, then to the nearest value of the format with ties to the even
  code, magnitudes above the largest finite one (infinities included)
  saturating to it, NaN to the NaN code (0x7F for both formats).

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


# ------------------------------------------------------------------ E5M2 --

E5M2_NAN_CODE = 0x7F
E5M2_MAX_FINITE = 57344.0
E5M2_MAX_CODE = 0x7B


def e5m2_value(code: int) -> float:
    """Real value of one E5M2 code (float64; +-inf and NaN for exponent 31)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (m / 4.0) * 2.0 ** -14
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)

# finite non-negative magnitudes, indexed by code 0x00 .. 0x7B
_E5M2_MAGNITUDES = E5M2_TABLE[: E5M2_MAX_CODE + 1]


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of an array of uint8 E5M2 codes."""
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode_one(x: float) -> int:
    """Nearest E5M2 code of a float32 value, ties to the even code,
    magnitudes of 57344 and above (infinities too) saturating to 57344."""
    x = float(np.float32(x))
    if np.isnan(x):
        return E5M2_NAN_CODE
    sign = 0x80 if np.signbit(x) else 0
    a = abs(x)
    if a >= E5M2_MAX_FINITE:
        return sign | E5M2_MAX_CODE
    d = np.abs(_E5M2_MAGNITUDES - a)
    best = np.flatnonzero(d == d.min())
    if best.size == 1:
        code = int(best[0])
    else:  # a tie between two neighbours: the code with an even mantissa
        code = int(best[0]) if int(best[0]) % 2 == 0 else int(best[1])
    return sign | code


def e5m2_encode(x: np.ndarray) -> np.ndarray:
    """Array form of ``e5m2_encode_one`` (same search as ``e4m3_encode``)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    top = E5M2_MAX_CODE
    hi = np.clip(np.searchsorted(_E5M2_MAGNITUDES, a, side="left"), 0, top)
    lo = np.clip(hi - 1, 0, top)
    d_lo = np.abs(a - _E5M2_MAGNITUDES[lo])
    d_hi = np.abs(_E5M2_MAGNITUDES[hi] - a)
    with np.errstate(invalid="ignore"):  # infinities: handled by saturation below
        code = np.where(d_lo < d_hi, lo, hi)
        tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(a >= E5M2_MAX_FINITE, top, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), E5M2_NAN_CODE, code)
    return code.astype(np.uint8)


# kv_dtype names of 8-bit pools and their formats
KV_FORMATS = {"fp8_e4m3": "e4m3", "fp8_e5m2": "e5m2"}


def encode(x: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    return e4m3_encode(x) if fmt == "e4m3" else e5m2_encode(x)


def decode(codes: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    return e4m3_decode(codes) if fmt == "e4m3" else e5m2_decode(codes)


def nan_code(fmt: str = "e4m3") -> int:
    return NAN_CODE if fmt == "e4m3" else E5M2_NAN_CODE


def inverse_scale(scale: np.ndarray) -> np.ndarray:
    """fp32(1 / scale), the factor quantisation multiplies by."""
    s = np.asarray(scale, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)


def quantize_rows(rows_f32: np.ndarray, scale: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Codes of rows [..., Hkv, D] (float32 values) with per-head scales [Hkv]."""
    rows = np.asarray(rows_f32, dtype=np.float32)
    prod = (rows * inverse_scale(scale)[:, None]).astype(np.float32)  # one float32 product
    return encode(prod, fmt)


def dequantize_rows(codes: np.ndarray, scale: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Float64 values scale[h] * value(code) of codes [..., Hkv, D]."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return decode(codes, fmt) * s[:, None]
