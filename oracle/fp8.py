"""Element decode for the oracle (test infrastructure; see oracle/__init__.py).

bf16: the upper half of an IEEE fp32 word, so widening is exact.
fp16 [IEEE 754 binary16; the RFC's decoder scope is BF16/FP16]: 1 sign bit,
5 exponent bits (bias 15), 10 mantissa bits; exponent 0 is subnormal
(M/1024 * 2^-14); exponent 31 is infinity (M = 0) or NaN.
e4m3fn [OCP E4M3; the RFC's Proposed Change names this OCP format as distinct
from MI300's e4m3fnuz]: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
exponent 0 is subnormal (M/8 * 2^-6); exponent 15 with mantissa 7 is NaN and
there are no infinities, so the largest finite magnitude is 448.
"""
import math

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_value(code: int) -> float:
    """Value of one IEEE binary16 pattern, from the bit-field definition."""
    code = int(code) & 0xFFFF
    sign = -1.0 if code & 0x8000 else 1.0
    exp = (code >> 10) & 0x1F
    man = code & 0x3FF
    if exp == 0x1F:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * (man / 1024.0) * 2.0 ** -14
    return sign * (1.0 + man / 1024.0) * 2.0 ** (exp - 15)


_FP16 = np.array([fp16_value(c) for c in range(1 << 16)], dtype=np.float64)


def decode_fp16(bits) -> np.ndarray:
    """uint16 binary16 bit patterns -> float64 (exact)."""
    return _FP16[np.asarray(bits, dtype=np.uint16)]


def decode_q(bits, kv_dtype: str) -> np.ndarray:
    """Query bit patterns -> float64: fp16 queries go with an fp16 cache, bf16
    queries with a bf16 or fp8 cache."""
    return decode_fp16(bits) if kv_dtype == "fp16" else decode_bf16(bits)


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, from the bit-field definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3FN = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 code values (no scale applied)."""
    return _E4M3FN[np.asarray(codes, dtype=np.uint8)]


def decode_kv(raw, kv_dtype: str, scale=None) -> np.ndarray:
    """Raw KV element codes -> dequantized float64 values.

    bf16 codes decode exactly; fp8 codes decode to code value x per-tensor scale
    (the scale is a plain multiplier applied in fp64).
    """
    if kv_dtype == "bf16":
        return decode_bf16(raw)
    if kv_dtype == "fp16":
        return decode_fp16(raw)
    if kv_dtype == "fp8":
        v = decode_e4m3fn(raw)
        return v if scale is None else v * float(scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def encode_e4m3fn(values) -> np.ndarray:
    """float values -> e4m3fn codes: the nearest finite code value, ties to the
    even code (round to nearest even), magnitudes at or above 448 saturate to
    +-448, NaN gives a NaN code of the same sign. The sign of zero is kept.
    Written as a search over the code values themselves."""
    v = np.asarray(values, dtype=np.float64)
    pos = _E4M3FN[:0x7F]                          # codes 0x00..0x7E, ascending values
    out = np.empty(v.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(v):
        sign = 0x80 if math.copysign(1.0, x) < 0 else 0
        if math.isnan(x):
            out[idx] = sign | 0x7F
            continue
        a = abs(x)
        if a >= 448.0:
            out[idx] = sign | 0x7E
            continue
        hi = int(np.searchsorted(pos, a, side="left"))   # first code value >= a
        if pos[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dl, dh = a - pos[lo], pos[hi] - a
            code = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        out[idx] = sign | code
    return out


def quantize_e4m3fn(bf16_bits, scale) -> np.ndarray:
    """bf16 codes -> e4m3fn codes of value / scale, the division taken in fp32
    (both operands are fp32 values) before rounding to the nearest code."""
    x = decode_bf16(bf16_bits).astype(np.float32)
    q = x / np.float32(scale)                      # IEEE fp32 division
    return encode_e4m3fn(q.astype(np.float64))
