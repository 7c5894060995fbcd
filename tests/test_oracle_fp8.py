"""Pins for the oracle's element decode (CPU only)."""
import math

import numpy as np
import torch

import oracle
from conftest import load_golden


def test_e4m3fn_points_from_spec():
    g = load_golden("e4m3fn_points.json")
    for p in g["points"]:
        v = oracle.e4m3fn_value(int(p["code"], 16))
        assert v == p["value"], p
        assert math.copysign(1.0, v) == math.copysign(1.0, p["value"]), p
    for c in g["nan_codes"]:
        assert math.isnan(oracle.e4m3fn_value(int(c, 16)))


def test_e4m3fn_matches_torch_cast_all_codes():
    """Independent implementation: torch's float8_e4m3fn -> float64 widening."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.decode_e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert nan.sum() == 2


def test_e4m3fn_order_and_symmetry():
    pos = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)             # strictly increasing magnitudes
    neg = oracle.decode_e4m3fn(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)
    # exactly representable in bf16: 3 mantissa bits, exponents 2^-9 .. 2^8
    f32 = pos.astype(np.float32).view(np.uint32)
    assert np.all((f32 & 0xFFFF) == 0)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.decode_bf16(bits), x.to(torch.float64).numpy())
    special = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 9.183549615799121e-41]
    assert list(oracle.decode_bf16(special)) == want


def test_decode_kv_scale_is_plain_multiplier():
    codes = np.array([0x38, 0x40, 0xB8], dtype=np.uint8)
    assert list(oracle.decode_kv(codes, "fp8", 0.5)) == [0.5, 1.0, -0.5]


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.encode_e4m3fn(oracle.decode_e4m3fn(codes))
    assert np.array_equal(back, codes)


def test_encode_midpoints_round_to_even_code():
    """Exactly half-way between two adjacent positive codes goes to the even
    code; one fp32 step either side goes to the nearer code."""
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3fn_value(c), oracle.e4m3fn_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2                     # exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_e4m3fn([float(mid)])[0] == even, c
        below = float(np.nextafter(mid, np.float32(0)))
        above = float(np.nextafter(mid, np.float32(1000)))
        assert oracle.encode_e4m3fn([below])[0] == c
        assert oracle.encode_e4m3fn([above])[0] == c + 1
        assert oracle.encode_e4m3fn([-float(mid)])[0] == 0x80 | even


def test_encode_saturates_and_keeps_signs():
    e = oracle.encode_e4m3fn
    assert list(e([448.0, 449.0, 480.0, 1e30, math.inf])) == [0x7E] * 5
    assert list(e([-448.0, -1e30, -math.inf])) == [0xFE] * 3
    assert e([0.0])[0] == 0x00 and e([-0.0])[0] == 0x80
    assert e([2.0 ** -10])[0] == 0x00                          # tie with 0 -> even
    assert e([-(2.0 ** -12)])[0] == 0x80
    n = e([math.nan, -math.nan])
    assert all(np.isnan(oracle.decode_e4m3fn(n)))


def test_encode_matches_torch_cast_in_range():
    """torch's float8_e4m3fn cast (an independent implementation) agrees on
    values inside the finite range."""
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 60, 4000),
                        rng.uniform(-447.9, 447.9, 4000), rng.normal(0, 0.01, 4000)])
    v = v.astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(v.astype(np.float64)), want)


def test_quantize_divides_in_fp32():
    """bf16 value / scale in fp32, then the nearest code: a value that is an
    exact code value times the scale comes back as that code."""
    scale = 0.0173
    codes = np.array([0x01, 0x08, 0x38, 0x40, 0x55, 0x7E, 0xC4], dtype=np.uint8)
    vals = oracle.decode_e4m3fn(codes) * np.float32(scale)
    bits = np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16    # truncate to bf16
    q = oracle.quantize_e4m3fn(bits.astype(np.uint16), scale)
    back = oracle.decode_e4m3fn(q)
    x = oracle.decode_bf16(bits.astype(np.uint16))
    # nearest code value to x / scale (fp32 division), checked by brute force
    table = oracle.decode_e4m3fn(np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                                          dtype=np.uint8))
    for xi, bi in zip(x, back):
        t = float(np.float32(xi) / np.float32(scale))
        assert abs(bi - t) == np.min(np.abs(table - t))


def test_fp16_points_from_the_bit_fields():
    """Hand-derived binary16 values: 1.0, -2.0, the largest finite, the least
    normal and subnormal, 1/3 rounded, infinities, NaN and -0."""
    pts = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
           0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x3555: 1365 / 4096,
           0x7C00: math.inf, 0xFC00: -math.inf}
    for code, want in pts.items():
        assert oracle.fp16_value(code) == want, hex(code)
    assert math.isnan(oracle.fp16_value(0x7E00)) and math.isnan(oracle.fp16_value(0x7C01))
    z = oracle.fp16_value(0x8000)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_fp16_decode_matches_numpy_all_codes():
    """Independent library routine: numpy's float16 widened to float64."""
    codes = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode_fp16(codes)
    want = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(oracle.decode_kv(codes, "fp16"), got, equal_nan=True)
