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
