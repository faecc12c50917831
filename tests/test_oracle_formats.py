"""Pins for the oracle's number formats (bf16 widening, OCP E4M3FN codec).

The fp8 KV cache is the "gemma-cuda-hybrid" README's server default (Features:
FP8 (e4m3) KV cache).  The pins compare the oracle with torch's own float8
and bfloat16 conversions (library routines) and with an exact rational brute
force, so that a wrong bias, a wrong subnormal rule, a wrong tie rule or a
missing saturation each fails a test.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import f64

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def torch_e4m3_codes(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_bf16_widening_matches_torch():
    got = oracle.bf16_value(ALL_BF16)
    want = f64(ALL_BF16)
    assert np.array_equal(got, want, equal_nan=True)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_value(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, want, equal_nan=True)
    fin = ~np.isnan(want)
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))  # signed zeros


def test_e4m3_landmarks():
    # Values fixed by the E4M3FN format itself: largest finite, smallest
    # normal, smallest subnormal, one, NaN, negative zero.
    v = oracle.e4m3_value(np.array([0x7E, 0x08, 0x01, 0x38, 0x7F, 0xFF, 0x80, 0xFE], np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 2.0 ** -9 and v[3] == 1.0
    assert np.isnan(v[4]) and np.isnan(v[5])
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -448.0


@pytest.mark.parametrize("scale", [1.0, 0.5, 2.0 ** -4, 8.0, 2.0 ** -10, 2.0 ** 7])
def test_e4m3_encode_matches_torch_power_of_two_scales(scale):
    # With a power-of-two scale, x / scale is exact in binary32, so torch's
    # float32 -> float8_e4m3fn conversion (round to nearest even) is the
    # reference.  torch turns overflow into NaN; the oracle saturates to +-448.
    x = ALL_BF16[~np.isnan(f64(ALL_BF16))]
    xv = f64(x)
    got = oracle.e4m3_encode(x, scale)
    with np.errstate(over="ignore"):
        want = torch_e4m3_codes((xv / scale).astype(np.float32))
    overflow = np.isnan(torch.from_numpy(want).view(torch.float8_e4m3fn).float().numpy())
    assert np.array_equal(got[~overflow], want[~overflow])
    sat = np.where(np.signbit(xv[overflow]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(got[overflow], sat)
    assert overflow.sum() > 0 or scale >= 2.0 ** 7


def _finite_table():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return [Fraction(float(v)) for v in vals]


def _brute_encode(x: float, scale: float, table) -> int:
    """Nearest E4M3FN code to the exact rational x/scale; ties to even;
    |x/scale| > 448 saturates."""
    sign = 0x80 if np.signbit(x) else 0
    v = abs(Fraction(x) / Fraction(scale))
    if v > 448:
        return sign | 0x7E
    best, best_d = None, None
    for c, t in enumerate(table):
        dd = abs(v - t)
        if best is None or dd < best_d or (dd == best_d and c % 2 == 0):
            best, best_d = c, dd
    return sign | best


def test_e4m3_encode_exact_rational_brute_force():
    table = _finite_table()
    g = synthetic.rng(77)
    x = synthetic.bf16_bits(g.standard_normal(1500, dtype=np.float32) * 3.0)
    # per-tensor style scales amax/448 with arbitrary mantissas
    scales = (g.uniform(1.0, 10.0, 1500) / 448.0).astype(np.float32)
    xv = f64(x)
    for i in range(x.size):
        got = int(oracle.e4m3_encode(x[i:i + 1], float(scales[i]))[0])
        assert got == _brute_encode(float(xv[i]), float(scales[i]), table), (xv[i], scales[i])


def test_e4m3_encode_ties_to_even():
    # 1.0625 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1):
    # the even neighbour 1.0 wins; 1.1875 lies between 1.125 and 1.25 -> 1.25.
    # 2^-10 lies halfway between 0 and the smallest subnormal 2^-9 -> 0.
    x = synthetic.bf16_bits(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10], np.float32))
    got = oracle.e4m3_encode(x, 1.0)
    assert list(got) == [0x38, 0x3A, 0x00, 0x02]


def test_e4m3_encode_saturation_nan_and_signed_zero():
    x = synthetic.bf16_bits(np.array([448.0, 460.0, 464.0, 1e30, -1e30, np.inf, -np.inf, -0.0, 0.0],
                                     np.float32))
    got = oracle.e4m3_encode(x, 1.0)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x80, 0x00]
    nan = np.array([0x7FC0, 0xFFC0], np.uint16)
    assert list(oracle.e4m3_encode(nan, 1.0)) == [0x7F, 0xFF]


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    bits = synthetic.bf16_bits(vals)  # exact: 4 significant bits fit in bf16
    assert np.array_equal(f64(bits), vals.astype(np.float64))
    assert np.array_equal(oracle.e4m3_encode(bits, 1.0), codes)


def test_region_bytes():
    assert oracle.region_bytes(1024, 8, 256, oracle.BF16) == 1024 * 8 * 256 * 2
    assert oracle.region_bytes(1024, 8, 256, oracle.FP8) == 1024 * 8 * 256
    with pytest.raises(ValueError):
        oracle.region_bytes(1001, 8, 256, oracle.BF16)
