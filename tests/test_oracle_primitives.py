"""Pins of the oracle's float primitives (exp, silu, bf16 rounding).

These primitives fix the rounding order of the conv step so that the GPU conv
can be compared bit for bit.  They are pinned here against mathematics and
against library routines, never against themselves:
  - the exp constants against their definitions computed in exact rational /
    50-digit decimal arithmetic;
  - exp against the double-precision libm exp (error <= 1 ulp);
  - bf16 rounding against torch's float32 -> bfloat16 conversion;
  - silu against the double-precision definition.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch


def nearest_f32(x: Fraction) -> np.float32:
    """The float32 nearest to an exact rational (ties to even)."""
    f = np.float32(float(x))
    best = f
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if abs(Fraction(float(cand)) - x) < abs(Fraction(float(best)) - x):
            best = cand
    return np.float32(best)


def ln2_fraction(digits=60) -> Fraction:
    getcontext().prec = digits
    return Fraction(Decimal(2).ln())


def test_exp32_constants_are_the_stated_roundings(orc):
    c = orc.exp32_constants()
    log2e, hi, lo = c[0], c[1], c[2]
    ln2 = ln2_fraction()
    assert log2e == nearest_f32(1 / ln2)
    # LN2_HI: ln 2 rounded to a multiple of 2^-16
    assert (Fraction(float(hi)) * 2 ** 16).denominator == 1
    assert abs(Fraction(float(hi)) - ln2) <= Fraction(1, 2 ** 17)
    assert lo == nearest_f32(ln2 - Fraction(float(hi)))
    for k in range(8):
        assert c[3 + k] == nearest_f32(Fraction(1, math.factorial(k))), k


def _ulp32(v: np.ndarray) -> np.ndarray:
    v = np.abs(v.astype(np.float32))
    return (np.nextafter(v, np.float32(np.inf)) - v).astype(np.float64)


def test_exp32_within_one_ulp_of_libm(orc):
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        np.linspace(-87.0, 88.7, 400_001, dtype=np.float64),
        rng.uniform(-20.0, 20.0, 200_000),
        rng.normal(0.0, 1.0, 100_000),
    ]).astype(np.float32)
    got = orc.exp32(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    err_ulp = np.abs(got - ref) / _ulp32(ref.astype(np.float32))
    assert np.max(err_ulp) <= 1.0, float(np.max(err_ulp))


def test_exp32_subnormal_range(orc):
    xs = np.linspace(-103.9, -87.4, 20_001).astype(np.float32)
    got = orc.exp32(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    # results below FLT_MIN are rounded once; error <= one subnormal step (2^-149)
    # plus the relative error of the polynomial
    assert np.all(np.abs(got - ref) <= 2.0 ** -149 + 2e-7 * ref)


def test_exp32_special_values(orc):
    f = lambda v: float(orc.exp32(np.float32(v))[0])
    assert f(0.0) == 1.0
    assert f(-0.0) == 1.0
    assert math.isnan(f(float("nan")))
    assert f(89.0) == math.inf and f(1e30) == math.inf and f(float("inf")) == math.inf
    assert f(-104.0) == 0.0 and f(-1e30) == 0.0 and f(float("-inf")) == 0.0
    assert f(1.0) == float(np.float32(math.e))


def test_exp32_monotone(orc):
    xs = np.linspace(-30.0, 30.0, 1_000_001).astype(np.float32)
    y = orc.exp32(xs)
    assert np.all(np.diff(y.astype(np.float64)) >= 0.0)


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, size=500_000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45,
                     1.17549435e-38, np.inf, -np.inf], dtype=np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd kept parts
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00008000, 0x00018000],
                    dtype=np.uint32).view(np.float32)
    xs = np.concatenate([xs, edge, ties])
    finite = ~np.isnan(xs)
    got = orc.bf16_rne_bits(xs)
    ref = torch.from_numpy(xs.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[finite], ref[finite])
    nan_out = got[~finite]
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x007F) != 0)


def test_silu32_against_double_definition(orc):
    xs = np.concatenate([np.linspace(-80, 80, 200_001), np.random.default_rng(3).normal(0, 2, 100_000)])
    xs = xs.astype(np.float32)
    got = orc.silu32(xs).astype(np.float64)
    x64 = xs.astype(np.float64)
    ref = x64 / (1.0 + np.exp(-x64))
    # exp <= 1 ulp, one add, one divide: a few ulp of the result
    tol = 4.0 * _ulp32(ref.astype(np.float32)) + 1e-45
    assert np.all(np.abs(got - ref) <= tol)


def test_silu32_special_values(orc):
    f = lambda v: orc.silu32(np.float32(v))[0]
    assert f(0.0) == 0.0
    assert f(200.0) == np.float32(200.0)
    r = f(-200.0)  # e^200 overflows: -200 / inf = -0
    assert r == 0.0 and math.copysign(1.0, float(r)) == -1.0
    assert math.isnan(float(f(float("nan"))))
