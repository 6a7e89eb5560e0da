"""Pins for the oracle's SwiGLU backward glue (no GPU).

The glue's arithmetic is a reading (fp32, fixed order, its own exp); these
tests check it against float64 math and exact rational rounding, not against
itself.
"""
import math
from fractions import Fraction

import numpy as np

from oracle import swiglu as sg


def test_exp32_against_math_exp():
    rng = np.random.default_rng(3)
    x = np.concatenate([np.linspace(-87.0, 88.0, 20001), rng.uniform(-20, 20, 20000)]).astype(np.float32)
    got = sg.exp32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 4e-7          # a few fp32 ulps
    assert sg.exp32(np.float32([0.0]))[0] == 1.0


def test_exp32_range_ends_and_nan():
    with np.errstate(over="ignore", under="ignore"):
        v = sg.exp32(np.float32([-200.0, -104.0, 89.0, 500.0, np.nan, -np.inf, np.inf]))
    assert v[0] == v[1] and v[1] < 1e-44          # clamped to the underflow end
    assert np.isinf(v[2]) and np.isinf(v[3]) and v[2] > 0
    assert np.isnan(v[4])
    assert v[5] == v[0] and np.isinf(v[6])


def _silu64(a):
    return a / (1.0 + math.exp(-a))


def test_silu_derivative_is_central_difference_of_silu():
    a = np.linspace(-30.0, 30.0, 601).astype(np.float32)
    _, silu, ds = sg.silu_parts(a)
    h = 1e-4
    for ai, si, di in zip(a.astype(np.float64), silu.astype(np.float64), ds.astype(np.float64)):
        assert abs(si - _silu64(ai)) <= 2e-7 * max(1.0, abs(ai))
        fd = (_silu64(ai + h) - _silu64(ai - h)) / (2 * h)
        assert abs(di - fd) <= 2e-6


def test_silu_closed_forms():
    s, silu, ds = sg.silu_parts(np.float32([0.0, 60.0, -60.0]))
    assert s[0] == 0.5 and silu[0] == 0.0 and ds[0] == 0.5
    assert silu[1] == 60.0 and ds[1] == 1.0
    assert abs(silu[2]) < 1e-20 and abs(ds[2]) < 1e-20


def _bf16_exact(v: float) -> int:
    """Nearest bfloat16 (ties to even) of a finite float32 value, by rational arithmetic."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    bits = int(np.float32(v).view(np.uint32))
    lo = bits & 0xFFFF0000
    hi = lo + 0x10000
    f = Fraction(float(np.float32(v)))
    flo = Fraction(float(np.uint32(lo).view(np.float32)))
    fhi = Fraction(float(np.uint32(hi).view(np.float32))) if (hi & 0x7F800000) != 0x7F800000 else None
    if fhi is None:   # rounding up would leave the finite range: inf
        fhi = Fraction(2) ** 128 * (1 if f > 0 else -1)
    dlo, dhi = abs(f - flo), abs(fhi - f)
    if dlo < dhi or (dlo == dhi and (lo >> 16) % 2 == 0):
        return lo >> 16
    return hi >> 16


def test_round_bf16_against_rational_rounding():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.4e38]]).astype(np.float32)
    got = sg.round_bf16(v)
    for x, g in zip(v, got):
        assert int(g) == _bf16_exact(float(x)), float(x)
    assert sg.round_bf16(np.float32([np.nan]))[0] == 0x7FC0


def test_glue_against_float64_textbook_derivative():
    rng = np.random.default_rng(9)
    n = 4000
    dH = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    a = sg.round_bf16(rng.standard_normal(n).astype(np.float32) * 3)
    u = sg.round_bf16(rng.standard_normal(n).astype(np.float32))
    gg, gu = sg.glue(dH, a, u)
    af, uf = sg.bf16_to_f32(a).astype(np.float64), sg.bf16_to_f32(u).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-af))
    ref_up = dH * af * sig
    ref_gate = dH * uf * (sig + af * sig * (1 - sig))
    for got, ref in ((gg, ref_gate), (gu, ref_up)):
        g = sg.bf16_to_f32(got).astype(np.float64)
        assert np.all(np.abs(g - ref) <= 2 ** -8 * np.abs(ref) * 1.01 + 1e-30)
