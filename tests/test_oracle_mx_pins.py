"""Pins for the MXFP4 oracle (oracle/mx.py) against the format's definition and exact arithmetic (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ec, mx, philox, quantize as oq


def test_e2m1_codes_follow_the_bit_layout():
    # sign, 2 exponent bits, 1 mantissa bit (bias 1; exponent 0 is subnormal: 0 and 0.5)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (0.5 * m) if e == 0 else (1 + 0.5 * m) * 2.0 ** (e - 1)
        v = -v if s else v
        assert mx.e2m1_decode(np.array([c], np.uint8))[0] == v
        if v != 0 or c == 0:
            assert mx.e2m1_encode(np.array([v]))[0] == c


def test_scale_is_the_smallest_non_saturating_power_of_two():
    rng = np.random.default_rng(1)
    a = np.concatenate([np.float32(2.0) ** rng.uniform(-140, 120, 2000).astype(np.float32),
                        [6.0, 12.0, 3.0, 3.0000002, 5.9999995, 1.0, 0.75, 2.0 ** -149, 2.0 ** -126]]).astype(np.float32)
    k, bad = mx.scale_exponent(a)
    assert not bad.any()
    for ai, ki in zip(a.astype(np.float64), k):
        A = Fraction(float(ai))
        if -127 < ki < 127:
            assert A <= 6 * Fraction(2) ** int(ki) and A > 6 * Fraction(2) ** (int(ki) - 1)
        elif ki == -127:
            assert A <= 6 * Fraction(2) ** -127
    k, bad = mx.scale_exponent(np.array([np.inf, np.nan, 0.0]))
    assert bad[0] and bad[1] and not bad[2] and k[2] == -127


def _grid_signed():
    return np.concatenate([-mx.GRID[:0:-1], mx.GRID])


def test_rtne_is_nearest_grid_value_ties_to_even_mantissa():
    rng = np.random.default_rng(2)
    grid = _grid_signed()
    y = np.concatenate([rng.uniform(-6, 6, 5000), (grid[1:] + grid[:-1]) / 2, grid])
    q = mx.round_e2m1(y)
    for yi, qi in zip(y, q):
        d = np.abs(grid - yi)
        best = grid[d == d.min()]
        if len(best) == 1:
            assert qi == best[0]
        else:   # a tie: the value whose code has mantissa bit 0
            even = [b for b in best if mx.e2m1_encode(np.array([b]))[0] & 1 == 0]
            assert qi == even[0]


def test_stochastic_rounding_is_the_exact_threshold_rule():
    # q is one of the two grid neighbours of y and equals the upper one exactly when
    # (y - lo) / (hi - lo) >= 1 - r (exact rationals), with r on the 7-bit and 23-bit grids
    rng = np.random.default_rng(3)
    grid = _grid_signed()
    y = rng.uniform(-6, 6, 4000).astype(np.float32).astype(np.float64)
    r = np.where(rng.random(4000) < 0.5, (2 * rng.integers(0, 128, 4000) + 1) / 256.0,
                 (2 * rng.integers(0, 2 ** 23, 4000) + 1) / 2.0 ** 24)
    q = mx.round_e2m1(y, r)
    for yi, ri, qi in zip(y, r, q):
        lo = grid[grid <= yi].max()
        if lo == yi:
            assert qi == yi
            continue
        hi = grid[grid > yi].min()
        p = (Fraction(float(yi)) - Fraction(float(lo))) / (Fraction(float(hi)) - Fraction(float(lo)))
        assert qi == (hi if p >= 1 - Fraction(float(ri)) else lo)


def test_quantize_axis_transposes_and_bounds_error():
    rng = np.random.default_rng(4)
    M = (rng.standard_t(3, (64, 96)) * 1e-3).astype(np.float32)
    a = mx.quantize(M, axis=0)
    b = mx.quantize(M.T.copy(), axis=1)
    np.testing.assert_array_equal(a["deq"], b["deq"].T)
    np.testing.assert_array_equal(a["codes"], b["codes"].T)
    np.testing.assert_array_equal(a["scale"], b["scale"])
    # RTNE error at most half the spacing at the scaled value, which is at most 1 (at |y| in [4, 6])
    k = a["scale"].astype(np.int64) - 127                       # [96 columns, 2 blocks]
    step = np.repeat(np.ldexp(1.0, k).T, 32, axis=0)             # [64, 96]
    assert np.all(np.abs(a["deq"] - M) <= step * 1.0 + 0)
    # the block maximum is never clipped
    assert np.all(np.abs(a["deq"]).reshape(2, 32, 96).max(axis=1) <= 6 * np.ldexp(1.0, k).T)


@pytest.mark.parametrize("mode", [oq.SR, oq.S3R])
def test_mx_stochastic_rounding_unbiased(mode):
    # Lemma 1 carried to the E2M1 grid: E[dq(Q)] = G up to the threshold grid's bias
    rng = np.random.default_rng(5)
    G = (rng.standard_t(3, (8, 64)) * 1e-3).astype(np.float32)
    n = 2000
    acc = np.zeros(G.shape)
    for seed in range(n):
        r = mx.thresholds(mode, seed, 0, 8, 64)
        acc += mx.quantize(G, axis=1, r=r)["deq"]
    k = mx.quantize(G, axis=1)["scale"].astype(np.int64) - 127
    unit = np.repeat(np.ldexp(1.0, k), 32, axis=1)              # 2^k per element; spacing <= 2 * 2^k
    bias = 2 * unit * (1 / 256 if mode == oq.S3R else 2.0 ** -24)
    tol = 4.5 * (2 * unit) * 0.5 / np.sqrt(n) + bias
    assert np.all(np.abs(acc / n - G) < tol)


def test_mx_backward_correction_and_dense_forms():
    # the corrected products equal the dense projection forms, and what remains of each
    # quantization's error sums to zero along rows and per-example columns
    rng = np.random.default_rng(6)
    T, D, K, S = 64, 64, 32, 32
    G = (rng.standard_t(3, (T, D)) * 1e-3).astype(np.float32)
    X = rng.standard_normal((T, K)).astype(np.float32)
    W = (0.02 * rng.standard_normal((D, K))).astype(np.float32)
    o = mx.backward(G, X, W, mode=oq.S3R, ec=oq.EC_TWO_WAY, rows_per_example=S, seed=2)
    Gd = G.astype(np.float64)
    for nm, q in (("h", o["qh"]), ("t", o["qt"])):
        P = ec.projection(o["eps_" + nm], o["ebar_" + nm], o["mu_" + nm], S)
        rem = q["deq"] - P - Gd
        np.testing.assert_allclose(rem.sum(axis=1), 0, atol=1e-12)
        np.testing.assert_allclose(rem.reshape(T // S, S, D).sum(axis=1), 0, atol=1e-12)
    Ph = ec.projection(o["eps_h"], o["ebar_h"], o["mu_h"], S)
    Pt = ec.projection(o["eps_t"], o["ebar_t"], o["mu_t"], S)
    np.testing.assert_allclose(o["dX"], (o["qh"]["deq"] - Ph) @ o["fw"]["deq"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o["dW"], (o["qt"]["deq"] - Pt).T @ o["fx"]["deq"], rtol=1e-12, atol=1e-15)


def test_mx_thresholds_are_the_int8_paths():
    r = mx.thresholds(oq.S3R, 5, 3, 40, 64)
    np.testing.assert_array_equal(r[:, 7], philox.s3r_thresholds(5, 3, 40))
    np.testing.assert_array_equal(mx.thresholds(oq.SR, 5, 3, 4, 64), philox.sr_thresholds(5, 3, 4, 64))


def test_pack_low_nibble_first():
    c = np.array([[1, 2, 15, 8]], np.uint8)
    np.testing.assert_array_equal(mx.pack(c), np.array([[0x21, 0x8F]], np.uint8))


def test_mx_backward_selection_changes_no_value():
    # selecting rows of dX / dW and columns of both equals slicing the full result
    rng = np.random.default_rng(8)
    T, D, K, S = 64, 64, 48, 32
    G = (rng.standard_t(3, (T, D)) * 1e-3).astype(np.float32)
    X = rng.standard_normal((T, K)).astype(np.float32)
    W = (0.02 * rng.standard_normal((D, K))).astype(np.float32)
    full = mx.backward(G, X, W, mode=oq.SR, ec=oq.EC_TWO_WAY, rows_per_example=S, seed=1)
    rows, cr, cols = np.array([0, 33, 63]), np.array([5, 40]), np.array([1, 17, 47])
    part = mx.backward(G, X, W, mode=oq.SR, ec=oq.EC_TWO_WAY, rows_per_example=S, seed=1, dx_rows=rows,
                       dw_rows=cr, cols=cols)
    np.testing.assert_allclose(part["dX"], full["dX"][np.ix_(rows, cols)], rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(part["dW"], full["dW"][np.ix_(cr, cols)], rtol=1e-13, atol=1e-18)
