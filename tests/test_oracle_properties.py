"""Property tests of the oracle (hypothesis): random shapes, zero rows and outlier tokens.

What they hold the oracle to is fixed by the pages and by arithmetic, not by the oracle itself:
- every stochastic code is floor(x) or floor(x) + 1 and RTNE is round-half-even (S3R page, eq. (1) and its
  reading Delta*floor(G/Delta + R)), all within the symmetric S8 range;
- an all-zero token gives zero codes; per-tensor steps put the largest magnitude on +-127;
- S3R rounds every element of a token with the same residual the same way, and rounds up exactly those whose
  residual reaches 1 - r_t (S3R page, "Structured Subspace Stochastic Rounding");
- thresholds are keyed on global indices, so a band of rows quantized with its row offset equals the same rows
  of the whole tensor (the partitionable generator the pages rely on);
- after the two-way correction the remaining error sums to zero along every token and along every channel of
  each example (S3R page, "Two-Way Correction").
"""
import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import ec, quantize as oq

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def gradients(draw):
    B = draw(st.integers(1, 3))
    S = draw(st.integers(1, 6))
    D = draw(st.integers(1, 40))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    g = (rng.standard_t(3.0, size=(B * S, D)) * 10.0 ** draw(st.integers(-6, 2))).astype(np.float32)
    if draw(st.booleans()):
        g[rng.integers(0, B * S)] = 0.0                       # a zero token
    if draw(st.booleans()):
        g[rng.integers(0, B * S)] *= np.float32(1e4)          # an outlier token
    return g, S


MODES = st.sampled_from([oq.RTNE, oq.SR, oq.S3R])
SCALES = st.sampled_from([oq.PER_TENSOR, oq.PER_TOKEN])


@SETTINGS
@given(gradients(), MODES, SCALES, st.integers(0, 2 ** 32 - 1))
def test_codes_are_floor_or_ceil_and_in_range(gs, mode, scale, seed):
    g, S = gs
    r = oq.quantize(g, "f32", mode=mode, scale=scale, seed=seed, rows_per_example=S)
    q = r["Q"].astype(np.int64)
    x = r["x"].astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    if mode == oq.RTNE:
        assert np.array_equal(q, np.clip(np.rint(x), -127, 127))
    else:
        lo = np.clip(np.floor(x), -127, 127)
        hi = np.clip(np.floor(x) + 1, -127, 127)
        assert np.all((q == lo) | (q == hi))
    zero_rows = ~np.any(g != 0, axis=1)
    assert np.all(q[zero_rows] == 0)
    if scale == oq.PER_TENSOR and np.any(g != 0):
        assert np.max(np.abs(x)) == 127.0 or abs(np.max(np.abs(x)) - 127.0) <= 127.0 * 2.0 ** -23


@SETTINGS
@given(gradients(), st.integers(0, 2 ** 32 - 1))
def test_s3r_rounds_up_exactly_the_residuals_reaching_its_token_threshold(gs, seed):
    g, S = gs
    r = oq.quantize(g, "f32", mode=oq.S3R, seed=seed, rows_per_example=S)
    x = r["x"].astype(np.float64)
    up = r["Q"].astype(np.float64) > np.floor(x)
    rt = oq.thresholds(oq.S3R, seed, 0, *g.shape)[:, 0]
    frac = x - np.floor(x)
    inside = np.abs(x) < 126                                   # away from the clamp
    for t in range(g.shape[0]):
        m = inside[t]
        assert np.array_equal(up[t][m], (frac[t][m] >= 1.0 - rt[t]))


@SETTINGS
@given(gradients(), st.sampled_from([oq.SR, oq.S3R]), st.integers(0, 2 ** 32 - 1), st.data())
def test_a_band_with_its_row_offset_equals_the_whole(gs, mode, seed, data):
    g, S = gs
    T = g.shape[0]
    k = data.draw(st.integers(0, T - 1))
    whole = oq.quantize(g, "f32", mode=mode, scale=oq.PER_TOKEN, seed=seed, rows_per_example=S)
    band = oq.quantize(g[k:], "f32", mode=mode, scale=oq.PER_TOKEN, seed=seed, rows_per_example=1, row0=k)
    assert np.array_equal(band["Q"], whole["Q"][k:])


@SETTINGS
@given(gradients(), SCALES, st.integers(0, 2 ** 32 - 1))
def test_corrected_error_sums_to_zero_per_token_and_per_example_channel(gs, scale, seed):
    g, S = gs
    r = oq.quantize(g, "f32", mode=oq.S3R, scale=scale, seed=seed, rows_per_example=S)
    E = ec.rounding_error(r["Q"], r["x"], r["delta"])
    eps, ebar, mu = ec.statistics(E, S)
    R = E - ec.projection(eps, ebar, mu, S)
    T, D = g.shape
    tol = 1e-9 * max(1.0, float(np.abs(E).max()) * D * S)
    assert np.all(np.abs(R.sum(axis=1)) <= tol)
    assert np.all(np.abs(R.reshape(T // S, S, D).sum(axis=1)) <= tol)
