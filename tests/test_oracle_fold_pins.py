"""Pins of the oracle's scale fold and of the rescales that undo it (CPU, no GPU).

S3R page, "Quantized Backpropagation with Stochastic Rounding", eq. (2): the
backward folds the forward scales into the gradient, G' = diag(s_x) G diag(s_w),
quantizes G' once with one step, and rescales the two products by 1/s_x and
1/s_w after the S32 accumulation.  In expectation over the thresholds the
quantized backward therefore reproduces the plain products of the original
gradient with the dequantized forward operands:

    E[dX] = G . (diag(s_w) Wq)      E[dW] = G^T . (diag(s_x) Xq)

Every expected value here is built in float64 from the original G and the
forward codes and steps: never from ``oq.fold`` or the oracle's rescales.  The
scales span three decades and some tokens are outliers, so a fold that divided
instead of multiplying, or a rescale by the wrong operand's scale, moves the
products by far more than the bounds allow (checked below by running the same
criterion on a deliberately wrong reading and requiring it to fail).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import backward, pipeline, quantize as oq


# ------------------------------------------------ exact fp32 rounding ----

def _round_to_f32(v: Fraction) -> float:
    """Round an exact rational to the nearest binary32 value (ties to even), subnormals included."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    m = abs(v)
    # e = floor(log2 m), from the bit lengths, then corrected exactly
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    if Fraction(2) ** (e + 1) <= m:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n, rem = divmod(m, ulp)
    n = int(n)
    if rem * 2 > ulp or (rem * 2 == ulp and n % 2 == 1):
        n += 1
    r = n * ulp
    if r >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(r)


def test_round_to_f32_agrees_with_hardware_on_representable_cases():
    # sanity of the helper itself: the product of two fp32 numbers is exact in float64 when it
    # stays in the normal range, and numpy's fp32 multiply rounds it correctly
    rng = np.random.default_rng(0)
    a = rng.standard_normal(500).astype(np.float32)
    b = rng.standard_normal(500).astype(np.float32)
    for x, y in zip(a, b):
        assert _round_to_f32(Fraction(float(x)) * Fraction(float(y))) == float(np.float32(x) * np.float32(y))
    # halfway cases and the subnormal grid
    assert _round_to_f32(Fraction(1) + Fraction(1, 2 ** 24)) == 1.0
    assert _round_to_f32(Fraction(1) + Fraction(3, 2 ** 24)) == 1.0 + 2.0 ** -22
    assert _round_to_f32(Fraction(3, 2 ** 150)) == 2.0 ** -148
    assert _round_to_f32(Fraction(1, 2 ** 150)) == 0.0
    assert _round_to_f32(Fraction(2) ** 128) == float("inf")


def test_fold_is_two_fp32_products_in_the_stated_order():
    # eq. (2): G' = diag(s_x) G diag(s_w); the reading fixes fl(fl(G * s_x[t]) * s_w[j]).
    # Scales span three decades and more, so products land in the subnormal range too.
    rng = np.random.default_rng(11)
    T, D = 24, 40
    g = (rng.standard_t(3, (T, D)) * 10.0 ** rng.uniform(-38, 2, (T, D))).astype(np.float32)
    g[0, :4] = [0.0, -0.0, 3e38, -1e-45]
    sx = (10.0 ** rng.uniform(-3, 1, T)).astype(np.float32)
    sw = (10.0 ** rng.uniform(-2, 1.5, D)).astype(np.float32)
    sx[1] = 1e-30
    got = oq.fold(g, sx, sw)
    for t in range(T):
        for j in range(D):
            first = _round_to_f32(Fraction(float(g[t, j])) * Fraction(float(sx[t])))
            want = _round_to_f32(Fraction(first) * Fraction(float(sw[j]))) if np.isfinite(first) else first
            assert float(got[t, j]) == want, (t, j, g[t, j], sx[t], sw[j])


# ----------------------------------- end to end: E[dX], E[dW] vs products ----

def _scaled_problem(seed, T, D, K, S):
    """Forward operands whose steps s_x (per token) and s_w (per channel) span three decades."""
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((T, K)) * 10.0 ** rng.uniform(-2, 1, (T, 1))).astype(np.float32)
    W = (0.02 * rng.standard_normal((D, K)) * 10.0 ** rng.uniform(-1.5, 1.5, (D, 1))).astype(np.float32)
    G = (1e-3 * rng.standard_t(3, (T, D))).astype(np.float32)
    G[rng.choice(T, 2, replace=False)] *= 100.0                    # outlier tokens
    fx, fw = pipeline.forward_operands(X, W, "f32", S)
    return dict(G=G, X=X, W=W, fx=fx, fw=fw, S=S)


def _exact_products(pr):
    """float64 E[dX] = G (diag(s_w) Wq), E[dW] = G^T (diag(s_x) Xq) from the original G."""
    g = pr["G"].astype(np.float64)
    sx = pr["fx"]["scale"].astype(np.float64)
    sw = pr["fw"]["scale"].astype(np.float64)
    w_dq = sw[:, None] * pr["fw"]["Q"].astype(np.float64)
    x_dq = sx[:, None] * pr["fx"]["Q"].astype(np.float64)
    return g @ w_dq, g.T @ x_dq


def _backward(pr, *, mode, ec_mode, seed, recip=False, no_rescale=False):
    """One draw of the oracle's quantized backward (quantize once, both products).

    Two planted mistakes, which the pins must reject: ``recip`` runs the same oracle calls on
    the reciprocal scales, fold and rescale alike (the consistent "divide instead of multiply"
    reading); ``no_rescale`` folds the scales in but never divides them out.
    """
    fx, fw = pr["fx"], pr["fw"]
    if recip:
        fx = dict(fx, scale=(1.0 / fx["scale"]).astype(np.float32))
        fw = dict(fw, scale=(1.0 / fw["scale"]).astype(np.float32))
    S = pr["S"]
    q = pipeline.quantize_gradient(pr["G"], "f32", fx, fw, mode=mode, scale=oq.PER_TENSOR, seed=seed,
                                   layer_id=3, rows_per_example=S)
    s_x = np.ones_like(fx["scale"]) if no_rescale else fx["scale"]
    s_w = np.ones_like(fw["scale"]) if no_rescale else fw["scale"]
    dx = backward.backward_dx(q["Q"], q["delta"], fw["Q"], s_x, ec=ec_mode, r_W=fw["code_colsum"][0],
                              eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
    dw = backward.backward_dw(q["Q"], q["delta"], fx["Q"], s_w, ec=ec_mode, xs=fx["code_colsum"],
                              eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
    return q, dx, dw


def _exact_step(pr):
    """max|G s_x s_w| / 127 in float64, widened by the fp32 roundings of the fold and of a/127."""
    g = np.abs(pr["G"].astype(np.float64))
    gp = g * pr["fx"]["scale"].astype(np.float64)[:, None] * pr["fw"]["scale"].astype(np.float64)[None, :]
    return gp.max() / 127 * (1 + 2.0 ** -20)


def _bounds(pr, per_elem, slack_rel=2.0 ** -19):
    """Propagated per-element bounds on dX and dW, for the step of the exact fold.

    A per-element deviation b of Delta*q from G' (bias or rounding) moves dX[t, i] by at most
    sum_j b |Wq[j, i]| / s_x[t] and dW[j, i] by sum_t b |Xq[t, i]| / s_w[j].  ``slack_rel`` covers
    the fp32 roundings of the fold, of x = G' * inv and of Delta * inv = 1 + O(2^-23), relative to
    |G'| = |G s_x s_w|.
    """
    delta = _exact_step(pr)
    g = np.abs(pr["G"].astype(np.float64))
    sx = pr["fx"]["scale"].astype(np.float64)
    sw = pr["fw"]["scale"].astype(np.float64)
    wq = np.abs(pr["fw"]["Q"].astype(np.float64))
    xq = np.abs(pr["fx"]["Q"].astype(np.float64))
    bx = (per_elem * delta) * wq.sum(axis=0)[None, :] / sx[:, None]
    bw = (per_elem * delta) * xq.sum(axis=0)[None, :] / sw[:, None]
    gp = g * sx[:, None] * sw[None, :]
    bx = bx + slack_rel * (gp @ wq) / sx[:, None]
    bw = bw + slack_rel * (gp.T @ xq) / sw[:, None]
    return bx, bw


def _rtne_within_half_step(pr, **mistake):
    q, dx, dw = _backward(pr, mode=oq.RTNE, ec_mode=oq.EC_NONE, seed=0, **mistake)
    ex, ew = _exact_products(pr)
    bx, bw = _bounds(pr, 0.5)
    return bool(np.all(np.abs(dx - ex) <= bx) and np.all(np.abs(dw - ew) <= bw))


def test_rtne_backward_within_half_step_of_exact_products():
    # RTNE: |Delta q - G'| <= Delta/2 per element, so dX and dW lie within the propagated
    # half-step bound of the exact products of the original G.
    for seed in (1, 2, 3):
        pr = _scaled_problem(seed, 16, 24, 12, 8)
        assert _rtne_within_half_step(pr)


@pytest.mark.parametrize("mistake", ["recip", "no_rescale"])
def test_rtne_bound_rejects_planted_mistakes(mistake):
    # the criterion has power: each planted misreading of the fold or the rescale fails it
    pr = _scaled_problem(1, 16, 24, 12, 8)
    assert not _rtne_within_half_step(pr, **{mistake: True})


def _mc_agrees(pr, mode, ec_mode, n, recip=False):
    ex, ew = _exact_products(pr)
    sx_ = np.zeros_like(ex); sxx = np.zeros_like(ex)
    sw_ = np.zeros_like(ew); sww = np.zeros_like(ew)
    for seed in range(n):
        q, dx, dw = _backward(pr, mode=mode, ec_mode=ec_mode, seed=seed, recip=recip)
        sx_ += dx; sxx += dx * dx
        sw_ += dw; sww += dw * dw
    mx, mw = sx_ / n, sw_ / n
    sdx = np.sqrt(np.maximum(sxx / n - mx * mx, 0.0))
    sdw = np.sqrt(np.maximum(sww / n - mw * mw, 0.0))
    # threshold-grid bias per element of Delta*q: 2^-24 Delta (SR), Delta/256 (S3R); the
    # correction adds the projection of that bias, at most three times it elementwise
    bias = 2.0 ** -24 if mode == oq.SR else 1.0 / 256
    if ec_mode != oq.EC_NONE:
        bias *= 4
    bx, bw = _bounds(pr, bias)
    okx = np.abs(mx - ex) <= 5.0 * sdx / np.sqrt(n) + bx
    okw = np.abs(mw - ew) <= 5.0 * sdw / np.sqrt(n) + bw
    return bool(okx.all() and okw.all())


@pytest.mark.parametrize("mode", [oq.SR, oq.S3R])
@pytest.mark.parametrize("ec_mode", [oq.EC_NONE, oq.EC_TWO_WAY])
def test_monte_carlo_backward_equals_exact_products(mode, ec_mode):
    # Lemma 1 (shared thresholds stay unbiased) and "Two-Way Correction" (the correction keeps
    # both gradients unbiased), carried through the fold and the rescales: the mean over seeds
    # of the oracle's dX and dW equals G (diag(s_w) Wq) and G^T (diag(s_x) Xq).
    pr = _scaled_problem(21, 16, 24, 12, 8)
    assert _mc_agrees(pr, mode, ec_mode, 1500)


def test_monte_carlo_criterion_rejects_reciprocal_scales():
    pr = _scaled_problem(21, 16, 24, 12, 8)
    assert not _mc_agrees(pr, oq.S3R, oq.EC_TWO_WAY, 300, recip=True)


def test_per_token_dx_within_half_step_of_exact_product():
    # per-token steps Delta_t: the same fold, one step per row; dX rescales by 1/s_x exactly as
    # in the per-tensor case, so RTNE dX lies within sum_j Delta_t/2 |Wq[j, i]| / s_x[t]
    pr = _scaled_problem(4, 16, 24, 12, 8)
    fx, fw = pr["fx"], pr["fw"]
    q = pipeline.quantize_gradient(pr["G"], "f32", fx, fw, mode=oq.RTNE, scale=oq.PER_TOKEN, seed=0,
                                   layer_id=0, rows_per_example=pr["S"])
    dx = backward.backward_dx(q["Q"], q["delta"], fw["Q"], fx["scale"])
    ex, _ = _exact_products(pr)
    d_t = q["delta"].astype(np.float64)
    wq = np.abs(fw["Q"].astype(np.float64))
    sx = fx["scale"].astype(np.float64)
    g = np.abs(pr["G"].astype(np.float64)) * sx[:, None] * fw["scale"].astype(np.float64)[None, :]
    bound = (0.5 * d_t[:, None] * wq.sum(axis=0)[None, :] + 2.0 ** -19 * (g @ wq)) / sx[:, None]
    assert np.all(np.abs(dx - ex) <= bound)
