"""The INT8 quantizer of the backward pass, step by step.  (Oracle: test use only.)

Follows the S3R page, section "Quantized Backpropagation with Stochastic
Rounding":
  * the stochastic rounding operator rounds an element up when its residual
    P = G/Delta - floor(G/Delta) reaches the threshold (eq. (1)); the
    quantizer computes Delta * floor(G/Delta + R), which is (1) with the
    threshold 1 - R;
  * the forward operands are RTNE-quantized with per-token scales s_x and
    per-output-channel scales s_w;
  * the backward pass folds both scales into the gradient,
    G' = diag(s_x) G diag(s_w), takes Delta = max|G'| / 127 and keeps the
    S8 codes Q = SR(G'; R) / Delta (eq. (2)), once for both GEMMs.
and the SR explainer page, "Stochastic rounding, defined" (round up with
probability frac(x/ulp)).

Readings where the text is silent (each is listed with its reason in the
design notes):
  * fold order: G' = fl(fl(G * s_x[t]) * s_w[j]) in fp32; absent scales are 1;
  * step: a = max|G'| (per tensor, or per row for the per-token variant);
    Delta = fl(a / 127), inv = fl(127 / a); a == 0 gives Delta = 1, inv = 0;
  * x = fl(G' * inv) in fp32;
  * RTNE code: rint(x) (ties to even) clamped to [-127, 127];
  * SR / S3R code: floor(x + r), the exact real floor, clamped to [-127, 127]
    (the code -128 is never used: the step is max/127);
  * a non-finite amax sets flag bit 0, an amax so small that 127/a overflows
    fp32 (or 127*2**24/a does) sets flag bit 1; either way the affected
    tensor (or row) gets all-zero codes and zero rounding error.
"""
from __future__ import annotations

import numpy as np

from . import philox

RTNE, SR, S3R, S3R_BCAST = 0, 1, 2, 3
PER_TENSOR, PER_TOKEN = 0, 1
EC_NONE, EC_DX_ONLY, EC_TWO_WAY, EC_DW_ONLY = 0, 1, 2, 3

FLAG_NONFINITE = 1
FLAG_TINY_STEP = 2

F32 = np.float32


def decode(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Stored gradient -> float32 values.  bf16 widens by a 16-bit left shift (exact)."""
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float32)
    if dtype == "bf16":
        return (np.asarray(storage, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def fold(g: np.ndarray, row_scale=None, col_scale=None) -> np.ndarray:
    """G' = diag(s_x) G diag(s_w), as fl(fl(G * s_x[t]) * s_w[j]) in fp32."""
    g = np.asarray(g, dtype=F32)
    T, D = g.shape
    sx = np.ones(T, F32) if row_scale is None else np.asarray(row_scale, F32)
    sw = np.ones(D, F32) if col_scale is None else np.asarray(col_scale, F32)
    with np.errstate(over="ignore", invalid="ignore"):
        return (g * sx[:, None]) * sw[None, :]


def step_from_amax(a: np.ndarray):
    """Delta = fl(a/127) and inv = fl(127/a) per amax value, with flags.

    Returns (delta f32, inv f32, flags uint32), all shaped like ``a``.
    """
    a = np.asarray(a, dtype=F32)
    flags = np.zeros(a.shape, np.uint32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        delta = np.where(a > 0, a / F32(127), F32(1)).astype(F32)
        inv = np.where(a > 0, F32(127) / a, F32(0)).astype(F32)
        inv24 = inv * F32(2.0 ** 24)
    nonfinite = ~np.isfinite(a)
    delta = np.where(np.isnan(a), a, delta).astype(F32)
    flags[nonfinite] |= FLAG_NONFINITE
    tiny = np.isfinite(a) & (a > 0) & ~np.isfinite(inv24)
    flags[tiny] |= FLAG_TINY_STEP
    return delta, inv, flags


def codes_rtne(x: np.ndarray) -> np.ndarray:
    """Round to nearest, ties to even, clamped to the symmetric S8 range."""
    return np.clip(np.rint(x.astype(np.float64)), -127, 127).astype(np.int8)


def floor_plus(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """floor(x + r) on the unit grid (float64 result): the operator Delta*floor(G/Delta + R) / Delta.

    x is fp32 (or any float64 with |x| < 2**28), r a dyadic threshold with at
    most 24 fractional bits.  The sum is taken in float64; it is exact whenever
    |x| >= 2**-23, and for smaller |x| float64 rounding cannot carry x + r across
    an integer, because a nonzero distance from x + r to the nearest integer is
    at least 2**-48 there.  Exact rational arithmetic checks this in the tests.
    """
    s = np.asarray(x, dtype=np.float64) + np.asarray(r, dtype=np.float64)
    return np.floor(s)


def codes_floor_plus(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """S8 codes of SR / S3R: floor(x + r) clamped to [-127, 127]."""
    return np.clip(floor_plus(x, r), -127, 127).astype(np.int8)


def thresholds(mode: int, seed: int, layer_id: int, T: int, D: int, row0: int = 0, rows_per_example=None,
               stream: int = 0):
    """Thresholds r (float64) broadcastable to [T, D] for the stochastic modes.

    SR: one per element; S3R: one per token (Phi_2D); S3R_BCAST: one per
    example of rows_per_example tokens (Phi_bcast).  ``stream`` selects an
    independent draw (0: the tensor shared by both products).
    """
    if mode == SR:
        return philox.sr_thresholds(seed, layer_id, T, D, row0, stream)
    if mode == S3R:
        return philox.s3r_thresholds(seed, layer_id, T, row0, stream)[:, None]
    if mode == S3R_BCAST:
        return philox.bcast_thresholds(seed, layer_id, T, rows_per_example, row0, stream)[:, None]
    raise ValueError(mode)


def quantize(g_store: np.ndarray, dtype: str, *, mode: int, scale: int = PER_TENSOR,
             row_scale=None, col_scale=None, seed: int = 0, layer_id: int = 0,
             rows_per_example: int | None = None, stream: int = 0, row0: int = 0, amax=None) -> dict:
    """Quantize one gradient tensor; returns codes, steps and the fp32 values x.

    ``row0`` is the global index of the first row: thresholds are keyed on the
    global token (element) index, so a slice of rows quantized with its offset
    draws the same thresholds as in the whole tensor.  ``amax`` (per-tensor step
    only) is max|G'| over the whole tensor when ``g_store`` is a slice of it, so
    the slice gets the whole tensor's step; by default it is the slice's own.

    Keys: "Q" int8 [T, D]; "delta" f32 ([1] per tensor, [T] per token);
    "x" f32 [T, D] (G'/Delta as the quantizer sees it, zero where flagged);
    "flags" (OR over rows); "row_flags" [T]; "code_colsum" int64 [B, D].
    """
    g = decode(g_store, dtype)
    T, D = g.shape
    S = rows_per_example or max(T, 1)
    gp = fold(g, row_scale, col_scale)
    if scale == PER_TENSOR:
        if amax is not None:
            a = F32(amax)
        else:
            a = np.max(np.abs(gp)) if gp.size else F32(0)
        delta, inv, fl = step_from_amax(np.array([a], F32))
        inv_rows = np.full(T, inv[0], F32)
        row_flags = np.full(T, fl[0], np.uint32)
    elif scale == PER_TOKEN:
        a = np.max(np.abs(gp), axis=1) if D else np.zeros(T, F32)
        delta, inv, row_flags = step_from_amax(a)
        inv_rows = inv
    else:
        raise ValueError(scale)
    with np.errstate(invalid="ignore", over="ignore"):
        x = (gp * inv_rows[:, None]).astype(F32)
    bad = row_flags != 0
    x[bad] = F32(0)
    if mode == RTNE:
        q = codes_rtne(x)
    else:
        q = codes_floor_plus(x, thresholds(mode, seed, layer_id, T, D, row0=row0, rows_per_example=S,
                                           stream=stream))
    q[bad] = 0
    flags = np.uint32(np.bitwise_or.reduce(row_flags)) if T else np.uint32(0)
    return {"Q": q, "delta": delta.astype(F32), "x": x, "flags": int(flags),
            "row_flags": row_flags, "code_colsum": code_colsums(q, S)}


def code_colsums(q: np.ndarray, rows_per_example: int) -> np.ndarray:
    """Per-example column sums of the codes (exact int64): r_W = W^T 1 or S * x_bar_b.

    S3R page, "Two-Way Correction": the dX term uses the precomputed row sums
    of the weight (W 1_D) and the dW term the per-example input means x_bar_b.
    """
    T, D = q.shape
    S = rows_per_example
    B = T // S if S else 0
    return q.astype(np.int64).reshape(B, S, D).sum(axis=1) if B else np.zeros((0, D), np.int64)


def forward_operand(store: np.ndarray, dtype: str, rows_per_example: int | None = None) -> dict:
    """Forward-pass operand prep: per-row absmax RTNE to S8 (X per token, W per output channel).

    S3R page, "Quantized Backpropagation with Stochastic Rounding": the forward
    product applies RTNE with per-token scales s_x and per-output-channel scales
    s_w.  The step is absmax/127 per row, the same rule as the gradient's step.
    Returns "Q", "scale" (= the row steps, s_x or s_w), "code_colsum".
    """
    out = quantize(store, dtype, mode=RTNE, scale=PER_TOKEN,
                   rows_per_example=rows_per_example)
    return {"Q": out["Q"], "scale": out["delta"], "code_colsum": out["code_colsum"],
            "flags": out["flags"]}
