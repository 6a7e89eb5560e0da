"""The two INT8 backward GEMMs and their dequantisation.  (Oracle: test use only.)

S3R page, "Quantized Backpropagation with Stochastic Rounding": the backward
pass computes the activation gradient G W^T and the weight gradient X^T G;
in the INT8 pipeline each is an S8 x S8 GEMM with S32 accumulation followed by
a rescale.  One S8 tensor Q feeds both, so one step Delta applies after the
accumulation; the fixed rescalings by 1/s_x and 1/s_w undo the fold.

Layouts (the weight is stored [D x d_in], the page's W^T):
    Q  [T x D]  int8   gradient codes
    Wq [D x d_in] int8 forward weight codes, s_w [D] their per-row steps
    Xq [T x d_in] int8 forward input codes, s_x [T] their per-row steps

    acc_dX = Q  @ Wq   (int, contracted over D)
    acc_dW = Q^T @ Xq  (int, contracted over T)

S3R-EC ("Two-Way Correction"): from the activation gradient subtract the
averages times the weight, which for the token means is the mean times the
precomputed row sums r_W = Wq^T 1; from the weight gradient subtract the
inputs times the same averages (per example, x_bar_b e_b^T with e_b the
channel-mean error and S x_bar_b the per-example input column sums xs_b):

    dX[t, i] = (Delta_t * acc_dX[t, i] - v_b[i] - (eps_t - mu_b) * r_W[i]) / s_x[t]
        v_b   = ebar_b @ Wq
    dW[j, i] = (Delta * acc_dW[j, i] - sum_b (ebar_b[j] * xs_b[i] + u_b[i])) / s_w[j]
        u_b   = sum_{t in b} (eps_t - mu_b) * Xq[t, :]

"Cost and the dX-Only Variant": the dX-only variant keeps only the activation
gradient's term.  The ablation of Table II ("dW-only corr.") keeps only the
weight gradient's term (EC_DW_ONLY).  Everything is float64; integer products are exact.

Per-token steps and dW (a reading beyond the pages).  The S3R page explains
that only a per-tensor step can be applied after the S32 accumulation of the
weight gradient, whose contraction runs over the tokens.  With one step
Delta_t per token the exact product is Q^T diag(Delta) Xq.  This oracle takes
the plainest realisation that keeps an S8 x S8 GEMM: fold the steps into the
input codes, Z = diag(Delta) Xq (fp32 products), and RTNE-requantize Z per
input column with the absmax rule of the forward operands, c_i = max_t |Z|/127.
Then acc' = Q^T Zq is exact in integers and

    dW[j, i] = (c_i * acc'[j, i] - sum_b (ebar_b[j] * xs_b[i] + u_b[i])) / s_w[j].
"""
from __future__ import annotations

import numpy as np

from .quantize import EC_NONE, EC_DX_ONLY, EC_TWO_WAY, EC_DW_ONLY  # noqa: F401
from .quantize import codes_rtne, step_from_amax


def int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact integer product of two int8 matrices, returned as int64.

    Computed as a float64 BLAS product: every partial sum is an integer of
    magnitude <= K * 127**2 < 2**53, so any summation order is exact.
    """
    K = a.shape[1]
    assert K * 127 * 127 < 2 ** 53
    out = a.astype(np.float64) @ b.astype(np.float64)
    return out.astype(np.int64)


def _delta_rows(delta: np.ndarray, rows: np.ndarray) -> np.ndarray:
    d = np.asarray(delta, dtype=np.float64)
    return np.full(rows.size, d[0]) if d.size == 1 else d[rows]


def backward_dx(Q, delta, Wq, s_x, *, ec=EC_NONE, r_W=None, eps=None, ebar=None, mu=None,
                rows_per_example=None, rows=None) -> np.ndarray:
    """Dequantised (and, for EC_DX_ONLY or EC_TWO_WAY, corrected) dX [len(rows), d_in] in float64.

    ``rows`` selects output rows (tokens); default all.  Rows are independent,
    so a sample is computed exactly as the full result would be.
    """
    T = Q.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    acc = int_matmul(Q[rows], Wq).astype(np.float64)
    out = _delta_rows(delta, rows)[:, None] * acc
    if ec in (EC_DX_ONLY, EC_TWO_WAY):
        S = rows_per_example
        b = rows // S
        v = np.asarray(ebar, np.float64) @ Wq.astype(np.float64)         # [B, d_in]
        c = np.asarray(eps, np.float64)[rows] - np.asarray(mu, np.float64)[b]
        out -= v[b] + c[:, None] * np.asarray(r_W, np.float64)[None, :]
    return out / np.asarray(s_x, np.float64)[rows][:, None]


def backward_dw(Q, delta, Xq, s_w, *, ec=EC_NONE, xs=None, eps=None, ebar=None, mu=None,
                rows_per_example=None, rows=None) -> np.ndarray:
    """Dequantised (and, for EC_TWO_WAY or EC_DW_ONLY, corrected) dW [len(rows), d_in] in float64.

    ``rows`` selects output rows (channels j of the gradient).  Requires a
    per-tensor step (one Delta for the whole of Q).
    """
    d = np.asarray(delta, dtype=np.float64)
    assert d.size == 1, "dW needs one per-tensor step"
    D = Q.shape[1]
    rows = np.arange(D) if rows is None else np.asarray(rows)
    acc = int_matmul(np.ascontiguousarray(Q[:, rows].T), Xq).astype(np.float64)
    out = d[0] * acc
    if ec in (EC_TWO_WAY, EC_DW_ONLY):
        out -= _dw_correction(Q.shape[0], Xq, xs, eps, ebar, mu, rows_per_example, rows)
    return out / np.asarray(s_w, np.float64)[rows][:, None]


def requantize_columns(Xq, delta_t):
    """(Zq int8 [T, d_in], c f32 [d_in]): Z = fl32(Delta_t * Xq[t, i]) RTNE-quantized per column.

    Step per column: a_i = max_t |Z[t, i]|, c_i = fl(a_i / 127), inv_i = fl(127 / a_i)
    (a_i == 0: c_i = 1, inv_i = 0), the rule of the forward operands.  Codes:
    rint(fl(Z * inv_i)) (ties to even) clamped to [-127, 127].  A column whose
    a_i or inv_i is not finite (a non-finite or subnormal-range step) gets zero
    codes; its c_i is the non-finite a_i or fl(a_i / 127) as usual.
    """
    F32 = np.float32
    X = np.asarray(Xq, dtype=F32)
    d = np.asarray(delta_t, dtype=F32).reshape(-1)
    with np.errstate(over="ignore", invalid="ignore"):
        Z = (d[:, None] * X).astype(F32)
    T, N = Z.shape
    a = np.abs(Z).max(axis=0) if T else np.zeros(N, F32)
    c, inv, _ = step_from_amax(a)
    with np.errstate(over="ignore", invalid="ignore"):
        x = (Z * inv[None, :]).astype(F32)
    bad = ~np.isfinite(a) | ~np.isfinite(inv)
    x[:, bad] = F32(0)
    return codes_rtne(x), c.astype(F32)


def backward_dw_per_token(Q, delta_t, Xq, s_w, *, ec=EC_NONE, xs=None, eps=None, ebar=None, mu=None,
                          rows_per_example=None, rows=None) -> np.ndarray:
    """dW [len(rows), d_in] (float64) for per-token steps Delta_t, via the per-column requantized Z.

    The correction terms (EC_TWO_WAY, EC_DW_ONLY) are those of the per-tensor case: the
    statistics already carry Delta_t (E' = Delta_t (q - x)), and the inputs enter
    through their exact codes Xq.
    """
    D = Q.shape[1]
    rows = np.arange(D) if rows is None else np.asarray(rows)
    Zq, c = requantize_columns(Xq, delta_t)
    acc = int_matmul(np.ascontiguousarray(Q[:, rows].T), Zq).astype(np.float64)
    out = c.astype(np.float64)[None, :] * acc
    if ec in (EC_TWO_WAY, EC_DW_ONLY):
        out -= _dw_correction(Q.shape[0], Xq, xs, eps, ebar, mu, rows_per_example, rows)
    return out / np.asarray(s_w, np.float64)[rows][:, None]


def _dw_correction(T, Xq, xs, eps, ebar, mu, S, rows):
    """sum_b (ebar_b[j] xs_b[i] + u_b[i]) for the channels j in ``rows``, float64."""
    B = T // S
    eb = np.asarray(ebar, np.float64)[:, rows]                        # [B, n]
    xsf = np.asarray(xs, np.float64)                                  # [B, d_in]
    c = np.asarray(eps, np.float64) - np.repeat(np.asarray(mu, np.float64), S)
    u = np.stack([c[b * S:(b + 1) * S] @ Xq[b * S:(b + 1) * S].astype(np.float64)
                  for b in range(B)])                                 # [B, d_in]
    return eb.T @ xsf + u.sum(axis=0)[None, :]
