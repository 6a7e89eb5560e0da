"""MXFP4 variant of the quantized backward.  (Oracle: test use only.)

The S3R page names 4-bit formats (NVFP4 and MXFP4) as the setting in which
the backward pass suffers most from deterministic rounding (Introduction;
Related Work), but defines none of their arithmetic.  This module takes the
plainest reading: the OCP Microscaling (MX) formats with the S3R page's
stochastic rounding and correction carried over.

Format (OCP MX, MXFP4):
  * elements E2M1: sign, 2 exponent bits, 1 mantissa bit; magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6; code = sign << 3 | index into that list;
    two elements per byte, the first in the low nibble;
  * one E8M0 scale per block of 32 consecutive elements along the
    contraction dimension: byte b means 2^(b - 127); 255 is NaN.

Readings (none of this is fixed by the pages):
  * scale: the smallest power of two 2^k with max|block| <= 6 * 2^k (so
    nothing saturates and rounding stays unbiased), k clamped to
    [-127, 127]; an all-zero block takes k = -127; a non-finite max gives
    the NaN scale (byte 255) and zero codes, with a flag;
  * rounding of y = g / 2^k (exact) onto the E2M1 grid: with the grid
    spacing s at |y| (0.5 below 2, 1 below 4, 2 from 4 to 6),
    RTNE: s * rint(y / s), ties to even, which is ties to the even
    mantissa; SR and S3R: s * floor(y / s + r), the exact floor (as in the
    INT8 path), r the threshold of the element from the same Philox maps
    (per element for SR, per token for S3R);
  * the contraction of each GEMM must run along the blocks, so G is
    quantized twice: Q_h with blocks along the hidden dimension for dX, and
    Q_t with blocks along the tokens for dW; both use the same thresholds
    R (the page's one threshold tensor for both products);
  * the forward operands are RTNE MXFP4: W with blocks along D (dX's
    contraction), X with blocks along T (dW's contraction);
  * no per-token or per-channel scale folding: the block scales replace it;
  * the correction (S3R-EC) is taken per quantization on its error
    E = dequant(Q) - G, with the dense path's statistics and projection:
      dX = dq(Q_h) dq(W) - v_b - (eps_t - mu_b) r_W,  v_b = ebar_b dq(W),
           r_W = the column sums of dq(W);
      dW = dq(Q_t)^T dq(X) - sum_b ebar'_b[j] xs_b[i] - u'[i],
           xs_b = per-example column sums of dq(X),
           u' = sum_t (eps'_t - mu'_b) dq(X)[t, :]
    (primes: the statistics of Q_t's error).
"""
from __future__ import annotations

import numpy as np

from . import ec as ecm, philox, quantize as oq

F32 = np.float32
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32
E8M0_NAN = 255


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Grid values (exact) -> 4-bit codes (uint8)."""
    v = np.asarray(v, np.float64)
    mag = np.abs(v)
    idx = np.searchsorted(GRID, mag)
    assert np.all(GRID[np.minimum(idx, 7)] == mag), "not an E2M1 value"
    return ((np.signbit(v) & (mag > 0)).astype(np.uint8) << 3) | idx.astype(np.uint8)


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, np.uint8)
    return np.where(c & 8, -1.0, 1.0) * GRID[c & 7]


def scale_exponent(amax: np.ndarray):
    """(k int64, flag bool): the smallest k with amax <= 6 * 2^k, clamped to [-127, 127]."""
    a = np.asarray(amax, np.float64)
    bad = ~np.isfinite(a)
    m, E = np.frexp(np.where(bad | (a == 0), 1.0, a))       # a = m 2^E, m in [0.5, 1)
    k = np.where(m <= 0.75, E - 3, E - 2)                     # 6 * 2^(E-3) = 0.75 * 2^E
    k = np.where(a == 0, -127, k)
    return np.clip(k, -127, 127).astype(np.int64), bad


def round_e2m1(y: np.ndarray, r=None) -> np.ndarray:
    """Round |y| <= 6 (float64 values of fp32 numbers) onto the E2M1 grid.

    r None: RTNE (ties to the even mantissa); else the exact floor(y / s + r).
    """
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    s = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    if r is None:
        q = s * np.rint(y / s)
    else:
        q = s * oq.floor_plus(y / s, r)
    return q


def thresholds(mode: int, seed: int, layer_id: int, T: int, D: int, stream: int = 0):
    """Per-element thresholds [T, D] of G's elements (row-major index t * D + j), or None (RTNE)."""
    if mode == oq.RTNE:
        return None
    if mode == oq.SR:
        return philox.sr_thresholds(seed, layer_id, T, D, stream=stream)
    if mode == oq.S3R:
        return np.repeat(philox.s3r_thresholds(seed, layer_id, T, stream=stream)[:, None], D, axis=1)
    raise ValueError(mode)


def quantize(M: np.ndarray, axis: int, r=None) -> dict:
    """MXFP4 of the fp32 matrix M [R x C] with blocks of 32 along ``axis`` (0: rows, 1: columns).

    r: thresholds shaped like M (or None for RTNE).  Returns "deq" (float64, like M),
    "codes" (E2M1 codes, uint8, like M), "kexp" (block exponents), "flag".  The blocked
    dimension must be a multiple of 32.
    """
    M = np.asarray(M, F32)
    X = M if axis == 1 else M.T
    Rr = None if r is None else (np.asarray(r, np.float64) if axis == 1 else np.asarray(r, np.float64).T)
    R_, C = X.shape
    assert C % BLOCK == 0
    Xb = X.reshape(R_, C // BLOCK, BLOCK).astype(np.float64)
    with np.errstate(invalid="ignore"):
        amax = np.abs(Xb).max(axis=2) if C else np.zeros((R_, 0))
    k, bad = scale_exponent(amax)
    y = Xb * np.ldexp(1.0, -k)[:, :, None]                    # exact: a power-of-two scaling
    y = np.where(bad[:, :, None], 0.0, y)
    if Rr is not None:
        Rr = Rr.reshape(R_, C // BLOCK, BLOCK)
    q = round_e2m1(y, Rr)
    q = np.where(bad[:, :, None], 0.0, q)
    deq = q * np.ldexp(1.0, k)[:, :, None]
    deq = np.where(bad[:, :, None], np.nan, deq)
    codes = e2m1_encode(q).reshape(R_, C)
    sbyte = np.where(bad, E8M0_NAN, k + 127).astype(np.uint8)
    deq = deq.reshape(R_, C)
    if axis == 0:
        deq, codes = deq.T, codes.T
    return {"deq": deq, "codes": codes, "scale": sbyte, "flag": bool(bad.any())}


def pack(codes: np.ndarray) -> np.ndarray:
    """[R x C] 4-bit codes -> [R x C/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def backward(G, X, W, *, mode: int, ec: int, rows_per_example: int, seed: int = 0, layer_id: int = 0,
             stream: int = 0, dx_rows=None, dw_rows=None, cols=None) -> dict:
    """The MXFP4 quantized backward of one linear layer (fp32 inputs G [T x D], X [T x d_in], W [D x d_in]).

    dx_rows / dw_rows select rows of dX / dW, cols the columns (inputs) of both:
    W's blocks run along D and X's along T, so a column of either is quantized
    on its own and the selection changes no value.
    """
    if cols is not None:
        cols = np.asarray(cols)
        X, W = np.asarray(X)[:, cols], np.asarray(W)[:, cols]
    G = np.asarray(G, F32)
    T, D = G.shape
    S = rows_per_example
    r = thresholds(mode, seed, layer_id, T, D, stream)
    qh = quantize(G, axis=1, r=r)               # blocks along D: the dX operand
    qt = quantize(G, axis=0, r=r)               # blocks along T: the dW operand
    fw = quantize(W, axis=0)                    # W [D x d_in], blocks along D
    fx = quantize(X, axis=0)                    # X [T x d_in], blocks along T
    Wd, Xd, Gd = fw["deq"], fx["deq"], G.astype(np.float64)
    out = {"qh": qh, "qt": qt, "fw": fw, "fx": fx}
    for name, q in (("h", qh), ("t", qt)):
        st = ecm.statistics(q["deq"] - Gd, S)
        out["eps_" + name], out["ebar_" + name], out["mu_" + name] = st
    dx_rows = np.arange(T) if dx_rows is None else np.asarray(dx_rows)
    dw_rows = np.arange(D) if dw_rows is None else np.asarray(dw_rows)
    dX = qh["deq"][dx_rows] @ Wd
    if ec in (oq.EC_DX_ONLY, oq.EC_TWO_WAY):
        b = dx_rows // S
        v = out["ebar_h"] @ Wd
        rW = Wd.sum(axis=0)
        dX = dX - v[b] - (out["eps_h"][dx_rows] - out["mu_h"][b])[:, None] * rW[None, :]
    dW = qt["deq"][:, dw_rows].T @ Xd
    if ec in (oq.EC_TWO_WAY, oq.EC_DW_ONLY):
        B = T // S
        xs = Xd.reshape(B, S, -1).sum(axis=1)
        c = out["eps_t"] - np.repeat(out["mu_t"], S)
        u = c @ Xd
        dW = dW - out["ebar_t"][:, dw_rows].T @ xs - u[None, :]
    out["dX"], out["dW"] = dX, dW
    return out
