"""The expert path of a mixture-of-experts layer: grouped quantized backward.  (Oracle: test use only.)

S3R page, Table IV and the MoE paragraph after it: on the MoE models the
correction runs "over the expert-sorted rows".  Each expert is a linear layer
whose backward sees only the rows routed to it; the rows are sorted by expert,
expert e owning rows [offsets[e], offsets[e+1]).  Per expert, this is exactly
the dense path of ``pipeline.linear_backward`` on its rows:

  * the forward operands: the expert inputs X (all rows) RTNE per token, each
    expert's weight W_e [D x d_in] RTNE per output channel; the correction's
    input sums xs_e are the column sums of X's codes over the expert's rows and
    r_W,e the column sums of W_e's codes;
  * one per-tensor step per expert, Delta_e = max |G'_e| / 127, on the folded
    G'_e = diag(s_x) G_e diag(s_w,e);
  * thresholds keyed on the global row index (the readings of the dense path,
    with the expert's first row as the offset), so they do not depend on how
    the rows are grouped;
  * S3R-EC statistics with the expert's rows as one example (its channel means
    over the expert's tokens, its grand mean);
  * dX rows of the expert and its own dW_e.

An expert with no rows has the step 1, zero statistics and dW_e = 0.
"""
from __future__ import annotations

import numpy as np

from . import backward, ec as ecm, quantize as oq


def forward_operands(X, W, dtype: str, offsets):
    """X [R x d_in] per token; W [E x D x d_in] per output channel of each expert.

    Returns (fx, fws, xs): fx as from quantize.forward_operand, fws a list of the
    experts' weight operands, xs int64 [E x d_in] the per-expert column sums of X's codes.
    """
    R = X.shape[0]
    fx = oq.forward_operand(X, dtype, rows_per_example=max(R, 1))
    E = W.shape[0]
    xs = np.stack([fx["Q"][offsets[e]:offsets[e + 1]].astype(np.int64).sum(axis=0) for e in range(E)])
    fws = [oq.forward_operand(W[e], dtype, rows_per_example=W.shape[1]) for e in range(E)]
    return fx, fws, xs


def grouped_backward(inp: dict, *, mode: int, ec: int, seed: int = 0, layer_id: int = 0, fx=None, fws=None,
                     xs=None, experts=None) -> dict:
    """Per-expert quantize, dX and dW for ``inp`` ("G", "X", "W", "dtype", "offsets").

    ``experts`` limits the work to a subset (dX rows and dW of those experts only).
    Returns per-expert lists: "Q", "delta", "eps", "ebar", "mu", "dW", and "dX" [R x d_in]
    (rows of experts outside the subset are left at zero).
    """
    dtype = inp["dtype"]
    off = np.asarray(inp["offsets"], np.int64)
    E = len(off) - 1
    if fx is None:
        fx, fws, xs = forward_operands(inp["X"], inp["W"], dtype, off)
    D = inp["W"].shape[1]
    d_in = inp["X"].shape[1]
    R = inp["G"].shape[0]
    out = {"fx": fx, "fws": fws, "xs": xs, "dX": np.zeros((R, d_in)), "Q": [None] * E, "delta": [None] * E,
           "eps": [None] * E, "ebar": [None] * E, "mu": [None] * E, "dW": [None] * E, "x": [None] * E}
    for e in (range(E) if experts is None else experts):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        fw = fws[e]
        q = oq.quantize(inp["G"][a:b], dtype, mode=mode, scale=oq.PER_TENSOR, row_scale=fx["scale"][a:b],
                        col_scale=fw["scale"], seed=seed, layer_id=layer_id, rows_per_example=max(n, 1), row0=a)
        out["Q"][e], out["delta"][e], out["x"][e] = q["Q"], q["delta"], q["x"]
        if n == 0:
            out["eps"][e], out["ebar"][e], out["mu"][e] = np.zeros(0), np.zeros((1, D)), np.zeros(1)
            out["dW"][e] = np.zeros((D, d_in))
            continue
        E_err = ecm.rounding_error(q["Q"], q["x"], q["delta"])
        eps, ebar, mu = ecm.statistics(E_err, n)
        out["eps"][e], out["ebar"][e], out["mu"][e] = eps, ebar, mu
        out["dX"][a:b] = backward.backward_dx(q["Q"], q["delta"], fw["Q"], fx["scale"][a:b], ec=ec,
                                              r_W=fw["code_colsum"][0], eps=eps, ebar=ebar, mu=mu,
                                              rows_per_example=n)
        out["dW"][e] = backward.backward_dw(q["Q"], q["delta"], fx["Q"][a:b], fw["scale"], ec=ec, xs=xs[e:e + 1],
                                            eps=eps, ebar=ebar, mu=mu, rows_per_example=n)
    return out
