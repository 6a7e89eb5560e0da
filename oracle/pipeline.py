"""The whole backward of one quantized linear layer, composed from the oracle steps.

(Oracle: test use only.)  Order follows the S3R page's pipeline (section
"Quantized Backpropagation with Stochastic Rounding", Figure 1): forward
operands X and W are RTNE-quantized per row; the backward folds their scales
into G, quantizes once, feeds the same codes to both GEMMs and rescales;
S3R-EC ("Two-Way Correction", "Cost and the dX-Only Variant") subtracts the
structured part of the rounding error from dX (both variants) and dW (two-way).
"""
from __future__ import annotations

import numpy as np

from . import backward, ec as ecm, quantize as oq


def forward_operands(X, W, dtype: str, rows_per_example: int):
    """RTNE per-row quantization of X (per token) and W (per output channel)."""
    fx = oq.forward_operand(X, dtype, rows_per_example=rows_per_example)
    fw = oq.forward_operand(W, dtype, rows_per_example=W.shape[0])
    return fx, fw


def quantize_gradient(G, dtype: str, fx, fw, *, mode: int, scale: int, seed: int, layer_id: int,
                      rows_per_example: int, stream: int = 0) -> dict:
    """Quantize G' = diag(s_x) G diag(s_w) once, with the S3R-EC statistics."""
    q = oq.quantize(G, dtype, mode=mode, scale=scale, row_scale=fx["scale"], col_scale=fw["scale"],
                    seed=seed, layer_id=layer_id, rows_per_example=rows_per_example, stream=stream)
    E = ecm.rounding_error(q["Q"], q["x"], q["delta"])
    q["eps"], q["ebar"], q["mu"] = ecm.statistics(E, rows_per_example)
    return q


def linear_backward(inp: dict, *, mode: int, ec: int, scale: int = oq.PER_TENSOR, seed: int = 0,
                    layer_id: int = 0, rows_per_example: int, dx_rows=None, dw_rows=None,
                    fx=None, fw=None) -> dict:
    """Forward-operand prep, quantizer, dX and dW for the inputs ``inp`` ("G", "X", "W", "dtype").

    dx_rows / dw_rows select output rows (tokens / channels); None computes all.
    """
    dtype = inp["dtype"]
    S = rows_per_example
    if fx is None or fw is None:
        fx, fw = forward_operands(inp["X"], inp["W"], dtype, S)
    q = quantize_gradient(inp["G"], dtype, fx, fw, mode=mode, scale=scale, seed=seed, layer_id=layer_id,
                          rows_per_example=S)
    out = {"fx": fx, "fw": fw, "q": q}
    out["dX"] = backward.backward_dx(q["Q"], q["delta"], fw["Q"], fx["scale"], ec=ec,
                                     r_W=fw["code_colsum"][0], eps=q["eps"], ebar=q["ebar"], mu=q["mu"],
                                     rows_per_example=S, rows=dx_rows)
    dw = backward.backward_dw if scale == oq.PER_TENSOR else backward.backward_dw_per_token
    out["dW"] = dw(q["Q"], q["delta"], fx["Q"], fw["scale"], ec=ec, xs=fx["code_colsum"], eps=q["eps"],
                   ebar=q["ebar"], mu=q["mu"], rows_per_example=S, rows=dw_rows)
    return out


def linear_backward_twice(inp: dict, *, mode_dx: int, mode_dw: int, seed: int = 0, layer_id: int = 0,
                          rows_per_example: int, fx=None, fw=None) -> dict:
    """The conventional configuration: G quantized separately for the two products.

    S3R page, "Quantized Backpropagation with Stochastic Rounding": conventional
    quantized training draws independent thresholds R^LHS and R^RHS for the
    activation-gradient and the weight-gradient products (independent SR as in
    AQT); Table II's causal ablation also mixes Phi_2D and Phi_bcast between the
    two.  Here the dX operand uses threshold stream 0 and the dW operand stream 1;
    there is no correction.
    """
    dtype = inp["dtype"]
    S = rows_per_example
    if fx is None or fw is None:
        fx, fw = forward_operands(inp["X"], inp["W"], dtype, S)
    qx = quantize_gradient(inp["G"], dtype, fx, fw, mode=mode_dx, scale=oq.PER_TENSOR, seed=seed,
                           layer_id=layer_id, rows_per_example=S, stream=0)
    qw = quantize_gradient(inp["G"], dtype, fx, fw, mode=mode_dw, scale=oq.PER_TENSOR, seed=seed,
                           layer_id=layer_id, rows_per_example=S, stream=1)
    dX = backward.backward_dx(qx["Q"], qx["delta"], fw["Q"], fx["scale"])
    dW = backward.backward_dw(qw["Q"], qw["delta"], fx["Q"], fw["scale"])
    return {"fx": fx, "fw": fw, "q_dx": qx, "q_dw": qw, "dX": dX, "dW": dW}


def raw_accumulators(Q, Wq, Xq, dx_rows=None, dw_rows=None):
    """Exact int32 accumulators of both GEMMs (optionally for a row sample)."""
    T, D = Q.shape
    dx_rows = np.arange(T) if dx_rows is None else np.asarray(dx_rows)
    dw_rows = np.arange(D) if dw_rows is None else np.asarray(dw_rows)
    acc_dx = backward.int_matmul(Q[dx_rows], Wq)
    acc_dw = backward.int_matmul(np.ascontiguousarray(Q[:, dw_rows].T), Xq)
    return acc_dx, acc_dw


def ffn_block_backward(inp: dict, *, mode: int, ec: int, seed: int = 0, rows_per_example: int) -> dict:
    """Backward of one SwiGLU FFN block (the S3R page's single-block benchmark, "Setup"; Table III).

    ``inp`` holds the bf16 bit patterns of make_ffn_block_inputs: G (the block's output gradient),
    X, H, A_gate, A_up, W_down, W_gate, W_up.  Each of the three projections runs the quantized
    linear backward above (layer ids: down 0, gate 1, up 2).  The down projection's dX, dH, enters
    the glue in fp32 (the dtype the backward hands over), and the glue's bf16 results are the gate
    and up projections' upstream gradients; the block's dX is the sum of theirs.
    """
    from . import swiglu
    S = rows_per_example
    down = linear_backward({"G": inp["G"], "X": inp["H"], "W": inp["W_down"], "dtype": "bf16"}, mode=mode, ec=ec,
                           seed=seed, layer_id=0, rows_per_example=S)
    dH = down["dX"].astype(np.float32)
    g_gate, g_up = swiglu.glue(dH, inp["A_gate"], inp["A_up"])
    fx = oq.forward_operand(inp["X"], "bf16", rows_per_example=S)
    out = {"down": down, "G_gate": g_gate, "G_up": g_up}
    for name, g, w, layer in (("gate", g_gate, inp["W_gate"], 1), ("up", g_up, inp["W_up"], 2)):
        fw = oq.forward_operand(w, "bf16", rows_per_example=w.shape[0])
        out[name] = linear_backward({"G": g, "X": inp["X"], "W": w, "dtype": "bf16"}, mode=mode, ec=ec, seed=seed,
                                    layer_id=layer, rows_per_example=S, fx=fx, fw=fw)
    out["dX"] = out["gate"]["dX"] + out["up"]["dX"]
    return out
