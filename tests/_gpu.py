"""Helpers for the GPU parity tests: host <-> device conversion and the GPU pipeline.

The GPU side goes only through the C ABI (via the thin binding); expected values
come only from oracle/.
"""
import json
import os

import numpy as np
import torch

from stochastic_rounding_quantization_amd import s3r

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array (float32 or uint16 bf16 bits) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_err(got, exp) -> float:
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    scale = np.abs(exp).max() if exp.size else 0.0
    return float(np.abs(got - exp).max() / scale) if scale > 0 else float(np.abs(got - exp).max() if got.size else 0)


def row_rel_err(got, exp) -> float:
    """Max over rows of max|got - exp| / max|exp| within the row.

    A row is a token of dX and a channel of dW: each is held to the tolerance on its own
    magnitude, so a small row beside outlier rows is not judged on the outliers' scale.  A row
    whose reference is exactly zero is held to the absolute difference.
    """
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    if got.size == 0:
        return 0.0
    g = got.reshape(got.shape[0], -1)
    e = exp.reshape(exp.shape[0], -1)
    diff = np.abs(g - e).max(axis=1)
    scale = np.abs(e).max(axis=1)
    return float(np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff).max())


def elementwise_fail_frac(got, exp, tol) -> float:
    """Fraction of elements with |got - exp| > tol * |exp| (each element on its own magnitude)."""
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    if got.size == 0:
        return 0.0
    return float((np.abs(got - exp) > tol * np.abs(exp)).mean())


def assert_rows_close(got, exp, tol, what=""):
    """Per-row relative bar (see row_rel_err); prints the elementwise failure fraction beside it.

    With S3R_PARITY_LOG set, each comparison is also appended to that file as one JSON line.
    """
    err = row_rel_err(got, exp)
    frac = elementwise_fail_frac(got, exp, tol)
    print(f"[parity] {what}: max per-row rel err {err:.3g}; elements beyond {tol:g} relative: {frac:.3g}",
          flush=True)
    log = os.environ.get("S3R_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"what": what, "shape": list(np.shape(got)), "row_rel_err": err,
                                "elementwise_fail_frac": frac, "tol": tol}) + "\n")
    assert err <= tol, f"{what}: per-row relative error {err:.3g} > {tol:g} (elementwise fraction {frac:.3g})"


def gpu_linear(inp: dict, *, mode, ec, scale=s3r.PER_TENSOR, seed=0, layer_id=0, rows_per_example, dw=True):
    """Forward-operand prep + quantize + dX (+ dW) on the GPU through the C ABI."""
    dt = inp["dtype"]
    G, X, W = to_dev(inp["G"], dt), to_dev(inp["X"], dt), to_dev(inp["W"], dt)
    S = rows_per_example
    fx = s3r.forward_operand(X, rows_per_example=S)
    fw = s3r.forward_operand(W, rows_per_example=W.shape[0])
    q = s3r.quantize(G, mode=mode, ec=ec, scale=scale, row_scale=fx.delta, col_scale=fw.delta, seed=seed,
                     layer_id=layer_id, rows_per_example=S)
    dX = s3r.backward_dx(q, fw.Q, s_x=fx.delta, r_W=fw.code_colsum[0])
    dW = s3r.backward_dw(q, fx.Q, s_w=fw.delta, xs_b=fx.code_colsum) if dw else None  # any step granularity
    torch.cuda.synchronize()
    return {"fx": fx, "fw": fw, "q": q, "dX": dX, "dW": dW}


def mx_rows(codes, rows: int, K: int) -> np.ndarray:
    """MXFP4 codes in the library's block layout (256-row x 128-element blocks of 16 KiB, one
    256-row block per tensor row) as plain row-major bytes [rows x K/2], on the host."""
    a = host(codes).reshape(-1, K // 128, 256, 64)
    return a.transpose(0, 2, 1, 3).reshape(-1, K // 2)[:rows]


def assert_nan_equal(got, exp, what=""):
    got = np.asarray(got)
    exp = np.asarray(exp)
    both_nan = np.isnan(got) & np.isnan(exp)
    ok = (got == exp) | both_nan
    assert ok.all(), f"{what}: {int((~ok).sum())} mismatches, first at {np.argwhere(~ok)[:3].tolist()}"
