"""Thin Python binding of libs3r.so (include/s3r.h).

The functions named ``s3r_*`` mirror the C entry points one to one: they only
marshal torch tensors (device memory) and the current HIP stream into the C
call.  Every step of the computation runs in the library's HIP kernels; if the
library is missing, loading it raises (there is no fallback).

The helpers without the prefix (``quantize``, ``backward_dx``, ``backward_dw``,
``forward_operand``) allocate outputs and workspaces with torch and then call
the entry points.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libs3r.so")

S3R_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported combination", -3: "workspace too small",
          -4: "device is not gfx950", -5: "HIP error"}
S3R_F32, S3R_BF16, S3R_I32_RAW, S3R_F32_ACC = 0, 1, 2, 3
RTNE, SR, S3R, S3R_BCAST = 0, 1, 2, 3
EC_NONE, EC_DX_ONLY, EC_TWO_WAY, EC_DW_ONLY = 0, 1, 2, 3
PER_TENSOR, PER_TOKEN = 0, 1
FLAG_NONFINITE, FLAG_TINY_STEP, FLAG_BAD_GROUPS = 1, 2, 8
S3R_NOALLOC_SCRATCH_BYTES = 32 << 20    # include/s3r.h: the no-alloc quantizer's device array

EXPORTED = ["s3r_quantize_workspace", "s3r_quantize", "s3r_quantize_with_amax", "s3r_quantize_noalloc", "s3r_backward_dx",
            "s3r_backward_dw", "s3r_backward_dw_pair", "s3r_backward_dw_pair_workspace", "s3r_backward_workspace", "s3r_swiglu_backward", "s3r_swiglu_amax_workspace",
            "s3r_swiglu_backward_amax", "s3r_swiglu_quantize_workspace", "s3r_swiglu_quantize", "s3r_grouped_workspace", "s3r_grouped_quantize",
            "s3r_grouped_backward_dx", "s3r_grouped_backward_dw", "s3r_mx_workspace", "s3r_mx_operand_workspace",
            "s3r_mx_operand", "s3r_mx_quantize", "s3r_mx_backward_dx", "s3r_mx_backward_dw", "s3r_time_next_gemm",
            "s3r_status_string", "s3r_version"]


class S3RError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({code})")
        self.code = code


class QDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("rows_per_example", ctypes.c_int64),
                ("mode", ctypes.c_int32), ("ec", ctypes.c_int32), ("scale", ctypes.c_int32),
                ("layer_id", ctypes.c_uint32), ("seed", ctypes.c_uint64), ("stream", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


def qdesc(rows, cols, rows_per_example=None, mode=S3R, ec=EC_NONE, scale=PER_TENSOR, layer_id=0, seed=0,
          stream=0) -> QDesc:
    S = rows_per_example if rows_per_example is not None else max(rows, 1)
    return QDesc(rows, cols, S, mode, ec, scale, layer_id, seed, stream, 0)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libs3r.so (built in-tree by ``python -m stochastic_rounding_quantization_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m stochastic_rounding_quantization_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(QDesc)
    L.s3r_quantize_workspace.argtypes = [DP]
    L.s3r_quantize_workspace.restype = SZ
    L.s3r_quantize.argtypes = [DP, P, I32, I64, P, P, P, I64, P, P, P, P, P, P, P, SZ, P]
    L.s3r_quantize.restype = ctypes.c_int
    L.s3r_quantize_with_amax.argtypes = [DP, P, I32, I64, P, P, P, P, I64, P, P, P, P, P, P, SZ, P]
    L.s3r_quantize_with_amax.restype = ctypes.c_int
    L.s3r_quantize_noalloc.argtypes = [DP, P, I32, I64, P, P, P, I64, P, P, P, P, P, P, P]
    L.s3r_quantize_noalloc.restype = ctypes.c_int
    L.s3r_backward_dx.argtypes = [DP, P, I64, P, P, I64, I64, P, P, P, P, P, P, I32, I64, P, SZ, P]
    L.s3r_backward_dx.restype = ctypes.c_int
    L.s3r_backward_dw.argtypes = [DP, P, I64, P, P, I64, I64, P, P, P, P, P, P, I32, I64, P, SZ, P]
    L.s3r_backward_dw.restype = ctypes.c_int
    L.s3r_backward_dw_pair.argtypes = [DP, P, P, I64, P, P, P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, I32, I64,
                                       P, SZ, P]
    L.s3r_backward_dw_pair.restype = ctypes.c_int
    L.s3r_backward_dw_pair_workspace.argtypes = [DP, I64]
    L.s3r_backward_dw_pair_workspace.restype = SZ
    L.s3r_backward_workspace.argtypes = [DP, I64]
    L.s3r_backward_workspace.restype = SZ
    L.s3r_swiglu_backward.argtypes = [I64, I64, P, I64, P, P, I64, P, P, I64, P]
    L.s3r_swiglu_backward.restype = ctypes.c_int
    L.s3r_swiglu_amax_workspace.argtypes = [I64, I64]
    L.s3r_swiglu_amax_workspace.restype = SZ
    L.s3r_swiglu_backward_amax.argtypes = [I64, I64, P, I64, P, P, I64, P, P, I64, P, P, P, P, P, SZ, P]
    L.s3r_swiglu_backward_amax.restype = ctypes.c_int
    L.s3r_swiglu_quantize_workspace.argtypes = [DP]
    L.s3r_swiglu_quantize_workspace.restype = SZ
    L.s3r_swiglu_quantize.argtypes = [DP, DP, P, I64, P, P, I64, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, SZ,
                                      P]
    L.s3r_swiglu_quantize.restype = ctypes.c_int
    L.s3r_grouped_workspace.argtypes = [DP, I64, I64]
    L.s3r_grouped_workspace.restype = SZ
    L.s3r_grouped_quantize.argtypes = [DP, I64, P, P, I32, I64, P, P, P, I64, P, P, P, P, P, P, P, SZ, P]
    L.s3r_grouped_quantize.restype = ctypes.c_int
    L.s3r_grouped_backward_dx.argtypes = [DP, I64, P, P, I64, P, P, I64, I64, I64, P, P, P, P, P, P, I32, I64, P, P,
                                          SZ, P]
    L.s3r_grouped_backward_dx.restype = ctypes.c_int
    L.s3r_grouped_backward_dw.argtypes = [DP, I64, P, P, I64, P, P, I64, I64, P, P, P, P, P, P, I32, I64, I64, P, P,
                                          SZ, P]
    L.s3r_grouped_backward_dw.restype = ctypes.c_int
    L.s3r_mx_workspace.argtypes = [DP, I64]
    L.s3r_mx_workspace.restype = SZ
    L.s3r_mx_operand_workspace.argtypes = [I64, I64]
    L.s3r_mx_operand_workspace.restype = SZ
    L.s3r_mx_operand.argtypes = [I64, I64, I64, P, I32, I64, P, I64, P, I64, P, P, P, SZ, P]
    L.s3r_mx_quantize.argtypes = [DP, P, I32, I64, P, I64, P, I64, P, I64, P, I64, P, P, P, P, P, P, P, P, SZ, P]
    L.s3r_mx_backward_dx.argtypes = [DP, P, I64, P, I64, P, I64, P, I64, I64, P, P, P, P, P, I64, P, SZ, P]
    L.s3r_mx_backward_dw.argtypes = [DP, P, I64, P, I64, P, I64, P, I64, I64, P, P, P, P, P, I64, P, SZ, P]
    L.s3r_time_next_gemm.argtypes = [P, P]
    L.s3r_time_next_gemm.restype = ctypes.c_int
    L.s3r_status_string.argtypes = [ctypes.c_int]
    L.s3r_status_string.restype = ctypes.c_char_p
    L.s3r_version.argtypes = []
    L.s3r_version.restype = ctypes.c_int
    _lib = L
    return L


# ------------------------------------------------------------ marshalling ----

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t, default=0):
    if t is None:
        return default
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor (unit column stride)")
    return t.stride(0)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != S3R_OK:
        raise S3RError(fn, rc)


def _gdtype(t):
    import torch
    if t.dtype == torch.float32:
        return S3R_F32
    if t.dtype == torch.bfloat16:
        return S3R_BF16
    raise ValueError(f"unsupported gradient dtype {t.dtype}")


def _odtype(t, accumulate=False):
    import torch
    if t.dtype == torch.float32:
        return S3R_F32_ACC if accumulate else S3R_F32
    if t.dtype == torch.int32:
        return S3R_I32_RAW
    raise ValueError(f"unsupported output dtype {t.dtype}")


def s3r_quantize_workspace(desc: QDesc) -> int:
    return lib().s3r_quantize_workspace(ctypes.byref(desc))


def s3r_quantize(desc: QDesc, G, row_scale, col_scale, Q, delta, code_colsum=None, ec_row=None, ec_col=None,
                 ec_mean=None, flags=None, ws=None, stream=None, *, rc_only=False):
    rc = lib().s3r_quantize(ctypes.byref(desc), _ptr(G), _gdtype(G) if G is not None else S3R_F32,
                            _ld(G, desc.cols), _ptr(row_scale), _ptr(col_scale), _ptr(Q), _ld(Q, desc.cols),
                            _ptr(delta), _ptr(code_colsum), _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean),
                            _ptr(flags), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                            _stream(stream))
    if rc_only:
        return rc
    _check("s3r_quantize", rc)


def s3r_quantize_noalloc(desc: QDesc, G, row_scale, col_scale, Q, delta, code_colsum=None, ec_row=None, ec_col=None,
                         ec_mean=None, flags=None, stream=None, *, rc_only=False):
    rc = lib().s3r_quantize_noalloc(ctypes.byref(desc), _ptr(G), _gdtype(G) if G is not None else S3R_F32,
                                    _ld(G, desc.cols), _ptr(row_scale), _ptr(col_scale), _ptr(Q), _ld(Q, desc.cols),
                                    _ptr(delta), _ptr(code_colsum), _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean),
                                    _ptr(flags), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_quantize_noalloc", rc)


def s3r_quantize_with_amax(desc: QDesc, G, row_scale, col_scale, amax_bits, Q, delta, ec_row=None, ec_col=None,
                           ec_mean=None, flags=None, ws=None, stream=None, *, rc_only=False):
    rc = lib().s3r_quantize_with_amax(ctypes.byref(desc), _ptr(G), _gdtype(G) if G is not None else S3R_F32,
                                      _ld(G, desc.cols), _ptr(row_scale), _ptr(col_scale), _ptr(amax_bits), _ptr(Q),
                                      _ld(Q, desc.cols), _ptr(delta), _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean),
                                      _ptr(flags), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                      _stream(stream))
    if rc_only:
        return rc
    _check("s3r_quantize_with_amax", rc)


def s3r_backward_workspace(desc: QDesc, d_in: int) -> int:
    return lib().s3r_backward_workspace(ctypes.byref(desc), d_in)


def s3r_backward_dx(desc: QDesc, Q, delta, Wq, s_x, r_W, ec_row, ec_col, ec_mean, dX, ws=None, stream=None,
                    *, accumulate=False, rc_only=False):
    d_in = dX.shape[1]
    rc = lib().s3r_backward_dx(ctypes.byref(desc), _ptr(Q), _ld(Q, desc.cols), _ptr(delta), _ptr(Wq),
                               _ld(Wq, d_in), d_in, _ptr(s_x), _ptr(r_W), _ptr(ec_row), _ptr(ec_col),
                               _ptr(ec_mean), _ptr(dX), _odtype(dX, accumulate), _ld(dX, d_in), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_backward_dx", rc)


def s3r_backward_dw(desc: QDesc, Q, delta, Xq, s_w, xs_b, ec_row, ec_col, ec_mean, dW, ws=None, stream=None,
                    *, rc_only=False):
    d_in = dW.shape[1]
    rc = lib().s3r_backward_dw(ctypes.byref(desc), _ptr(Q), _ld(Q, desc.cols), _ptr(delta), _ptr(Xq),
                               _ld(Xq, d_in), d_in, _ptr(s_w), _ptr(xs_b), _ptr(ec_row), _ptr(ec_col),
                               _ptr(ec_mean), _ptr(dW), _odtype(dW), _ld(dW, d_in), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_backward_dw", rc)


def s3r_backward_dw_pair_workspace(desc: QDesc, d_in: int) -> int:
    return lib().s3r_backward_dw_pair_workspace(ctypes.byref(desc), d_in)


def s3r_backward_dw_pair(desc: QDesc, Q0, Q1, delta0, delta1, Xq, s_w0, s_w1, xs_b, ec0, ec1, dW0, dW1, ws=None,
                         stream=None, *, rc_only=False):
    """Both dW products of two projections of one input in one launch; ec0 / ec1 are the
    (ec_row, ec_col, ec_mean) triples of the two quantize calls."""
    d_in = dW0.shape[1]
    if _ld(Q1, desc.cols) != _ld(Q0, desc.cols) or _ld(dW1, d_in) != _ld(dW0, d_in) or dW1.dtype != dW0.dtype:
        raise ValueError("the two products need codes and outputs of one layout")
    rc = lib().s3r_backward_dw_pair(
        ctypes.byref(desc), _ptr(Q0), _ptr(Q1), _ld(Q0, desc.cols), _ptr(delta0), _ptr(delta1), _ptr(Xq),
        _ld(Xq, d_in), d_in, _ptr(s_w0), _ptr(s_w1), _ptr(xs_b), _ptr(ec0[0]), _ptr(ec0[1]), _ptr(ec0[2]),
        _ptr(ec1[0]), _ptr(ec1[1]), _ptr(ec1[2]), _ptr(dW0), _ptr(dW1), _odtype(dW0), _ld(dW0, d_in), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_backward_dw_pair", rc)


def s3r_swiglu_backward(dH, A_gate, A_up, G_gate, G_up, stream=None, *, rc_only=False):
    """bf16 tensors are passed as torch.bfloat16 (their bit patterns are the C ABI's uint16)."""
    T, F = dH.shape
    if A_up.stride() != A_gate.stride() or G_up.stride() != G_gate.stride():
        raise ValueError("A_gate / A_up and G_gate / G_up must share their layouts")
    rc = lib().s3r_swiglu_backward(T, F, _ptr(dH), _ld(dH, F), _ptr(A_gate), _ptr(A_up), _ld(A_gate, F),
                                   _ptr(G_gate), _ptr(G_up), _ld(G_gate, F), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_swiglu_backward", rc)


def s3r_swiglu_amax_workspace(T: int, F: int) -> int:
    return lib().s3r_swiglu_amax_workspace(T, F)


def s3r_swiglu_backward_amax(dH, A_gate, A_up, G_gate, G_up, row_scale, col_scale_gate, col_scale_up, amax_bits,
                             ws, stream=None, *, rc_only=False):
    """Glue and the gate / up amax (uint32 [2] device tensor amax_bits) in one pass."""
    T, F = dH.shape
    if A_up.stride() != A_gate.stride() or G_up.stride() != G_gate.stride():
        raise ValueError("A_gate / A_up and G_gate / G_up must share their layouts")
    rc = lib().s3r_swiglu_backward_amax(T, F, _ptr(dH), _ld(dH, F), _ptr(A_gate), _ptr(A_up), _ld(A_gate, F),
                                        _ptr(G_gate), _ptr(G_up), _ld(G_gate, F), _ptr(row_scale),
                                        _ptr(col_scale_gate), _ptr(col_scale_up), _ptr(amax_bits), _ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_swiglu_backward_amax", rc)


def s3r_swiglu_quantize_workspace(desc: QDesc) -> int:
    return lib().s3r_swiglu_quantize_workspace(ctypes.byref(desc))


def s3r_swiglu_quantize(desc_gate: QDesc, desc_up: QDesc, dH, A_gate, A_up, row_scale, col_scale_gate, col_scale_up,
                        Q_gate, Q_up, delta_gate, delta_up, ec_gate=(None, None, None), ec_up=(None, None, None),
                        flags=None, ws=None, stream=None, *, rc_only=False):
    """The gate and up quantizers with the glue inside (G_gate, G_up never written); ec_gate / ec_up are
    (ec_row, ec_col, ec_mean) triples."""
    F = desc_gate.cols
    if A_up.stride() != A_gate.stride() or _ld(Q_up, F) != _ld(Q_gate, F):
        raise ValueError("A_gate / A_up and Q_gate / Q_up must share their layouts")
    rc = lib().s3r_swiglu_quantize(
        ctypes.byref(desc_gate), ctypes.byref(desc_up), _ptr(dH), _ld(dH, F), _ptr(A_gate), _ptr(A_up),
        _ld(A_gate, F), _ptr(row_scale), _ptr(col_scale_gate), _ptr(col_scale_up), _ptr(Q_gate), _ptr(Q_up),
        _ld(Q_gate, F), _ptr(delta_gate), _ptr(delta_up), _ptr(ec_gate[0]), _ptr(ec_gate[1]), _ptr(ec_gate[2]),
        _ptr(ec_up[0]), _ptr(ec_up[1]), _ptr(ec_up[2]), _ptr(flags), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_swiglu_quantize", rc)


def s3r_grouped_workspace(desc: QDesc, groups: int, d_in: int) -> int:
    return lib().s3r_grouped_workspace(ctypes.byref(desc), groups, d_in)


def _nbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def s3r_grouped_quantize(desc: QDesc, offsets, G, row_scale, col_scale, Q, delta, code_colsum=None, ec_row=None,
                         ec_col=None, ec_mean=None, flags=None, ws=None, stream=None, *, rc_only=False):
    """offsets: int64 device tensor [groups + 1]; col_scale [groups x D] (or None)."""
    rc = lib().s3r_grouped_quantize(ctypes.byref(desc), offsets.numel() - 1, _ptr(offsets), _ptr(G),
                                    _gdtype(G) if G is not None else S3R_F32, _ld(G, desc.cols), _ptr(row_scale),
                                    _ptr(col_scale), _ptr(Q), _ld(Q, desc.cols), _ptr(delta), _ptr(code_colsum),
                                    _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean), _ptr(flags), _ptr(ws), _nbytes(ws),
                                    _stream(stream))
    if rc_only:
        return rc
    _check("s3r_grouped_quantize", rc)


def s3r_grouped_backward_dx(desc: QDesc, offsets, Q, delta, Wq, s_x, r_W, ec_row, ec_col, ec_mean, dX, flags=None,
                            ws=None, stream=None, *, accumulate=False, rc_only=False):
    """Wq: int8 [groups x D x d_in] (3-D, rows with unit stride)."""
    d_in = dX.shape[1]
    if Wq.dim() != 3 or Wq.stride(2) != 1:
        raise ValueError("expected Wq as [groups x D x d_in] with unit column stride")
    rc = lib().s3r_grouped_backward_dx(ctypes.byref(desc), offsets.numel() - 1, _ptr(offsets), _ptr(Q),
                                       _ld(Q, desc.cols), _ptr(delta), _ptr(Wq), Wq.stride(1), Wq.stride(0), d_in,
                                       _ptr(s_x), _ptr(r_W), _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean), _ptr(dX),
                                       _odtype(dX, accumulate), _ld(dX, d_in), _ptr(flags), _ptr(ws), _nbytes(ws),
                                       _stream(stream))
    if rc_only:
        return rc
    _check("s3r_grouped_backward_dx", rc)


def s3r_grouped_backward_dw(desc: QDesc, offsets, Q, delta, Xq, s_w, xs, ec_row, ec_col, ec_mean, dW, flags=None,
                            ws=None, stream=None, *, rc_only=False):
    """dW: float32 / int32 [groups x D x d_in] (3-D, unit column stride)."""
    d_in = Xq.shape[1]
    if dW.dim() != 3 or dW.stride(2) != 1:
        raise ValueError("expected dW as [groups x D x d_in] with unit column stride")
    rc = lib().s3r_grouped_backward_dw(ctypes.byref(desc), offsets.numel() - 1, _ptr(offsets), _ptr(Q),
                                       _ld(Q, desc.cols), _ptr(delta), _ptr(Xq), _ld(Xq, d_in), d_in, _ptr(s_w),
                                       _ptr(xs), _ptr(ec_row), _ptr(ec_col), _ptr(ec_mean), _ptr(dW), _odtype(dW),
                                       dW.stride(1), dW.stride(0), _ptr(flags), _ptr(ws), _nbytes(ws),
                                       _stream(stream))
    if rc_only:
        return rc
    _check("s3r_grouped_backward_dw", rc)


def s3r_mx_workspace(desc: QDesc, d_in: int) -> int:
    return lib().s3r_mx_workspace(ctypes.byref(desc), d_in)


def s3r_mx_operand_workspace(rows: int, cols: int) -> int:
    return lib().s3r_mx_operand_workspace(rows, cols)


def s3r_mx_operand(M, Mt, Mt_scales, colsum=None, rows_per_example=None, flags=None, ws=None, stream=None, *,
                   rc_only=False):
    """M [rows x cols] f32/bf16 -> Mt (mx_codes(cols, rows)), Mt_scales uint8 [rows/128 x 4*cols] (step-grouped)."""
    rows, cols = M.shape
    S = rows if rows_per_example is None else rows_per_example
    rc = lib().s3r_mx_operand(rows, cols, S, _ptr(M), _gdtype(M), _ld(M, cols), _ptr(Mt), _ld(Mt),
                              _ptr(Mt_scales), _ld(Mt_scales, 4 * cols), _ptr(colsum), _ptr(flags), _ptr(ws),
                              _nbytes(ws), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_mx_operand", rc)


def s3r_mx_quantize(desc: QDesc, G, Qh, Qh_scales, Qt, Qt_scales, ec_row_h=None, ec_col_h=None, ec_mean_h=None,
                    ec_row_t=None, ec_col_t=None, ec_mean_t=None, flags=None, ws=None, stream=None, *,
                    rc_only=False):
    T, D = desc.rows, desc.cols
    rc = lib().s3r_mx_quantize(ctypes.byref(desc), _ptr(G), _gdtype(G) if G is not None else S3R_F32, _ld(G, D),
                               _ptr(Qh), _ld(Qh), _ptr(Qh_scales), _ld(Qh_scales, 4 * T), _ptr(Qt),
                               _ld(Qt), _ptr(Qt_scales), _ld(Qt_scales, 4 * D), _ptr(ec_row_h),
                               _ptr(ec_col_h), _ptr(ec_mean_h), _ptr(ec_row_t), _ptr(ec_col_t), _ptr(ec_mean_t),
                               _ptr(flags), _ptr(ws), _nbytes(ws), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_mx_quantize", rc)


def s3r_mx_backward_dx(desc: QDesc, Qh, Qh_scales, Wt, Wt_scales, r_W, ec_row_h, ec_col_h, ec_mean_h, dX, ws=None,
                       stream=None, *, rc_only=False):
    """Wt: mx_codes(d_in, D), Wt_scales [D/128 x 4*d_in]; dX f32 [T x d_in]."""
    d_in = dX.shape[1]
    rc = lib().s3r_mx_backward_dx(ctypes.byref(desc), _ptr(Qh), _ld(Qh), _ptr(Qh_scales),
                                  _ld(Qh_scales, 4 * desc.rows), _ptr(Wt), _ld(Wt), _ptr(Wt_scales),
                                  _ld(Wt_scales, 4 * d_in), d_in, _ptr(r_W), _ptr(ec_row_h), _ptr(ec_col_h),
                                  _ptr(ec_mean_h), _ptr(dX), _ld(dX, d_in), _ptr(ws), _nbytes(ws), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_mx_backward_dx", rc)


def s3r_mx_backward_dw(desc: QDesc, Qt, Qt_scales, Xt, Xt_scales, xs, ec_row_t, ec_col_t, ec_mean_t, dW, ws=None,
                       stream=None, *, rc_only=False):
    """Xt: mx_codes(d_in, T), Xt_scales [T/128 x 4*d_in]; dW f32 [D x d_in]."""
    d_in = dW.shape[1]
    rc = lib().s3r_mx_backward_dw(ctypes.byref(desc), _ptr(Qt), _ld(Qt), _ptr(Qt_scales),
                                  _ld(Qt_scales, 4 * desc.cols), _ptr(Xt), _ld(Xt), _ptr(Xt_scales),
                                  _ld(Xt_scales, 4 * d_in), d_in, _ptr(xs), _ptr(ec_row_t), _ptr(ec_col_t),
                                  _ptr(ec_mean_t), _ptr(dW), _ld(dW, d_in), _ptr(ws), _nbytes(ws), _stream(stream))
    if rc_only:
        return rc
    _check("s3r_mx_backward_dw", rc)


def swiglu_backward(dH, A_gate, A_up, stream=None):
    """Allocate G_gate, G_up (bf16, like A_gate) and run s3r_swiglu_backward."""
    import torch
    G_gate = torch.empty(A_gate.shape, dtype=torch.bfloat16, device=A_gate.device)
    G_up = torch.empty_like(G_gate)
    s3r_swiglu_backward(dH, A_gate, A_up, G_gate, G_up, stream)
    return G_gate, G_up


def swiglu_quantize(dH, A_gate, A_up, *, mode=S3R, ec=EC_NONE, row_scale=None, col_scale_gate=None,
                    col_scale_up=None, seed=0, layer_gate=0, layer_up=0, rows_per_example=None, stream=None,
                    threshold_stream=0):
    """Allocate the outputs and run s3r_swiglu_quantize: (Quantized gate, Quantized up)."""
    import torch
    T, F = dH.shape
    dev = dH.device
    dg = qdesc(T, F, rows_per_example, mode, ec, PER_TENSOR, layer_gate, seed, threshold_stream)
    du = qdesc(T, F, rows_per_example, mode, ec, PER_TENSOR, layer_up, seed, threshold_stream)
    B = T // dg.rows_per_example
    out = []
    for d in (dg, du):
        e = (None, None, None)
        if ec != EC_NONE:
            e = (torch.empty(T, dtype=torch.float32, device=dev), torch.empty(B, F, dtype=torch.float32, device=dev),
                 torch.empty(B, dtype=torch.float32, device=dev))
        out.append((q_buffer(T, F, dev), torch.empty(1, dtype=torch.float32, device=dev), e))
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(s3r_swiglu_quantize_workspace(dg), dev)
    s3r_swiglu_quantize(dg, du, dH, A_gate, A_up, row_scale, col_scale_gate, col_scale_up, out[0][0], out[1][0],
                        out[0][1], out[1][1], out[0][2], out[1][2], flags, ws, stream)
    return (Quantized(out[0][0], out[0][1], dg, None, *out[0][2], flags),
            Quantized(out[1][0], out[1][1], du, None, *out[1][2], flags))


def s3r_time_next_gemm(start_event, stop_event) -> None:
    """Record two torch.cuda.Event objects around the next GEMM kernel launched from this thread."""
    _check("s3r_time_next_gemm", lib().s3r_time_next_gemm(
        ctypes.c_void_p(start_event.cuda_event) if start_event is not None else None,
        ctypes.c_void_p(stop_event.cuda_event) if stop_event is not None else None))


def s3r_version() -> int:
    return lib().s3r_version()


def s3r_status_string(code: int) -> str:
    return lib().s3r_status_string(code).decode()


# ------------------------------------------------------ allocating helpers ----

def _pad16(n: int) -> int:
    return (n + 15) // 16 * 16


def _workspace(nbytes: int, device):
    import torch
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes else None


def q_buffer(rows: int, cols: int, device):
    """int8 [rows x cols] view with a leading dimension padded to 16 (what the GEMMs need)."""
    import torch
    return torch.empty(rows, _pad16(cols), dtype=torch.int8, device=device)[:, :cols]


@dataclass
class Quantized:
    Q: object            # int8 [T x D] (leading dim padded to 16)
    delta: object        # f32 [1] or [T]
    desc: QDesc
    code_colsum: object = None
    ec_row: object = None
    ec_col: object = None
    ec_mean: object = None
    flags: object = None


def quantize(G, *, mode=S3R, ec=EC_NONE, scale=PER_TENSOR, row_scale=None, col_scale=None, seed=0, layer_id=0,
             rows_per_example=None, colsum=False, stream=None, threshold_stream=0) -> Quantized:
    import torch
    T, D = G.shape
    desc = qdesc(T, D, rows_per_example, mode, ec, scale, layer_id, seed, threshold_stream)
    dev = G.device
    S = desc.rows_per_example
    B = T // S
    Q = q_buffer(T, D, dev)
    delta = torch.empty(T if scale == PER_TOKEN else 1, dtype=torch.float32, device=dev)
    cs = torch.empty(B, D, dtype=torch.int32, device=dev) if colsum else None
    e_r = e_c = e_m = None
    if ec != EC_NONE:
        e_r = torch.empty(T, dtype=torch.float32, device=dev)
        e_c = torch.empty(B, D, dtype=torch.float32, device=dev)
        e_m = torch.empty(B, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(s3r_quantize_workspace(desc), dev)
    s3r_quantize(desc, G, row_scale, col_scale, Q, delta, cs, e_r, e_c, e_m, flags, ws, stream)
    return Quantized(Q, delta, desc, cs, e_r, e_c, e_m, flags)


def forward_operand(X, rows_per_example=None, stream=None) -> Quantized:
    """Per-row absmax RTNE of a forward operand (X per token, W per output channel) with code column sums."""
    return quantize(X, mode=RTNE, ec=EC_NONE, scale=PER_TOKEN, rows_per_example=rows_per_example, colsum=True,
                    stream=stream)


def backward_dx(q: Quantized, Wq, s_x=None, r_W=None, out_dtype=None, stream=None, out=None):
    """dX of one projection; with ``out`` (f32) the result is added into it."""
    import torch
    d_in = Wq.shape[1]
    T = q.desc.rows
    dX = out if out is not None else torch.empty(T, d_in, dtype=out_dtype or torch.float32, device=Wq.device)
    ws = _workspace(s3r_backward_workspace(q.desc, d_in), Wq.device)
    s3r_backward_dx(q.desc, q.Q, q.delta, Wq, s_x, r_W, q.ec_row, q.ec_col, q.ec_mean, dX, ws, stream,
                    accumulate=out is not None)
    return dX


def backward_dw(q: Quantized, Xq, s_w=None, xs_b=None, out_dtype=None, stream=None):
    import torch
    d_in = Xq.shape[1]
    D = q.desc.cols
    dW = torch.empty(D, d_in, dtype=out_dtype or torch.float32, device=Xq.device)
    ws = _workspace(s3r_backward_workspace(q.desc, d_in), Xq.device)
    s3r_backward_dw(q.desc, q.Q, q.delta, Xq, s_w, xs_b, q.ec_row, q.ec_col, q.ec_mean, dW, ws, stream)
    return dW


def backward_dw_pair(qa: Quantized, qb: Quantized, Xq, s_w_a=None, s_w_b=None, xs_b=None, out_dtype=None,
                     stream=None):
    """dW of two projections of the input Xq (one GEMM launch); qa and qb share shape and layout."""
    import torch
    d_in = Xq.shape[1]
    D = qa.desc.cols
    dWa = torch.empty(D, d_in, dtype=out_dtype or torch.float32, device=Xq.device)
    dWb = torch.empty_like(dWa)
    ws = _workspace(s3r_backward_dw_pair_workspace(qa.desc, d_in), Xq.device)
    s3r_backward_dw_pair(qa.desc, qa.Q, qb.Q, qa.delta, qb.delta, Xq, s_w_a, s_w_b, xs_b,
                         (qa.ec_row, qa.ec_col, qa.ec_mean), (qb.ec_row, qb.ec_col, qb.ec_mean), dWa, dWb, ws, stream)
    return dWa, dWb


# ------------------------------------------------------------ MXFP4 helpers ----

def mx_codes(rows: int, K: int, device):
    """uint8 buffer for the MXFP4 codes of a rows x K matrix in the library's block layout:
    [ceil(rows/256) x 128*K], one row per 256-row block (its stride is the layout's ld)."""
    import torch
    return torch.empty((rows + 255) // 256, 128 * K, dtype=torch.uint8, device=device)


@dataclass
class MxQuantized:
    Qh: object           # mx_codes(T, D): E2M1 codes, blocks along D
    Qh_scales: object    # uint8 [D/128 x 4T] E8M0, step-grouped
    Qt: object           # mx_codes(D, T): codes of G^T, blocks along T
    Qt_scales: object    # uint8 [T/128 x 4D]
    desc: QDesc
    ec_h: tuple = (None, None, None)   # (eps_t [T], ebar [B x D], mu [B]) of Q_h's error
    ec_t: tuple = (None, None, None)   # the same for Q_t
    flags: object = None


def mx_quantize(G, *, mode=S3R, ec=EC_NONE, seed=0, layer_id=0, rows_per_example=None, stream=None,
                threshold_stream=0) -> MxQuantized:
    import torch
    T, D = G.shape
    desc = qdesc(T, D, rows_per_example, mode, ec, PER_TENSOR, layer_id, seed, threshold_stream)
    dev = G.device
    B = T // desc.rows_per_example
    u8 = dict(dtype=torch.uint8, device=dev)
    Qh, Qhs = mx_codes(T, D, G.device), torch.empty(D // 128, 4 * T, **u8)
    Qt, Qts = mx_codes(D, T, G.device), torch.empty(T // 128, 4 * D, **u8)
    ec_h = ec_t = (None, None, None)
    if ec != EC_NONE:
        f32 = dict(dtype=torch.float32, device=dev)
        ec_h = (torch.empty(T, **f32), torch.empty(B, D, **f32), torch.empty(B, **f32))
        ec_t = (torch.empty(T, **f32), torch.empty(B, D, **f32), torch.empty(B, **f32))
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(s3r_mx_workspace(desc, 0), dev)
    s3r_mx_quantize(desc, G, Qh, Qhs, Qt, Qts, *ec_h, *ec_t, flags, ws, stream)
    return MxQuantized(Qh, Qhs, Qt, Qts, desc, ec_h, ec_t, flags)


def mx_operand(M, rows_per_example=None, colsum=True, stream=None):
    """RTNE MXFP4 of a forward operand, stored transposed: (Mt, Mt_scales, colsum or None)."""
    import torch
    rows, cols = M.shape
    S = rows if rows_per_example is None else rows_per_example
    dev = M.device
    Mt = mx_codes(cols, rows, dev)
    Mts = torch.empty(rows // 128, 4 * cols, dtype=torch.uint8, device=dev)
    cs = torch.empty(rows // S, cols, dtype=torch.float32, device=dev) if colsum else None
    ws = _workspace(s3r_mx_operand_workspace(rows, cols), dev)
    s3r_mx_operand(M, Mt, Mts, cs, S, None, ws, stream)
    return Mt, Mts, cs


def mx_backward_dx(q: MxQuantized, Wt, Wt_scales, r_W=None, stream=None):
    import torch
    d_in = Wt_scales.shape[1] // 4
    dX = torch.empty(q.desc.rows, d_in, dtype=torch.float32, device=Wt.device)
    ws = _workspace(s3r_mx_workspace(q.desc, d_in), Wt.device)
    s3r_mx_backward_dx(q.desc, q.Qh, q.Qh_scales, Wt, Wt_scales, r_W, *q.ec_h, dX, ws, stream)
    return dX


def mx_backward_dw(q: MxQuantized, Xt, Xt_scales, xs=None, stream=None):
    import torch
    d_in = Xt_scales.shape[1] // 4
    dW = torch.empty(q.desc.cols, d_in, dtype=torch.float32, device=Xt.device)
    ws = _workspace(s3r_mx_workspace(q.desc, d_in), Xt.device)
    s3r_mx_backward_dw(q.desc, q.Qt, q.Qt_scales, Xt, Xt_scales, xs, *q.ec_t, dW, ws, stream)
    return dW
