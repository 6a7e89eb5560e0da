"""libs3r.so loads and exports what include/s3r.h declares; host-side checks (no GPU needed).

Argument validation happens before any HIP call, so these error paths run on
a machine without a GPU.
"""
import ctypes
import os
import re

import numpy as np

import pytest

from stochastic_rounding_quantization_amd import s3r

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(s3r.LIB_PATH):
        from stochastic_rounding_quantization_amd import build
        build.build()
    return s3r.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "s3r.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s3r_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(s3r.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status(L):
    assert s3r.s3r_version() == 200
    assert s3r.s3r_status_string(0) == "ok"
    assert s3r.s3r_status_string(-3) == "workspace too small"


def _call_quantize(L, desc, G=1, gdt=0, ldg=None, Q=1, ldq=None, delta=1, ec=(None, None, None), ws=None,
                   wsb=0, colsum=None):
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    ldg = desc.cols if ldg is None else ldg
    ldq = desc.cols if ldq is None else ldq
    return L.s3r_quantize(ctypes.byref(desc) if desc is not None else None, P(G), gdt, ldg, None, None, P(Q), ldq,
                          P(delta), P(colsum), P(ec[0]), P(ec[1]), P(ec[2]), None, P(ws), wsb, None)


def test_quantize_argument_errors(L):
    d = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE)
    assert L.s3r_quantize(None, None, 0, 0, None, None, None, 0, None, None, None, None, None, None, None, 0,
                          None) == -1
    bad = s3r.qdesc(64, 96, 30)                         # T % S != 0
    assert _call_quantize(L, bad) == -1
    assert _call_quantize(L, d, gdt=2) == -2            # int32 gradient
    assert _call_quantize(L, s3r.qdesc(64, 96, 32, s3r.RTNE, s3r.EC_TWO_WAY), ec=(1, 1, 1)) == -2
    assert _call_quantize(L, s3r.qdesc(64, 96, 32, s3r.SR, s3r.EC_DW_ONLY), ec=(1, 1, 1)) == -2
    assert _call_quantize(L, s3r.qdesc(64, 96, 32, 4)) == -2                      # no such mode
    assert _call_quantize(L, s3r.qdesc(64, 96, 32, s3r.S3R, 4)) == -2             # no such correction
    assert _call_quantize(L, s3r.qdesc(64, 96, 32, stream=65536)) == -1           # stream beyond 16 bits
    r = s3r.qdesc(64, 96, 32)
    r.reserved = 1
    assert _call_quantize(L, r) == -1
    assert _call_quantize(L, d, ldg=95) == -1           # leading dim < cols
    assert _call_quantize(L, d, G=None) == -1
    assert _call_quantize(L, d, delta=None) == -1
    ecd = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_TWO_WAY)
    assert _call_quantize(L, ecd) == -1                 # EC outputs missing
    need = s3r.s3r_quantize_workspace(ecd)
    assert need > 0
    assert _call_quantize(L, ecd, ec=(256, 512, 768), ws=4096, wsb=need - 1) == -3
    assert _call_quantize(L, d, ec=(256, 512, 768)) == -1   # EC outputs without EC
    m = s3r.qdesc(64, 96, 32, 7)
    assert _call_quantize(L, m) == -2


def test_backward_argument_errors(L):
    P = ctypes.c_void_p
    d = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE)
    args = dict(Q=P(4096), ldq=96, delta=P(16), W=P(8192), ldw=128, din=128, out=P(4096), odt=0, ldo=128)

    def dx(**kw):
        a = {**args, **kw}
        return L.s3r_backward_dx(ctypes.byref(d if "d" not in kw else kw["d"]), a["Q"], a["ldq"], a["delta"],
                                 a["W"], a["ldw"], a["din"], None, None, None, None, None, a["out"], a["odt"],
                                 a["ldo"], None, 0, None)

    def dw(**kw):
        a = {**args, **kw}
        return L.s3r_backward_dw(ctypes.byref(d if "d" not in kw else kw["d"]), a["Q"], a["ldq"], a["delta"],
                                 a["W"], a["ldw"], a["din"], None, None, None, None, None, a["out"], a["odt"],
                                 a["ldo"], None, 0, None)

    assert dx(ldq=100) == -1                 # GEMM operand leading dim not a multiple of 16
    assert dx(Q=P(4097)) == -1               # misaligned operand
    assert dx(odt=1) == -2                   # bf16 output not offered
    assert dx(ldo=100) == -1
    big = s3r.qdesc(64, 200000, 32)
    assert dx(d=big, ldq=200000) == -1       # K beyond the int32 accumulator bound
    ecd = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_DX_ONLY)
    assert dx(d=ecd) == -1                   # correction inputs missing
    pt = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE, s3r.PER_TOKEN)
    assert dw(d=pt) == -3                    # per-token dW requantizes the inputs in the workspace
    assert s3r.s3r_backward_workspace(pt, 128) >= 64 * 128 + 2 * 128 * 4
    assert s3r.s3r_backward_workspace(s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_TWO_WAY), 128) > 0
    assert s3r.s3r_backward_workspace(d, 128) == 0


def test_backward_dw_pair_argument_errors(L):
    P = ctypes.c_void_p
    d = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE)
    args = dict(Q0=P(4096), Q1=P(8192), ldq=96, X=P(16384), ldx=128, din=128, out0=P(32768), out1=P(65536), odt=0,
                ldo=128, ec=(None,) * 6, xs=None, ws=None, wsb=0)

    def pair(**kw):
        a = {**args, **kw}
        return L.s3r_backward_dw_pair(ctypes.byref(kw.get("d", d)), a["Q0"], a["Q1"], a["ldq"], P(16), P(32), a["X"],
                                      a["ldx"], a["din"], None, None, a["xs"], *a["ec"], a["out0"], a["out1"],
                                      a["odt"], a["ldo"], a["ws"], a["wsb"], None)

    assert pair(Q1=P(4097)) == -1            # misaligned second operand
    assert pair(out1=None) == -1             # second output missing
    assert pair(odt=3) == -2                 # accumulation is dX only
    pt = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE, s3r.PER_TOKEN)
    assert pair(d=pt) == -2                  # per-tensor steps only
    ec = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_TWO_WAY)
    assert pair(d=ec) == -1                  # correction inputs missing
    full = dict(xs=P(1 << 20), ec=tuple(P(1 << 21 + i) for i in range(6)))
    need = s3r.s3r_backward_dw_pair_workspace(ec, 128)
    one = s3r.s3r_backward_workspace(s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_DW_ONLY), 128)   # a dW's alone
    assert need == 2 * ((one + 255) // 256 * 256) > 0                 # one correction GEMV's workspace per product
    assert pair(d=ec, **full, ws=P(1 << 22), wsb=need - 1) == -3
    assert pair(d=ec, **full, ws=P((1 << 22) + 64), wsb=need) == -3    # workspace not 256-byte aligned
    assert s3r.s3r_backward_dw_pair_workspace(d, 128) == 0
    assert s3r.s3r_backward_dw_pair_workspace(pt, 128) == 0


def test_swiglu_argument_errors(L):
    P = ctypes.c_void_p
    ok = dict(T=4, F=16, dH=P(256), ldh=16, Ag=P(512), Au=P(768), lda=16, Gg=P(1024), Gu=P(1280), ldg=16)

    def call(**kw):
        a = {**ok, **kw}
        return L.s3r_swiglu_backward(a["T"], a["F"], a["dH"], a["ldh"], a["Ag"], a["Au"], a["lda"], a["Gg"],
                                     a["Gu"], a["ldg"], None)

    assert call(T=-1) == -1
    assert call(ldh=8) == -1 and call(lda=8) == -1 and call(ldg=8) == -1
    assert call(dH=None) == -1 and call(Gu=None) == -1


def test_swiglu_amax_and_quantize_with_amax_argument_errors(L):
    P = ctypes.c_void_p
    ok = dict(T=4, F=16, dH=P(256), ldh=16, Ag=P(512), Au=P(768), lda=16, Gg=P(1024), Gu=P(1280), ldg=16,
              amax=P(2048), ws=P(4096), wsb=1 << 20)

    def glue(**kw):
        a = {**ok, **kw}
        return L.s3r_swiglu_backward_amax(a["T"], a["F"], a["dH"], a["ldh"], a["Ag"], a["Au"], a["lda"], a["Gg"],
                                          a["Gu"], a["ldg"], None, None, None, a["amax"], a["ws"], a["wsb"], None)

    assert glue(T=-1) == -1 and glue(ldg=8) == -1 and glue(dH=None) == -1
    assert glue(amax=None) == -1                     # the amax output is required
    need = s3r.s3r_swiglu_amax_workspace(4, 16)
    assert need > 0 and glue(wsb=need - 1) == -3     # workspace below s3r_swiglu_amax_workspace
    assert glue(ws=P(4100)) == -1                    # workspace not 256-byte aligned
    assert s3r.s3r_swiglu_amax_workspace(8192, 14336) > need

    def qa(desc, amax=P(64), G=P(1), Q=P(1), delta=P(1), ec=(None, None, None), wsb=0, ws=None):
        return L.s3r_quantize_with_amax(ctypes.byref(desc), G, 0, desc.cols, None, None, amax, Q, desc.cols, delta,
                                        ec[0], ec[1], ec[2], None, ws, wsb, None)

    d = s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE)
    assert qa(s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_NONE, s3r.PER_TOKEN)) == -2   # per-tensor steps only
    assert qa(d, amax=None) == -1
    assert qa(d, Q=None) == -1
    assert qa(s3r.qdesc(64, 96, 32, s3r.S3R, s3r.EC_TWO_WAY)) == -1               # statistics outputs missing
    assert qa(d, wsb=0) in (-3, -4, -5)                                           # workspace or no device


def test_swiglu_quantize_argument_errors(L):
    P = ctypes.c_void_p
    T, F, S = 64, 96, 32

    def call(dg=None, du=None, dH=P(256), ldh=F, Ag=P(512), Au=P(768), lda=F, Qg=P(1024), Qu=P(1280), ldq=F,
             dlg=P(64), dlu=P(128), ecg=(None, None, None), ecu=(None, None, None), ws=P(4096), wsb=1 << 24):
        dg = dg or s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_NONE)
        du = du or s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_NONE, layer_id=1)
        return L.s3r_swiglu_quantize(ctypes.byref(dg), ctypes.byref(du), dH, ldh, Ag, Au, lda, None, None, None, Qg,
                                     Qu, ldq, dlg, dlu, *ecg, *ecu, None, ws, wsb, None)

    pt = s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_NONE, s3r.PER_TOKEN)
    assert call(dg=pt, du=pt) == -2                                            # per-tensor steps only
    assert call(du=s3r.qdesc(T, F, S, s3r.SR, s3r.EC_NONE)) == -1              # modes differ
    assert call(du=s3r.qdesc(T, F + 8, S, s3r.S3R, s3r.EC_NONE)) == -1         # shapes differ
    assert call(du=s3r.qdesc(T, F, 64, s3r.S3R, s3r.EC_NONE)) == -1            # examples differ
    sr_ec = s3r.qdesc(T, F, S, s3r.SR, s3r.EC_TWO_WAY)
    assert call(dg=sr_ec, du=sr_ec) == -2                                      # correction needs shared thresholds
    assert call(ldh=F - 1) == -1 and call(lda=F - 1) == -1 and call(ldq=F - 1) == -1
    assert call(dH=None) == -1 and call(Qu=None) == -1 and call(dlg=None) == -1
    ec = s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_TWO_WAY)
    assert call(dg=ec, du=ec) == -1                                            # statistics outputs missing
    assert call(ecg=(P(1), None, None)) == -1                                  # statistics without correction
    need = s3r.s3r_swiglu_quantize_workspace(s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_NONE))
    assert need > 0 and call(wsb=need - 1) == -3
    assert call(ws=P(4100)) == -1
    assert s3r.s3r_swiglu_quantize_workspace(pt) == 0
    # two quantizers' partial sums (1 + 1/512 floats per element each) and the glue pass's partial maxima
    big = s3r.s3r_swiglu_quantize_workspace(s3r.qdesc(8192, 14336, 2048, s3r.S3R, s3r.EC_TWO_WAY))
    assert big >= 2 * 4 * (8192 * 14336 // 64 + 8192 * 28) + s3r.s3r_swiglu_amax_workspace(8192, 14336)
    assert call(wsb=need) in (-4, -5)                                          # valid: no device here


class _FakeDev:
    """Stands in for a device tensor in the binding's marshalling (never dereferenced on the host)."""

    def __init__(self, shape, stride, addr=1 << 20, elem=1, dtype=None):
        import torch
        self._shape, self._stride, self._addr, self._elem = shape, stride, addr, elem
        self.shape = shape
        self.dtype = dtype or {1: torch.int8, 4: torch.float32, 8: torch.int64}[elem]

    def data_ptr(self):
        return self._addr

    def dim(self):
        return len(self._shape)

    def stride(self, i=None):
        return self._stride if i is None else self._stride[i]

    def numel(self):
        n = 1
        for d in self._shape:
            n *= d
        return n

    def element_size(self):
        return self._elem


def test_grouped_binding_marshals_valid_arguments(L):
    # through the Python binding with consistent shapes, every check passes and (without a GPU)
    # the call stops at the device check: the argument order matches the C declarations
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    R, D, d_in, E = 96, 64, 48, 4
    desc = s3r.qdesc(R, D, 1, s3r.S3R, s3r.EC_TWO_WAY)
    ws = _FakeDev((s3r.s3r_grouped_workspace(desc, E, d_in),), (1,), addr=1 << 24)
    off = _FakeDev((E + 1,), (1,), elem=8)
    f32 = lambda *shape: _FakeDev(shape, tuple(int(np.prod(shape[i + 1:])) for i in range(len(shape))), elem=4)
    Q = _FakeDev((R, D), (D, 1))
    st = (f32(R), f32(E, D), f32(E))
    expect = (-4, -5)
    assert s3r.s3r_grouped_quantize(desc, off, f32(R, D), f32(R), f32(E, D), Q, f32(E), None, *st, None, ws, 0,
                                    rc_only=True) in expect
    Wq = _FakeDev((E, D, d_in), (D * 48, 48, 1))
    dX = f32(R, d_in)
    assert s3r.s3r_grouped_backward_dx(desc, off, Q, f32(E), Wq, f32(R), f32(E, d_in), *st, dX, None, ws, 0,
                                       rc_only=True) in expect
    dW = f32(E, D, d_in)
    Xq = _FakeDev((R, d_in), (48, 1))
    assert s3r.s3r_grouped_backward_dw(desc, off, Q, f32(E), Xq, f32(E, D), f32(E, d_in), *st, dW, None, ws, 0,
                                       rc_only=True) in expect
    # the grouped dW's output leading dimension stays below 2^21 (its dropped stores' offsets must not wrap)
    for ld, rc in (((1 << 21) - 1, expect), (1 << 21, (-1,))):
        wide = _FakeDev((E, D, d_in), (D * ld, ld, 1), elem=4)
        assert s3r.s3r_grouped_backward_dw(desc, off, Q, f32(E), Xq, f32(E, D), f32(E, d_in), *st, wide, None, ws,
                                           0, rc_only=True) in rc, ld


def test_mx_argument_errors(L):
    P = ctypes.c_void_p
    T, D, d_in = 256, 128, 96
    ok = s3r.qdesc(T, D, 128, s3r.S3R, s3r.EC_TWO_WAY)
    ec6 = [P(4096 * (i + 1)) for i in range(6)]

    # codes: ld is the byte stride between 256-row blocks, a multiple of 16384 and at least 128 K
    def q(desc, G=P(1 << 20), Qh=P(1 << 21), Qt=P(1 << 22), ld_qt=None, ec=ec6, wsb=1 << 24, ws=P(1 << 23)):
        return L.s3r_mx_quantize(ctypes.byref(desc), G, 0, desc.cols, Qh, 128 * desc.cols, P(1 << 19),
                                 4 * desc.rows, Qt, 128 * desc.rows if ld_qt is None else ld_qt, P(1 << 18),
                                 4 * desc.cols, *ec, None, ws, wsb, None)

    assert q(s3r.qdesc(T, 96, 128, s3r.S3R)) == -1                      # D not a multiple of 128
    assert q(s3r.qdesc(T, D, 64, s3r.S3R)) == -1                        # rows per example not a multiple of 128
    assert q(s3r.qdesc(T, D, 128, s3r.S3R_BCAST)) == -2                 # no per-example thresholds here
    assert q(s3r.qdesc(T, D, 128, s3r.SR, s3r.EC_TWO_WAY)) == -2        # EC needs S3R
    assert q(s3r.qdesc(T, D, 128, s3r.S3R, scale=s3r.PER_TOKEN)) == -2
    assert q(ok, ec=[None] * 6) == -1                                   # statistics outputs missing
    assert q(s3r.qdesc(T, D, 128, s3r.S3R), ec=[None] * 6, ld_qt=128 * T + 16) == -1   # block stride not 16 KiB-aligned
    assert q(s3r.qdesc(T, D, 128, s3r.S3R), ec=[None] * 6, ld_qt=128 * T - 16384) == -1  # below 128 K
    assert q(ok, Qt=P((1 << 22) + 8)) == -1                              # Qt base not 16-aligned
    assert q(ok, G=P((1 << 20) + 4)) == -1                               # G not 16-byte aligned
    assert q(ok, wsb=16) == -3
    assert q(ok, ws=P((1 << 23) + 64)) == -1
    assert s3r.s3r_mx_workspace(s3r.qdesc(T, 96, 128), d_in) == 0

    def dx(desc, ld_wt=128 * D, ldws=4 * d_in, Wt=P(1 << 24), ec=True, wsb=1 << 24):
        e = ec6[:3] if ec else [None] * 3
        return L.s3r_mx_backward_dx(ctypes.byref(desc), P(1 << 20), 128 * D, P(1 << 19), 4 * T, Wt, ld_wt,
                                    P(1 << 18), ldws, d_in, ec6[3], *e, P(1 << 25), d_in, P(1 << 23), wsb, None)

    assert dx(ok, ld_wt=D // 2) == -1                                   # a plain row stride is not the layout
    assert dx(ok, ldws=4 * d_in - 4) == -1                              # scale step stride below 4 rows
    assert dx(ok, Wt=P((1 << 24) + 4)) == -1
    assert dx(ok, ec=False) == -1                                       # TWO_WAY needs the statistics
    assert dx(ok, wsb=0) == -3

    def dw(desc, xs=ec6[3]):
        R = desc.rows
        return L.s3r_mx_backward_dw(ctypes.byref(desc), P(1 << 20), 128 * R, P(1 << 19), 4 * D, P(1 << 24),
                                    128 * R, P(1 << 18), 4 * d_in, d_in, xs, *ec6[:3], P(1 << 25), d_in,
                                    P(1 << 23), 1 << 24, None)

    assert dw(ok, xs=None) == -1
    assert dw(s3r.qdesc(128 * 9, D, 128, s3r.S3R, s3r.EC_TWO_WAY)) in (-4, -5)  # nine examples: accepted
    assert dw(s3r.qdesc(128 * 9, D, 128, s3r.S3R, s3r.EC_DX_ONLY)) in (-4, -5)  # dW uncorrected: any B

    def op(rows=T, cols=d_in, S=T, ld_t=128 * T, wsb=1 << 20):
        return L.s3r_mx_operand(rows, cols, S, P(1 << 20), 0, cols, P(1 << 21), ld_t, P(1 << 19), 4 * cols,
                                None, None, P(1 << 23), wsb, None)

    assert op(rows=200) == -1 and op(S=96) == -1 and op(ld_t=T // 2) == -1 and op(ld_t=128 * T + 4) == -1
    assert op(wsb=8) == -3
    assert op() in (-4, -5)


def test_mx_binding_marshals_valid_arguments(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    T, D, d_in = 256, 128, 96
    desc = s3r.qdesc(T, D, 128, s3r.S3R, s3r.EC_TWO_WAY)
    ws = _FakeDev((s3r.s3r_mx_workspace(desc, d_in),), (1,), addr=1 << 24)
    f32 = lambda *shape: _FakeDev(shape, tuple(int(np.prod(shape[i + 1:])) for i in range(len(shape))), elem=4)
    u8 = lambda r, c: _FakeDev((r, c), (c, 1), dtype=torch.uint8)
    codes = lambda rows, K: u8((rows + 255) // 256, 128 * K)     # the block layout's shape (s3r.mx_codes)
    st = (f32(T), f32(2, D), f32(2))
    expect = (-4, -5)
    assert s3r.s3r_mx_quantize(desc, f32(T, D), codes(T, D), u8(D // 128, 4 * T), codes(D, T), u8(T // 128, 4 * D),
                               *st, *st, None, ws, 0, rc_only=True) in expect
    assert s3r.s3r_mx_backward_dx(desc, codes(T, D), u8(D // 128, 4 * T), codes(d_in, D), u8(D // 128, 4 * d_in),
                                  f32(d_in), *st, f32(T, d_in), ws, 0, rc_only=True) in expect
    assert s3r.s3r_mx_backward_dw(desc, codes(D, T), u8(T // 128, 4 * D), codes(d_in, T), u8(T // 128, 4 * d_in),
                                  f32(2, d_in), *st, f32(D, d_in), ws, 0, rc_only=True) in expect
    ows = _FakeDev((s3r.s3r_mx_operand_workspace(T, d_in),), (1,), addr=1 << 24)
    assert s3r.s3r_mx_operand(f32(T, d_in), codes(d_in, T), u8(T // 128, 4 * d_in), f32(2, d_in), 128, None, ows, 0,
                              rc_only=True) in expect


def test_no_gpu_reports_hip_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = s3r.qdesc(64, 96, 32, s3r.RTNE)
    rc = _call_quantize(L, d, ws=4096, wsb=1 << 20)
    assert rc in (-4, -5)


def test_product_path_does_not_import_oracle():
    # the product path (package + bench entry) must not route through the CPU oracle
    pkg = os.path.join(ROOT, "stochastic_rounding_quantization_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_gemm_m0_written_only_by_its_dma_assembly(tmp_path):
    """The GEMM rings issue their LDS DMAs as inline assembly that sets M0 (the LDS address) itself; the
    compiler is not told, so no compiler-generated instruction of gemm.hip may read or write M0."""
    from stochastic_rounding_quantization_amd import build
    import subprocess
    src = os.path.join(build.CSRC, "gemm.hip")
    out = tmp_path / "gemm.s"
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(build.ROOT, "include"), src,
           "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    inside, dma_blocks, stray = False, 0, []
    for line in out.read_text().splitlines():
        if "ASMSTART" in line:
            inside = True
            continue
        if "ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0]
        if inside:
            dma_blocks += "buffer_load_dwordx4" in code and " lds" in code
        elif re.search(r"\bm0\b", code):
            stray.append(line.strip())
    assert dma_blocks > 0
    assert not stray, stray[:5]


def test_quantize_noalloc_size_limit(L):
    # the no-alloc quantizer refuses, before touching the device, a call whose partials exceed its
    # array: with EC the column partials of 2^20 tokens x 4096 channels need 1 GiB
    P = ctypes.c_void_p
    assert s3r.S3R_NOALLOC_SCRATCH_BYTES == 32 << 20

    def call(T, D, S, ec, colsum=None):
        d = s3r.qdesc(T, D, S, s3r.S3R, ec)
        ecp = (P(1024), P(2048), P(4096)) if ec else (None, None, None)
        return L.s3r_quantize_noalloc(ctypes.byref(d), P(256), s3r.S3R_BF16, D, None, None, P(512), D, P(768),
                                      colsum, *ecp, None, None)

    assert call(1 << 20, 4096, 1 << 20, s3r.EC_TWO_WAY) == -3
    # within the limit the size check passes; without a GPU the call then stops at the device checks
    assert call(8192, 4096, 2048, s3r.EC_TWO_WAY) in (-4, -5)
    assert call(8192, 14336, 2048, s3r.EC_TWO_WAY, colsum=P(8192)) in (-4, -5)
    # argument errors are still reported as for s3r_quantize
    d = s3r.qdesc(64, 96, 31, s3r.S3R, s3r.EC_NONE)
    assert L.s3r_quantize_noalloc(ctypes.byref(d), P(256), 1, 96, None, None, P(512), 96, P(768), None, None, None,
                                  None, None, None) == -1
