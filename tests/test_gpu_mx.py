"""Parity of the MXFP4 variant with the oracle (oracle/mx.py), through the C ABI, on an MI355X.

Bars: E2M1 codes and E8M0 scales of both quantizations of G and of the two
forward operands bit-exact; the error statistics and the operand column sums
within 1e-5 (fp32 results of fp64 sums); dX and dW, raw and corrected, within
1e-5 of the oracle relative to the largest magnitude (fp32 accumulation of
exact FP4 products in the matrix cores against fp64).
"""
import numpy as np
import pytest
import torch

from oracle import mx, quantize as oq
from stochastic_rounding_quantization_amd import inputs, s3r
from tests._gpu import DEV, assert_rows_close, host, mx_rows, rel_err, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5

MODE = {oq.RTNE: s3r.RTNE, oq.SR: s3r.SR, oq.S3R: s3r.S3R}
EC = {oq.EC_NONE: s3r.EC_NONE, oq.EC_DX_ONLY: s3r.EC_DX_ONLY, oq.EC_TWO_WAY: s3r.EC_TWO_WAY,
      oq.EC_DW_ONLY: s3r.EC_DW_ONLY}


def _problem(T, D, d_in, dtype, seed, outliers=0):
    h = inputs.MX_WORKLOADS["mx-down-8192x14336x4096-bf16"]
    w = inputs.Workload(f"mx-{T}x{d_in}x{D}", 60 + seed, T, d_in, D, T, dtype, h.g_nu, h.g_scale)
    inp = inputs.make_linear_inputs(w)
    if outliers:
        g = inputs.bf16_bits_to_f32(inp["G"]) if dtype == "bf16" else inp["G"].copy()
        rng = np.random.default_rng(seed)
        g[rng.integers(0, T, outliers)] *= 1e4
        inp["G"] = inputs.f32_to_bf16_bits(g) if dtype == "bf16" else g
    return inp


def _f32(inp, k):
    a = inp[k]
    return inputs.bf16_bits_to_f32(a) if inp["dtype"] == "bf16" else np.asarray(a, np.float32)


def gpu_mx(inp, *, mode, ec, S, seed=0, layer_id=0):
    dt = inp["dtype"]
    G, X, W = to_dev(inp["G"], dt), to_dev(inp["X"], dt), to_dev(inp["W"], dt)
    D = G.shape[1]
    q = s3r.mx_quantize(G, mode=MODE[mode], ec=EC[ec], seed=seed, layer_id=layer_id, rows_per_example=S)
    Wt, Wts, rW = s3r.mx_operand(W, rows_per_example=D)
    Xt, Xts, xs = s3r.mx_operand(X, rows_per_example=S)
    dX = s3r.mx_backward_dx(q, Wt, Wts, rW[0])
    dW = s3r.mx_backward_dw(q, Xt, Xts, xs)
    torch.cuda.synchronize()
    return dict(q=q, Wt=Wt, Wts=Wts, rW=rW, Xt=Xt, Xts=Xts, xs=xs, dX=dX, dW=dW)


def step_grouped(scale):
    """Scales [R x K/32] (one byte per row and block) -> the library's layout [K/128][R][4]."""
    R, nb = scale.shape
    return np.ascontiguousarray(scale.reshape(R, nb // 4, 4).transpose(1, 0, 2)).reshape(nb // 4, 4 * R)


def _check_quant(gpu, ref):
    q = gpu["q"]
    T, D = q.desc.rows, q.desc.cols
    d_in = gpu["Wts"].shape[1] // 4
    np.testing.assert_array_equal(mx_rows(q.Qh, T, D), mx.pack(ref["qh"]["codes"]))
    np.testing.assert_array_equal(host(q.Qh_scales), step_grouped(ref["qh"]["scale"]))
    np.testing.assert_array_equal(mx_rows(q.Qt, D, T), mx.pack(ref["qt"]["codes"].T))
    np.testing.assert_array_equal(host(q.Qt_scales), step_grouped(ref["qt"]["scale"]))
    np.testing.assert_array_equal(mx_rows(gpu["Wt"], d_in, D), mx.pack(ref["fw"]["codes"].T))
    np.testing.assert_array_equal(host(gpu["Wts"]), step_grouped(ref["fw"]["scale"]))
    np.testing.assert_array_equal(mx_rows(gpu["Xt"], d_in, T), mx.pack(ref["fx"]["codes"].T))
    np.testing.assert_array_equal(host(gpu["Xts"]), step_grouped(ref["fx"]["scale"]))
    assert int(host(q.flags)[0]) == 0


def _check_stats(gpu, ref, S):
    Wd, Xd = ref["fw"]["deq"], ref["fx"]["deq"]
    assert rel_err(host(gpu["rW"])[0], Wd.sum(axis=0)) < TOL
    B = Xd.shape[0] // S
    assert rel_err(host(gpu["xs"]), Xd.reshape(B, S, -1).sum(axis=1)) < TOL
    q = gpu["q"]
    if q.ec_h[0] is None:
        return
    for nm, st in (("h", q.ec_h), ("t", q.ec_t)):
        assert rel_err(host(st[0]), ref["eps_" + nm]) < TOL, nm
        assert rel_err(host(st[1]), ref["ebar_" + nm]) < TOL, nm
        # mu_b is a mean of the eps_t: compared on their scale (it may be near zero itself)
        assert np.abs(host(st[2]) - ref["mu_" + nm]).max() <= TOL * np.abs(ref["eps_" + nm]).max(), nm


@pytest.mark.parametrize("mode,ec", [(oq.RTNE, oq.EC_NONE), (oq.SR, oq.EC_NONE), (oq.S3R, oq.EC_NONE),
                                     (oq.S3R, oq.EC_TWO_WAY), (oq.S3R, oq.EC_DX_ONLY), (oq.S3R, oq.EC_DW_ONLY)])
def test_mx_small_f32_modes(mode, ec):
    # two examples, a ragged d_in (not a multiple of 32 or of the 256-wide tile)
    T, D, d_in, S = 256, 384, 200, 128
    inp = _problem(T, D, d_in, "f32", 1)
    gpu = gpu_mx(inp, mode=mode, ec=ec, S=S, seed=3, layer_id=2)
    ref = mx.backward(_f32(inp, "G"), _f32(inp, "X"), _f32(inp, "W"), mode=mode, ec=ec, rows_per_example=S,
                      seed=3, layer_id=2)
    _check_quant(gpu, ref)
    _check_stats(gpu, ref, S)
    assert_rows_close(host(gpu["dX"]), ref["dX"], TOL, "mx dX")
    assert_rows_close(host(gpu["dW"]), ref["dW"], TOL, "mx dW")


@pytest.mark.parametrize("T,D,d_in,S", [(384, 256, 40, 128), (768, 640, 600, 256), (512, 128, 520, 512),
                                         (256, 2304, 100, 128)])
def test_mx_tiles_and_tails_bf16(T, D, d_in, S):
    # partial 256-row tiles (T = 384), several tiles both ways, outlier tokens; D = 2304 gives the v
    # correction product one whole 2048-element chunk and a partial one (8 of 64 blocks), d_in = 100 a
    # partial group of 32 rows
    inp = _problem(T, D, d_in, "bf16", 2, outliers=3)
    gpu = gpu_mx(inp, mode=oq.S3R, ec=oq.EC_TWO_WAY, S=S, seed=11)
    ref = mx.backward(_f32(inp, "G"), _f32(inp, "X"), _f32(inp, "W"), mode=oq.S3R, ec=oq.EC_TWO_WAY,
                      rows_per_example=S, seed=11)
    _check_quant(gpu, ref)
    _check_stats(gpu, ref, S)
    assert_rows_close(host(gpu["dX"]), ref["dX"], TOL, "mx dX")
    assert_rows_close(host(gpu["dW"]), ref["dW"], TOL, "mx dW")


@pytest.mark.parametrize("ec", [oq.EC_DX_ONLY, oq.EC_TWO_WAY])
def test_mx_many_examples(ec):
    # nine examples: the dX correction's GEMV runs in passes of four examples (4 + 4 + 1);
    # the dW epilogue applies the first eight examples' terms and a rank-update pass the ninth
    T, D, d_in, S = 128 * 9, 256, 136, 128
    inp = _problem(T, D, d_in, "f32", 5)
    gpu = gpu_mx(inp, mode=oq.S3R, ec=ec, S=S, seed=4)
    ref = mx.backward(_f32(inp, "G"), _f32(inp, "X"), _f32(inp, "W"), mode=oq.S3R, ec=ec,
                      rows_per_example=S, seed=4)
    _check_quant(gpu, ref)
    _check_stats(gpu, ref, S)
    assert_rows_close(host(gpu["dX"]), ref["dX"], TOL, f"mx dX, 9 examples, ec={ec}")
    assert_rows_close(host(gpu["dW"]), ref["dW"], TOL, f"mx dW, 9 examples, ec={ec}")


def test_mx_headline_workload_sampled():
    # T = 8192 (4 examples of 2048), D = 4096, d_in = 14336, bf16, S3R-EC two-way, in the launch
    # configuration the benchmark times; every code and scale of G compared, dX / dW on sampled
    # rows and columns (the oracle quantizes the sampled columns of W and X on their own)
    w = inputs.MX_WORKLOADS["mx-down-8192x14336x4096-bf16"]
    inp = inputs.make_linear_inputs(w)
    T, D, d_in, S = w.tokens, w.d_out, w.d_in, w.rows_per_example
    print(f"mx headline {T}x{D}x{d_in}", flush=True)
    gpu = gpu_mx(inp, mode=oq.S3R, ec=oq.EC_TWO_WAY, S=S, seed=0)
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, S - 1, S, T - 1], rng.choice(T, 12, replace=False)])
    crow = np.concatenate([[0, D - 1], rng.choice(D, 10, replace=False)])
    cols = np.concatenate([[0, 255, 256, d_in - 1], rng.choice(d_in, 12, replace=False)])
    ref = mx.backward(_f32(inp, "G"), _f32(inp, "X"), _f32(inp, "W"), mode=oq.S3R, ec=oq.EC_TWO_WAY,
                      rows_per_example=S, seed=0, dx_rows=rows, dw_rows=crow, cols=cols)
    q = gpu["q"]
    np.testing.assert_array_equal(mx_rows(q.Qh, T, D), mx.pack(ref["qh"]["codes"]))
    np.testing.assert_array_equal(host(q.Qh_scales), step_grouped(ref["qh"]["scale"]))
    np.testing.assert_array_equal(mx_rows(q.Qt, D, T), mx.pack(ref["qt"]["codes"].T))
    np.testing.assert_array_equal(host(q.Qt_scales), step_grouped(ref["qt"]["scale"]))
    np.testing.assert_array_equal(mx_rows(gpu["Wt"], d_in, D)[cols], mx.pack(ref["fw"]["codes"].T))
    np.testing.assert_array_equal(mx_rows(gpu["Xt"], d_in, T)[cols], mx.pack(ref["fx"]["codes"].T))
    for nm, st in (("h", q.ec_h), ("t", q.ec_t)):
        assert rel_err(host(st[0]), ref["eps_" + nm]) < TOL, nm
        assert rel_err(host(st[1]), ref["ebar_" + nm]) < TOL, nm
    assert_rows_close(host(gpu["dX"])[np.ix_(rows, cols)], ref["dX"], TOL, "mx headline dX (sampled)")
    assert_rows_close(host(gpu["dW"])[np.ix_(crow, cols)], ref["dW"], TOL, "mx headline dW (sampled)")
