"""Parity of the grouped (MoE expert) path with the oracle, through the C ABI, on an MI355X.

Rows are sorted by expert; every expert is one linear layer whose backward is the
dense path on its rows (oracle/moe.py).  Bars as for the dense path: bit-exact
codes, steps and int32 accumulators; corrected dX / dW within 1e-5 of the
oracle relative to the largest magnitude; statistics within 1e-5.
"""
import numpy as np
import pytest
import torch

from oracle import backward, moe, quantize as oq
from stochastic_rounding_quantization_amd import inputs, s3r
from tests._gpu import DEV, assert_rows_close, host, rel_err, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _problem(counts, D, d_in, dtype, seed):
    m = inputs.MOE["moe-64x16384-top2-2048x1408-bf16"]
    rng = np.random.default_rng(seed)
    R, E = int(sum(counts)), len(counts)
    g = inputs.student_t(seed, (R, D), m.g_nu, m.g_scale)
    g[rng.integers(0, max(R, 1), 3)] *= 50.0 if R else 1.0
    x = inputs.gaussian(seed + 1, (R, d_in), 1.0)
    w = inputs.gaussian(seed + 2, (E, D, d_in), m.w_std)
    st = (lambda a: a) if dtype == "f32" else inputs.f32_to_bf16_bits
    return {"dtype": dtype, "offsets": np.concatenate([[0], np.cumsum(counts)]).astype(np.int64),
            "G": st(g), "X": st(x), "W": st(w)}


def gpu_grouped(inp, *, mode, ec, seed=0, layer_id=0, raw=False):
    dt = inp["dtype"]
    off = torch.from_numpy(inp["offsets"]).to(DEV)
    E = len(inp["offsets"]) - 1
    R, D = inp["G"].shape
    d_in = inp["X"].shape[1]
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    # forward operands: X per token with per-expert code column sums; the experts' W per output channel
    X = to_dev(inp["X"], dt)
    dx_desc = s3r.qdesc(R, d_in, 1, s3r.RTNE, s3r.EC_NONE, s3r.PER_TOKEN)
    Xq = s3r.q_buffer(R, d_in, DEV)
    sx = torch.empty(R, device=DEV)
    xs = torch.empty(E, d_in, dtype=torch.int32, device=DEV)
    ws = torch.zeros(max(s3r.s3r_grouped_workspace(dx_desc, E, d_in), 1), dtype=torch.uint8, device=DEV)
    s3r.s3r_grouped_quantize(dx_desc, off, X, None, None, Xq, sx, xs, flags=flags, ws=ws)
    W = to_dev(inp["W"].reshape(E * D, d_in), dt)
    ld = (d_in + 15) // 16 * 16
    wbuf = torch.empty(E * D, ld, dtype=torch.int8, device=DEV)
    wdesc = s3r.qdesc(E * D, d_in, D, s3r.RTNE, s3r.EC_NONE, s3r.PER_TOKEN)
    sw = torch.empty(E * D, device=DEV)
    rW = torch.empty(E, d_in, dtype=torch.int32, device=DEV)
    wws = torch.zeros(max(s3r.s3r_quantize_workspace(wdesc), 1), dtype=torch.uint8, device=DEV)
    s3r.s3r_quantize(wdesc, W, None, None, wbuf[:, :d_in], sw, rW, ws=wws)
    Wq3 = wbuf.view(E, D, ld)[:, :, :d_in]
    # gradient
    desc = s3r.qdesc(R, D, 1, mode, ec, s3r.PER_TENSOR, layer_id=layer_id, seed=seed)
    Q = s3r.q_buffer(R, D, DEV)
    delta = torch.empty(E, device=DEV)
    st = (torch.empty(R, device=DEV), torch.empty(E, D, device=DEV), torch.empty(E, device=DEV)) if ec \
        else (None, None, None)
    ws = torch.zeros(max(s3r.s3r_grouped_workspace(desc, E, d_in), 1), dtype=torch.uint8, device=DEV)
    s3r.s3r_grouped_quantize(desc, off, to_dev(inp["G"], dt), sx, sw.view(E, D), Q, delta, None, *st, flags, ws)
    odt = torch.int32 if raw else torch.float32
    dX = torch.full((R, d_in), -3, dtype=odt, device=DEV)
    dW = torch.full((E, D, d_in), -3, dtype=odt, device=DEV)
    s3r.s3r_grouped_backward_dx(desc, off, Q, delta, Wq3, sx, rW, *st, dX, flags, ws)
    s3r.s3r_grouped_backward_dw(desc, off, Q, delta, Xq, sw.view(E, D), xs, *st, dW, flags, ws)
    torch.cuda.synchronize()
    return dict(Xq=Xq, sx=sx, xs=xs, Wq=Wq3, sw=sw, rW=rW, Q=Q, delta=delta, st=st, dX=dX, dW=dW, flags=flags)


def _check(inp, gpu, ref, ec, experts=None, rows=None):
    off = inp["offsets"]
    E = len(off) - 1
    assert int(host(gpu["flags"])[0]) == 0
    np.testing.assert_array_equal(host(gpu["Xq"]), ref["fx"]["Q"])
    np.testing.assert_array_equal(host(gpu["sx"]), ref["fx"]["scale"])
    np.testing.assert_array_equal(host(gpu["xs"]), ref["xs"])
    Q, delta = host(gpu["Q"]), host(gpu["delta"])
    dX, dW = host(gpu["dX"]), host(gpu["dW"])
    for e in (range(E) if experts is None else experts):
        a, b = off[e], off[e + 1]
        np.testing.assert_array_equal(host(gpu["Wq"][e]), ref["fws"][e]["Q"])
        np.testing.assert_array_equal(Q[a:b], ref["Q"][e], err_msg=f"expert {e}")
        np.testing.assert_array_equal(delta[e:e + 1], ref["delta"][e], err_msg=f"expert {e}")
        if ec and b > a:
            assert rel_err(host(gpu["st"][0])[a:b], ref["eps"][e]) <= TOL
            assert rel_err(host(gpu["st"][1])[e:e + 1], ref["ebar"][e]) <= TOL
        r = np.arange(a, b) if rows is None else np.array([t for t in rows if a <= t < b], dtype=np.int64)
        if r.size:
            assert_rows_close(dX[r], ref["dX"][r], TOL, f"dX expert {e}")
        assert_rows_close(dW[e], ref["dW"][e], TOL, f"dW expert {e}")


@pytest.mark.parametrize("mode,ec", [(s3r.S3R, s3r.EC_TWO_WAY), (s3r.S3R, s3r.EC_DX_ONLY), (s3r.SR, s3r.EC_NONE),
                                     (s3r.RTNE, s3r.EC_NONE), (s3r.S3R, s3r.EC_DW_ONLY)])
def test_grouped_ragged_experts(mode, ec):
    # ragged expert sizes (empty, single-row, several 64- and 256-row tiles), ragged D and d_in
    counts = [5, 0, 300, 17, 1, 64, 129, 0, 513]
    inp = _problem(counts, 320, 200, "f32", 11)
    gpu = gpu_grouped(inp, mode=mode, ec=ec, seed=3, layer_id=1)
    ref = moe.grouped_backward(inp, mode=mode, ec=ec, seed=3, layer_id=1)
    _check(inp, gpu, ref, ec)


def test_grouped_raw_accumulators_bf16():
    counts = [200, 3, 0, 260, 77]
    inp = _problem(counts, 256, 136, "bf16", 5)
    gpu = gpu_grouped(inp, mode=s3r.S3R, ec=s3r.EC_NONE, seed=2, raw=True)
    ref = moe.grouped_backward(inp, mode=s3r.S3R, ec=s3r.EC_NONE, seed=2)
    off = inp["offsets"]
    Q = host(gpu["Q"])
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        np.testing.assert_array_equal(Q[a:b], ref["Q"][e])
        np.testing.assert_array_equal(host(gpu["dX"])[a:b], backward.int_matmul(ref["Q"][e], ref["fws"][e]["Q"]))
        np.testing.assert_array_equal(host(gpu["dW"][e]),
                                      backward.int_matmul(np.ascontiguousarray(ref["Q"][e].T), ref["fx"]["Q"][a:b]))


def test_grouped_invalid_offsets_flagged_and_nothing_written():
    R, D, d_in, E = 64, 96, 64, 3
    desc = s3r.qdesc(R, D, 1, s3r.S3R, s3r.EC_NONE)
    G = torch.randn(R, D, device=DEV) * 1e-3
    Q = torch.full((R, D), 9, dtype=torch.int8, device=DEV)
    delta = torch.full((E,), 5.0, device=DEV)
    ws = torch.zeros(s3r.s3r_grouped_workspace(desc, E, d_in), dtype=torch.uint8, device=DEV)
    for bad in ([0, 40, 20, 64], [0, 10, 20, 63], [1, 10, 20, 64], [0, 10, 10, 63]):
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        off = torch.tensor(bad, dtype=torch.int64, device=DEV)
        s3r.s3r_grouped_quantize(desc, off, G, None, None, Q, delta, flags=flags, ws=ws)
        dW = torch.full((E, D, d_in), 7.0, device=DEV)
        Xq = torch.zeros(R, d_in, dtype=torch.int8, device=DEV)
        s3r.s3r_grouped_backward_dw(desc, off, Q, delta, Xq, None, None, None, None, None, dW, flags, ws)
        torch.cuda.synchronize()
        assert int(host(flags)[0]) & s3r.FLAG_BAD_GROUPS, bad
        assert (host(Q) == 9).all() and (host(dW) == 7.0).all() and (host(delta) == 5.0).all()


def test_moe_workload_sampled():
    # the MoE workload: 64 experts, 32768 rows (Zipf sizes), d_model 2048, d_ff 1408, bf16, S3R-EC
    # two-way; the oracle checks the largest, the smallest and two other experts in full (codes, dW)
    # and sampled dX rows of them
    m = inputs.MOE["moe-64x16384-top2-2048x1408-bf16"]
    inp = inputs.make_moe_inputs(m)
    gpu = gpu_grouped(inp, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, seed=0, layer_id=0)
    counts = inp["counts"]
    experts = sorted({int(np.argmax(counts)), int(np.argmin(counts)), 7, 40})
    fx, fws, xs = moe.forward_operands(inp["X"], inp["W"], "bf16", inp["offsets"])
    ref = moe.grouped_backward(inp, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, fx=fx, fws=fws, xs=xs, experts=experts)
    rng = np.random.default_rng(0)
    rows = sorted(set(int(inp["offsets"][e] + rng.integers(0, counts[e])) for e in experts for _ in range(3)))
    _check(inp, gpu, ref, s3r.EC_TWO_WAY, experts=experts, rows=rows)
