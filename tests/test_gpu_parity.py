"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Bars: bit-exact INT8 codes, steps, code column sums and int32 accumulators;
dequantised / corrected dX and dW within 1e-5 of the oracle relative to the
largest oracle magnitude of the tensor; S3R-EC statistics (fp32 on the GPU,
fp64 in the oracle) within 1e-5 of their largest magnitude.
Small cases cover several tiles and ragged tails; the workload-size cases run
in the launch configuration bench.py times and compare sampled output rows.
"""
import numpy as np
import pytest
import torch

from oracle import backward, pipeline, quantize as oq
from stochastic_rounding_quantization_amd import inputs, s3r
from tests._gpu import DEV, assert_nan_equal, assert_rows_close, gpu_linear, host, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
MODES = [(s3r.RTNE, s3r.EC_NONE), (s3r.SR, s3r.EC_NONE), (s3r.S3R, s3r.EC_NONE),
         (s3r.S3R, s3r.EC_DX_ONLY), (s3r.S3R, s3r.EC_TWO_WAY)]


def _rand_i8(rng, shape):
    a = rng.integers(-127, 128, shape).astype(np.int8)
    if a.size:
        a.flat[0] = 127
        a.flat[-1] = -127
    return a


def _padded_i8(a: np.ndarray) -> torch.Tensor:
    r, c = a.shape
    buf = torch.zeros(r, (c + 15) // 16 * 16 + 16, dtype=torch.int8, device=DEV)
    v = buf[:, :c]
    v.copy_(torch.from_numpy(a))
    return v


# ------------------------------------------------------------- GEMMs ----

# K steps of 64: 1, 2, 3 (the rings' prologues), 4, 5, 6 (the dW ring's five stages), 12, 13, 25 (the dX
# ring's twelve-step schedule and its tail), 16, 65; ragged M, N and K.
@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (1, 17, 3), (64, 300, 128), (300, 64, 150), (300, 520, 200),
                                   (257, 128, 320), (128, 257, 384), (256, 256, 768), (130, 260, 832),
                                   (512, 768, 1024), (256, 512, 1600), (257, 255, 4100)])
def test_gemm_raw_accumulators_exact(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    # dX-shaped: Q [M x K] . Wq [K x N]
    Q = _rand_i8(rng, (M, K))
    Wq = _rand_i8(rng, (K, N))
    d = s3r.qdesc(M, K, M, s3r.S3R, s3r.EC_NONE)
    delta = torch.ones(1, device=DEV)
    out = torch.full((M, N), -7, dtype=torch.int32, device=DEV)
    s3r.s3r_backward_dx(d, _padded_i8(Q), delta, _padded_i8(Wq), None, None, None, None, None, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), backward.int_matmul(Q, Wq))
    # dW-shaped: Q^T with Q [K x M] . Xq [K x N]
    Qt = _rand_i8(rng, (K, M))
    Xq = _rand_i8(rng, (K, N))
    d = s3r.qdesc(K, M, K, s3r.S3R, s3r.EC_NONE)
    out = torch.full((M, N), -7, dtype=torch.int32, device=DEV)
    s3r.s3r_backward_dw(d, _padded_i8(Qt), delta, _padded_i8(Xq), None, None, None, None, None, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), backward.int_matmul(np.ascontiguousarray(Qt.T), Xq))


def test_gemm_output_leading_dim_and_extremes():
    # all +-127 operands at the int32 bound region, output written with a padded leading dim
    M, N, K = 96, 80, 4096
    Q = np.full((M, K), 127, np.int8)
    Q[1::2] = -127
    Wq = np.full((K, N), -127, np.int8)
    d = s3r.qdesc(M, K, M)
    buf = torch.full((M, N + 13), 5, dtype=torch.int32, device=DEV)
    s3r.s3r_backward_dx(d, _padded_i8(Q), torch.ones(1, device=DEV), _padded_i8(Wq), None, None, None, None, None,
                        buf[:, :N])
    torch.cuda.synchronize()
    got = host(buf)
    np.testing.assert_array_equal(got[:, :N], backward.int_matmul(Q, Wq))
    assert (got[:, N:] == 5).all()


# --------------------------------------------------------- quantizer ----

QCASES = [  # (T, D, S, dtype)
    (256, 1024, 256, "f32"),
    (64, 100, 32, "bf16"),     # D % 8 != 0: partial last chunk
    (33, 77, 33, "f32"),       # D % 4 != 0: SR per-element Philox path
    (1, 1, 1, "bf16"),
    (192, 600, 64, "bf16"),    # three examples, two column tiles
]


def _grad(T, D, dtype, seed):
    g = inputs.student_t(seed, (T, D), 3.0, 1e-3)
    rng = np.random.default_rng(seed)
    if T > 4:
        g[rng.choice(T, max(1, T // 50), replace=False)] *= 100
    sx = rng.uniform(0.01, 0.05, T).astype(np.float32)
    sw = rng.uniform(1e-4, 5e-4, D).astype(np.float32)
    store = inputs.f32_to_bf16_bits(g) if dtype == "bf16" else g
    return store, sx, sw


@pytest.mark.parametrize("T,D,S,dtype", QCASES)
@pytest.mark.parametrize("scale", [s3r.PER_TENSOR, s3r.PER_TOKEN])
def test_quantize_bit_exact(T, D, S, dtype, scale):
    store, sx, sw = _grad(T, D, dtype, T * 131 + D)
    G = to_dev(store, dtype)
    for mode, ec in MODES:
        seed, layer = 12345 + mode, 3
        q = s3r.quantize(G, mode=mode, ec=ec, scale=scale, row_scale=torch.from_numpy(sx).to(DEV),
                         col_scale=torch.from_numpy(sw).to(DEV), seed=seed, layer_id=layer, rows_per_example=S,
                         colsum=True)
        torch.cuda.synchronize()
        ref = oq.quantize(store, dtype, mode=mode, scale=scale, row_scale=sx, col_scale=sw, seed=seed,
                          layer_id=layer, rows_per_example=S)
        tag = f"T={T} D={D} {dtype} mode={mode} ec={ec} scale={scale}"
        np.testing.assert_array_equal(host(q.Q), ref["Q"], err_msg=tag)
        np.testing.assert_array_equal(host(q.delta), ref["delta"], err_msg=tag)
        np.testing.assert_array_equal(host(q.code_colsum), ref["code_colsum"], err_msg=tag)
        assert int(host(q.flags)[0]) == ref["flags"], tag
        if ec != s3r.EC_NONE:
            from oracle import ec as oec
            E = oec.rounding_error(ref["Q"], ref["x"], ref["delta"])
            eps, ebar, mu = oec.statistics(E, S)
            assert rel_err(host(q.ec_row), eps) <= TOL, tag
            assert rel_err(host(q.ec_col), ebar) <= TOL, tag
            assert np.abs(host(q.ec_mean) - mu).max() <= TOL * np.abs(E).max(), tag


# Per-tensor bf16 shapes: the benchmark's down projection; 1000-row and 96-row tensors whose rows do
# not fill the 64-row tiles evenly; a ragged T = 4097 with one 4097-token example; a 300-row tensor.
RCASES = [(8192, 4096, 2048), (1000, 8192, 1000), (96, 1024, 32), (4097, 2048, 4097), (300, 512, 300)]


@pytest.mark.parametrize("T,D,S", RCASES)
def test_quantize_bf16_per_tensor_matches_oracle(T, D, S):
    store, sx, sw = _grad(T, D, "bf16", T * 7 + D)
    if T == 96:
        store[5, 7] = 0x7FC0          # a NaN: flags, zero codes, NaN step
    G = to_dev(store, "bf16")
    sx_d, sw_d = torch.from_numpy(sx).to(DEV), torch.from_numpy(sw).to(DEV)
    for mode, ec in MODES:
        ref = oq.quantize(store, "bf16", mode=mode, scale=s3r.PER_TENSOR, row_scale=sx, col_scale=sw, seed=77,
                          layer_id=5, rows_per_example=S)
        q = s3r.quantize(G, mode=mode, ec=ec, row_scale=sx_d, col_scale=sw_d, seed=77, layer_id=5,
                         rows_per_example=S)
        torch.cuda.synchronize()
        tag = f"T={T} D={D} S={S} mode={mode} ec={ec}"
        np.testing.assert_array_equal(host(q.Q), ref["Q"], err_msg=tag)
        assert_nan_equal(host(q.delta), ref["delta"], tag)
        assert int(host(q.flags)[0]) == ref["flags"], tag
        if ec != s3r.EC_NONE and not ref["flags"]:
            from oracle import ec as oec
            E = oec.rounding_error(ref["Q"], ref["x"], ref["delta"])
            eps, ebar, mu = oec.statistics(E, S)
            assert rel_err(host(q.ec_row), eps) <= TOL, tag
            assert rel_err(host(q.ec_col), ebar) <= TOL, tag
            assert np.abs(host(q.ec_mean) - mu).max() <= TOL * np.abs(E).max(), tag


def test_quantize_zero_tensor():
    G = torch.zeros(64, 512, dtype=torch.bfloat16, device=DEV)
    q = s3r.quantize(G, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, rows_per_example=64)
    torch.cuda.synchronize()
    assert (host(q.Q) == 0).all() and host(q.delta)[0] == 1.0 and int(host(q.flags)[0]) == 0
    assert (host(q.ec_row) == 0).all() and (host(q.ec_col) == 0).all() and (host(q.ec_mean) == 0).all()


def test_quantize_strided_and_unaligned():
    # G with a padded leading dim, Q written into a padded buffer; then the scalar path (odd ld).
    T, D = 40, 72
    store, sx, sw = _grad(T, D, "f32", 5)
    ref = oq.quantize(store, "f32", mode=s3r.S3R, seed=9, rows_per_example=T)
    for pad in (8, 3):
        Gbuf = torch.zeros(T, D + pad, dtype=torch.float32, device=DEV)
        Gbuf[:, :D] = torch.from_numpy(store)
        Qbuf = torch.full((T, D + pad + 1), 99, dtype=torch.int8, device=DEV)
        d = s3r.qdesc(T, D, T, s3r.S3R, s3r.EC_NONE, seed=9)
        delta = torch.empty(1, device=DEV)
        ws = torch.zeros(max(s3r.s3r_quantize_workspace(d), 1), dtype=torch.uint8, device=DEV)
        s3r.s3r_quantize(d, Gbuf[:, :D], None, None, Qbuf[:, :D], delta, ws=ws)
        torch.cuda.synchronize()
        got = host(Qbuf)
        np.testing.assert_array_equal(got[:, :D], ref["Q"])
        assert (got[:, D:] == 99).all()


def test_quantize_degenerate_inputs():
    dev = DEV
    # empty tensors
    for T, D in ((0, 16), (16, 0)):
        G = torch.zeros(T, D, device=dev)
        q = s3r.quantize(G, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, rows_per_example=max(T, 1), colsum=True)
        torch.cuda.synchronize()
        assert host(q.delta)[0] == 1.0
        if T:
            assert not host(q.ec_row).any()
    # all-zero, NaN, Inf, tiny amax: flags and zero codes, as the oracle
    base = inputs.student_t(3, (24, 40), 3.0, 1e-3)
    cases = {"zero": np.zeros((24, 40), np.float32), "nan": base.copy(), "inf": base.copy(),
             "tiny": np.full((24, 40), 1e-38, np.float32)}
    cases["nan"][3, 5] = np.nan
    cases["inf"][7, 1] = -np.inf
    for name, g in cases.items():
        for scale in (s3r.PER_TENSOR, s3r.PER_TOKEN):
            for mode in (s3r.RTNE, s3r.SR, s3r.S3R):
                q = s3r.quantize(to_dev(g, "f32"), mode=mode, scale=scale, seed=1, rows_per_example=24)
                torch.cuda.synchronize()
                ref = oq.quantize(g, "f32", mode=mode, scale=scale, seed=1, rows_per_example=24)
                tag = f"{name} scale={scale} mode={mode}"
                np.testing.assert_array_equal(host(q.Q), ref["Q"], err_msg=tag)
                assert_nan_equal(host(q.delta), ref["delta"], tag)
                assert int(host(q.flags)[0]) == ref["flags"], tag


def test_deterministic():
    store, sx, sw = _grad(512, 1024, "bf16", 77)
    G = to_dev(store, "bf16")
    outs = []
    for _ in range(2):
        q = s3r.quantize(G, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, rows_per_example=128, seed=4)
        W = _padded_i8(_rand_i8(np.random.default_rng(1), (1024, 384)))
        dX = s3r.backward_dx(q, W, r_W=torch.zeros(384, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        outs.append([host(q.Q), host(q.ec_row), host(q.ec_col), host(q.ec_mean), host(dX)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a.view(np.uint8) if a.dtype == np.int8 else a.view(np.uint32),
                                      b.view(np.uint8) if b.dtype == np.int8 else b.view(np.uint32))


# -------------------------------------------------------- end to end ----

def _check_linear(inp, S, mode, ec, scale=s3r.PER_TENSOR, dx_rows=None, dw_rows=None, seed=0, layer=0):
    gpu = gpu_linear(inp, mode=mode, ec=ec, scale=scale, seed=seed, layer_id=layer, rows_per_example=S)
    tag = f"mode={mode} ec={ec} scale={scale}"
    fx, fw = pipeline.forward_operands(inp["X"], inp["W"], inp["dtype"], S)
    # forward-operand prep (a0): codes, row steps, column sums bit-exact
    np.testing.assert_array_equal(host(gpu["fx"].Q), fx["Q"])
    np.testing.assert_array_equal(host(gpu["fx"].delta), fx["scale"])
    np.testing.assert_array_equal(host(gpu["fx"].code_colsum), fx["code_colsum"])
    np.testing.assert_array_equal(host(gpu["fw"].Q), fw["Q"])
    np.testing.assert_array_equal(host(gpu["fw"].delta), fw["scale"])
    np.testing.assert_array_equal(host(gpu["fw"].code_colsum), fw["code_colsum"])
    ref = pipeline.linear_backward(inp, mode=mode, ec=ec, scale=scale, seed=seed, layer_id=layer,
                                   rows_per_example=S, dx_rows=dx_rows, dw_rows=dw_rows, fx=fx, fw=fw)
    q = gpu["q"]
    np.testing.assert_array_equal(host(q.Q), ref["q"]["Q"], err_msg=tag)
    np.testing.assert_array_equal(host(q.delta), ref["q"]["delta"], err_msg=tag)
    if ec != s3r.EC_NONE:
        assert rel_err(host(q.ec_row), ref["q"]["eps"]) <= TOL, tag
        assert rel_err(host(q.ec_col), ref["q"]["ebar"]) <= TOL, tag
    dX = host(gpu["dX"])
    dX = dX if dx_rows is None else dX[dx_rows]
    assert_rows_close(dX, ref["dX"], TOL, f"{tag} dX {dX.shape}")
    dW = host(gpu["dW"])
    dW = dW if dw_rows is None else dW[dw_rows]
    assert_rows_close(dW, ref["dW"], TOL, f"{tag} dW {dW.shape}")
    return gpu, ref


@pytest.mark.parametrize("mode,ec", MODES)
def test_linear_256x512x1024_f32(mode, ec):
    w = inputs.WORKLOADS["linear-256x512x1024-f32"]
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, w.rows_per_example, mode, ec)


def test_linear_ragged_multi_example_bf16():
    # three examples of 128 tokens, ragged D and d_in, both EC variants and per-token steps for dX
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(384, 300, 700, rows_per_example=128)
    inp = inputs.make_linear_inputs(w)
    for mode, ec in ((s3r.S3R, s3r.EC_TWO_WAY), (s3r.S3R, s3r.EC_DX_ONLY), (s3r.SR, s3r.EC_NONE)):
        _check_linear(inp, 128, mode, ec, seed=7, layer=2)
    _check_linear(inp, 128, s3r.S3R, s3r.EC_TWO_WAY, scale=s3r.PER_TOKEN, seed=7, layer=2)


@pytest.mark.parametrize("B", [2, 5, 8, 11])
def test_linear_example_counts(B):
    # B examples of 40 tokens: GEMM tiles span several examples; the dW epilogue's compile-time
    # example slots (1, 2, 4, 8) and, past 8 examples, the rank-update kernel
    w = inputs.WORKLOADS["down-8192x14336x4096-bf16"].scaled(40 * B, 330, 200, rows_per_example=40)
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, 40, s3r.S3R, s3r.EC_TWO_WAY, seed=B, layer=1)


def _sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, min(n, k), replace=False).tolist()) | {0, n - 1, n - 2}
    return np.array(sorted(rows))


@pytest.mark.parametrize("mode,ec", [(s3r.S3R, s3r.EC_TWO_WAY), (s3r.SR, s3r.EC_NONE), (s3r.RTNE, s3r.EC_NONE),
                                     (s3r.S3R, s3r.EC_DX_ONLY)])
def test_down_4096x11008x4096_bf16_sampled(mode, ec):
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"]
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, w.rows_per_example, mode, ec, dx_rows=_sample_rows(w.tokens, 20, 1),
                  dw_rows=_sample_rows(w.d_out, 12, 2))


def test_down_8192x14336x4096_bf16_sampled():
    # the bench workload: Llama-8B FFN down-projection, four examples of 2048 tokens, S3R-EC two-way
    w = inputs.WORKLOADS["down-8192x14336x4096-bf16"]
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, w.rows_per_example, s3r.S3R, s3r.EC_TWO_WAY, dx_rows=_sample_rows(w.tokens, 16, 3),
                  dw_rows=_sample_rows(w.d_out, 10, 4))


def test_dx_accumulate_two_projections():
    # dX of two projections of the same input (the SwiGLU block's gate and up) added into one
    # output with S3R_F32_ACC: equals the sum of the two oracle products
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(192, 136, 300, rows_per_example=64)
    a = inputs.make_linear_inputs(w)
    raw = inputs.make_linear_inputs(inputs.WORKLOADS["linear-256x512x1024-f32"].scaled(192, 136, 300, 64))
    b = {"G": inputs.f32_to_bf16_bits(raw["G"]), "X": a["X"], "W": inputs.f32_to_bf16_bits(raw["W"]), "dtype": "bf16"}
    S = 64
    fx = s3r.forward_operand(to_dev(a["X"], "bf16"), rows_per_example=S)
    dX = None
    refs = []
    for layer, inp in ((1, a), (2, b)):
        fw = s3r.forward_operand(to_dev(inp["W"], "bf16"), rows_per_example=inp["W"].shape[0])
        q = s3r.quantize(to_dev(inp["G"], "bf16"), mode=s3r.S3R, ec=s3r.EC_TWO_WAY, row_scale=fx.delta,
                         col_scale=fw.delta, seed=3, layer_id=layer, rows_per_example=S)
        dX = s3r.backward_dx(q, fw.Q, s_x=fx.delta, r_W=fw.code_colsum[0], out=dX)
        refs.append(pipeline.linear_backward(inp, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, seed=3, layer_id=layer,
                                             rows_per_example=S)["dX"])
    torch.cuda.synchronize()
    assert_rows_close(host(dX), refs[0] + refs[1], TOL, "accumulated dX")


@pytest.mark.parametrize("D", [136, 144, 200, 256, 264, 520])
def test_ec_statistics_partial_column_tiles(D):
    # D not a multiple of the quantizer's 512-column tiles: a wave of the last column tile holds both
    # full 8-column chunks and chunks past D; the per-token error sums eps_t, their means and both
    # corrected products still match the oracle
    T, d_in, S = 192, 300, 64
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, d_in, D, rows_per_example=S)
    inp = inputs.make_linear_inputs(w)
    gpu, ref = _check_linear(inp, S, s3r.S3R, s3r.EC_TWO_WAY, seed=5, layer=1)
    assert rel_err(host(gpu["q"].ec_mean), ref["q"]["mu"]) <= TOL


def _two_projections(T, D, d_in, S):
    # two projections of one input X (a SwiGLU block's gate and up): own G and W, shared X
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, d_in, D, rows_per_example=S)
    a = inputs.make_linear_inputs(w)
    raw = inputs.make_linear_inputs(inputs.WORKLOADS["linear-256x512x1024-f32"].scaled(T, d_in, D, S))
    b = {"G": inputs.f32_to_bf16_bits(raw["G"]), "X": a["X"], "W": inputs.f32_to_bf16_bits(raw["W"]), "dtype": "bf16"}
    return a, b


@pytest.mark.parametrize("T,D,d_in,S,mode,ec,raw", [
    (384, 300, 700, 128, s3r.S3R, s3r.EC_TWO_WAY, False),      # ragged, three examples
    (440, 330, 200, 40, s3r.S3R, s3r.EC_TWO_WAY, False),       # eleven examples: the rank-update pass
    (192, 136, 300, 64, s3r.S3R, s3r.EC_DW_ONLY, False),
    (256, 512, 1024, 256, s3r.SR, s3r.EC_NONE, False),
    (256, 520, 264, 128, s3r.S3R, s3r.EC_TWO_WAY, True),       # raw int32 accumulators
])
def test_dw_pair_equals_two_single_calls(T, D, d_in, S, mode, ec, raw):
    # s3r_backward_dw_pair gives each product bit for bit as s3r_backward_dw does, and both match the oracle
    a, b = _two_projections(T, D, d_in, S)
    fx = s3r.forward_operand(to_dev(a["X"], "bf16"), rows_per_example=S)
    qs, fws, refs = [], [], []
    for layer, inp in ((1, a), (2, b)):
        fw = s3r.forward_operand(to_dev(inp["W"], "bf16"), rows_per_example=inp["W"].shape[0])
        qs.append(s3r.quantize(to_dev(inp["G"], "bf16"), mode=mode, ec=ec, row_scale=fx.delta, col_scale=fw.delta,
                               seed=5, layer_id=layer, rows_per_example=S))
        fws.append(fw)
        if not raw:
            refs.append(pipeline.linear_backward(inp, mode=mode, ec=ec, seed=5, layer_id=layer,
                                                 rows_per_example=S)["dW"])
    odt = torch.int32 if raw else None
    single = [s3r.backward_dw(q, fx.Q, s_w=fw.delta, xs_b=fx.code_colsum, out_dtype=odt) for q, fw in zip(qs, fws)]
    pair = s3r.backward_dw_pair(qs[0], qs[1], fx.Q, fws[0].delta, fws[1].delta, fx.code_colsum, out_dtype=odt)
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(pair[k], single[k]), f"product {k}: the paired launch differs from the single call"
        if not raw:
            assert_rows_close(host(pair[k]), refs[k], TOL, f"paired dW {k} T={T} D={D} d_in={d_in}")


def test_dw_pair_ffn_block_size():
    # the FFN block's gate and up dW at full size (two 14336 x 4096 outputs, K = 8192): bit for bit the
    # single calls', sampled rows against the oracle
    T, M, F, S = 8192, 4096, 14336, 2048
    a, b = _two_projections(T, F, M, S)
    fx = s3r.forward_operand(to_dev(a["X"], "bf16"), rows_per_example=S)
    qs, fws = [], []
    for layer, inp in ((1, a), (2, b)):
        fw = s3r.forward_operand(to_dev(inp["W"], "bf16"), rows_per_example=inp["W"].shape[0])
        qs.append(s3r.quantize(to_dev(inp["G"], "bf16"), mode=s3r.S3R, ec=s3r.EC_TWO_WAY, row_scale=fx.delta,
                               col_scale=fw.delta, seed=9, layer_id=layer, rows_per_example=S))
        fws.append(fw)
    pair = s3r.backward_dw_pair(qs[0], qs[1], fx.Q, fws[0].delta, fws[1].delta, fx.code_colsum)
    for k in range(2):
        single = s3r.backward_dw(qs[k], fx.Q, s_w=fws[k].delta, xs_b=fx.code_colsum)
        torch.cuda.synchronize()
        assert torch.equal(pair[k], single), f"product {k}: the paired launch differs from the single call"
        del single
    rows = _sample_rows(F, 4, 11)
    ref = pipeline.linear_backward(a, mode=s3r.S3R, ec=s3r.EC_TWO_WAY, seed=9, layer_id=1, rows_per_example=S,
                                   dx_rows=np.array([0]), dw_rows=rows)["dW"]
    assert_rows_close(host(pair[0])[rows], ref, TOL, "paired dW gate, FFN block size")


def test_gate_projection_ffn_block_size_sampled():
    # the FFN block's gate / up projection shape: G [8192 x 14336] (two-pass quantizer, 224 MiB of
    # bf16), W [14336 x 4096], X [8192 x 4096]; S3R-EC two-way, rows sampled
    w = inputs.WORKLOADS["down-8192x14336x4096-bf16"].scaled(8192, 4096, 14336, rows_per_example=2048)
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, 2048, s3r.S3R, s3r.EC_TWO_WAY, dx_rows=_sample_rows(w.tokens, 6, 5),
                  dw_rows=_sample_rows(w.d_out, 6, 6), layer=1)


# --------------------------------------------- per-token steps and dW ----

@pytest.mark.parametrize("T,D,d_in,S", [(300, 200, 77, 100), (512, 96, 1100, 256), (40, 33, 8, 40)])
def test_per_token_dw_requantized_inputs(T, D, d_in, S):
    # dW with one step per token: the inputs Xq are folded with the steps and requantized per
    # column (ragged against the 256-row bands and the 8-column lanes); the raw accumulators
    # Q^T Zq are bit-exact and the dequantized, corrected dW is within the tolerance
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, d_in, D, rows_per_example=S)
    inp = inputs.make_linear_inputs(w)
    for ec in (s3r.EC_NONE, s3r.EC_TWO_WAY):
        gpu, ref = _check_linear(inp, S, s3r.S3R, ec, scale=s3r.PER_TOKEN, seed=T, layer=3)
        q = gpu["q"]
        raw = torch.full((D, d_in), -7, dtype=torch.int32, device=DEV)
        ws = torch.zeros(max(s3r.s3r_backward_workspace(q.desc, d_in), 1), dtype=torch.uint8, device=DEV)
        s3r.s3r_backward_dw(q.desc, q.Q, q.delta, gpu["fx"].Q, None, None, None, None, None, raw, ws)
        torch.cuda.synchronize()
        Zq, _ = backward.requantize_columns(ref["fx"]["Q"], ref["q"]["delta"])
        np.testing.assert_array_equal(host(raw), backward.int_matmul(np.ascontiguousarray(ref["q"]["Q"].T), Zq))


def test_per_token_dw_flagged_token_poisons_steps():
    # a non-finite gradient row gives that token a non-finite step: every column step of Z is then
    # NaN and the codes are 0, so dW is NaN throughout, as in the oracle
    T, D, d_in = 64, 48, 40
    rng = np.random.default_rng(3)
    G = (1e-3 * rng.standard_normal((T, D))).astype(np.float32)
    G[5, 7] = np.inf
    Xq = _rand_i8(rng, (T, d_in))
    q = s3r.quantize(to_dev(G, "f32"), mode=s3r.S3R, scale=s3r.PER_TOKEN, seed=2, rows_per_example=T)
    dW = s3r.backward_dw(q, _padded_i8(Xq))
    torch.cuda.synchronize()
    ref = oq.quantize(G, "f32", mode=s3r.S3R, scale=s3r.PER_TOKEN, seed=2, rows_per_example=T)
    np.testing.assert_array_equal(host(q.delta).view(np.uint32), ref["delta"].view(np.uint32))
    exp = backward.backward_dw_per_token(ref["Q"], ref["delta"], Xq, np.ones(D, np.float32))
    assert np.isnan(exp).all() and np.isnan(host(dW)).all()


def test_down_8192x14336x4096_bf16_per_token_sampled():
    # the headline shape with per-token steps for both products (two-way correction), rows sampled
    w = inputs.WORKLOADS["down-8192x14336x4096-bf16"]
    inp = inputs.make_linear_inputs(w)
    _check_linear(inp, w.rows_per_example, s3r.S3R, s3r.EC_TWO_WAY, scale=s3r.PER_TOKEN,
                  dx_rows=_sample_rows(w.tokens, 8, 7), dw_rows=_sample_rows(w.d_out, 8, 8))


# ------------------------------------------------ quantize with a known amax ----

@pytest.mark.parametrize("mode,ec", [(s3r.S3R, s3r.EC_TWO_WAY), (s3r.SR, s3r.EC_NONE), (s3r.RTNE, s3r.EC_NONE)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_with_amax_equals_quantize(mode, ec, dtype):
    # with the amax supplied (here the oracle's), one pass over G gives the oracle's codes, step and
    # statistics
    T, D, S = 1024, 2048, 256
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, 64, D, rows_per_example=S)
    inp = inputs.make_linear_inputs(w)
    g = inp["G"] if dtype == "bf16" else oq.decode(inp["G"], "bf16")
    rng = np.random.default_rng(1)
    sx = rng.uniform(0.01, 0.05, T).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, D).astype(np.float32)
    ref = pipeline.quantize_gradient(g, dtype, {"scale": sx}, {"scale": sw}, mode=mode, scale=oq.PER_TENSOR,
                                     seed=5, layer_id=2, rows_per_example=S)
    a = np.abs(oq.fold(oq.decode(g, dtype), sx, sw)).max()
    amax = torch.from_numpy(np.array([a], np.float32).view(np.int32)).to(DEV)
    d = s3r.qdesc(T, D, S, mode, ec, layer_id=2, seed=5)
    Q = s3r.q_buffer(T, D, DEV)
    delta = torch.empty(1, device=DEV)
    st = (torch.empty(T, device=DEV), torch.empty(T // S, D, device=DEV), torch.empty(T // S, device=DEV)) if ec \
        else (None, None, None)
    ws = torch.zeros(s3r.s3r_quantize_workspace(d), dtype=torch.uint8, device=DEV)
    s3r.s3r_quantize_with_amax(d, to_dev(g, dtype), torch.from_numpy(sx).to(DEV), torch.from_numpy(sw).to(DEV), amax,
                               Q, delta, *st, None, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Q), ref["Q"])
    np.testing.assert_array_equal(host(delta), ref["delta"])
    if ec:
        assert rel_err(host(st[0]), ref["eps"]) <= TOL
        assert rel_err(host(st[1]), ref["ebar"]) <= TOL
        assert np.abs(host(st[2]) - ref["mu"]).max() <= TOL * np.abs(ref["eps"]).max()


# --------------------------------------------------- ablation configurations ----

@pytest.mark.parametrize("mode,ec", [(s3r.S3R_BCAST, s3r.EC_NONE), (s3r.S3R_BCAST, s3r.EC_TWO_WAY),
                                     (s3r.S3R_BCAST, s3r.EC_DX_ONLY), (s3r.S3R, s3r.EC_DW_ONLY),
                                     (s3r.S3R_BCAST, s3r.EC_DW_ONLY)])
def test_ablation_configurations(mode, ec):
    # Phi_bcast (one threshold per example) and the dW-only correction: codes bit-exact, dX / dW
    # within the tolerance; three examples with ragged shapes, and a power-of-two D
    for (T, d_in, D, S) in ((384, 300, 700, 128), (1024, 96, 512, 256)):
        w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, d_in, D, rows_per_example=S)
        inp = inputs.make_linear_inputs(w)
        _check_linear(inp, S, mode, ec, seed=D, layer=4)


@pytest.mark.parametrize("mode", [s3r.SR, s3r.S3R, s3r.S3R_BCAST])
def test_second_threshold_stream(mode):
    # quantizing G a second time with threshold stream 1 (the conventional configuration's
    # independent R^RHS) gives the oracle's stream-1 codes, different from stream 0's
    T, D, S = 512, 1100, 128
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, 64, D, rows_per_example=S)
    inp = inputs.make_linear_inputs(w)
    G = to_dev(inp["G"], "bf16")
    codes = []
    for stream in (0, 1):
        q = s3r.quantize(G, mode=mode, seed=3, layer_id=2, rows_per_example=S, threshold_stream=stream)
        torch.cuda.synchronize()
        ref = oq.quantize(inp["G"], "bf16", mode=mode, seed=3, layer_id=2, rows_per_example=S, stream=stream)
        np.testing.assert_array_equal(host(q.Q), ref["Q"])
        codes.append(ref["Q"])
    assert (codes[0] != codes[1]).any()


def test_quantize_twice_backward_equals_oracle():
    # Table II's causal ablation: dX from Phi_bcast codes (stream 0), dW from Phi_2D codes (stream 1)
    T, d_in, D, S = 256, 200, 320, 64
    w = inputs.WORKLOADS["down-4096x11008x4096-bf16"].scaled(T, d_in, D, rows_per_example=S)
    inp = inputs.make_linear_inputs(w)
    G, X, W = (to_dev(inp[k], "bf16") for k in ("G", "X", "W"))
    fx = s3r.forward_operand(X, rows_per_example=S)
    fw = s3r.forward_operand(W, rows_per_example=D)
    qx = s3r.quantize(G, mode=s3r.S3R_BCAST, row_scale=fx.delta, col_scale=fw.delta, seed=1, rows_per_example=S)
    qw = s3r.quantize(G, mode=s3r.S3R, row_scale=fx.delta, col_scale=fw.delta, seed=1, rows_per_example=S,
                      threshold_stream=1)
    dX = s3r.backward_dx(qx, fw.Q, s_x=fx.delta)
    dW = s3r.backward_dw(qw, fx.Q, s_w=fw.delta)
    torch.cuda.synchronize()
    ref = pipeline.linear_backward_twice(inp, mode_dx=s3r.S3R_BCAST, mode_dw=s3r.S3R, seed=1, rows_per_example=S)
    np.testing.assert_array_equal(host(qx.Q), ref["q_dx"]["Q"])
    np.testing.assert_array_equal(host(qw.Q), ref["q_dw"]["Q"])
    assert_rows_close(host(dX), ref["dX"], TOL, "quantize twice dX")
    assert_rows_close(host(dW), ref["dW"], TOL, "quantize twice dW")
