"""Parity of the SwiGLU backward glue (s3r_swiglu_backward) with the oracle: bit-exact bf16.

The glue's arithmetic is fixed (fp32, fixed order, the library's exp), so the
GPU and the oracle give the same bf16 bits for every element, including
ragged rows, strided layouts and extreme or non-finite inputs.
"""
import numpy as np
import pytest
import torch

from oracle import swiglu as sg
from stochastic_rounding_quantization_amd import inputs, s3r
from tests._gpu import DEV, host

pytestmark = pytest.mark.gpu


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def _draw(T, F, seed):
    dH = inputs.student_t(seed, (T, F), 3.0, 1e-4)
    ag = inputs.f32_to_bf16_bits(inputs.gaussian(seed + 1, (T, F), 2.0))
    au = inputs.f32_to_bf16_bits(inputs.gaussian(seed + 2, (T, F), 1.0))
    return dH, ag, au


@pytest.mark.parametrize("T,F", [(64, 1024), (33, 77), (1, 8), (5, 3000)])
def test_glue_bit_exact(T, F):
    dH, ag, au = _draw(T, F, T * 31 + F)
    gg, gu = s3r.swiglu_backward(torch.from_numpy(dH).to(DEV), _bf16_dev(ag), _bf16_dev(au))
    torch.cuda.synchronize()
    ref_g, ref_u = sg.glue(dH, ag, au)
    np.testing.assert_array_equal(_bits(gg), ref_g)
    np.testing.assert_array_equal(_bits(gu), ref_u)


def test_glue_extremes_and_strides():
    vals_a = np.float32([0.0, -0.0, 1e-39, -1e-39, 1.0, -1.0, 50.0, -50.0, 88.0, -88.0, 103.0, -103.0,
                         200.0, -200.0, 3e38, -3e38, np.inf, -np.inf, np.nan, 0.5])
    vals_h = np.float32([0.0, -0.0, 1e-38, 1.0, -1.0, 1e30, -1e30, 3e38, np.inf, np.nan])
    T, F = len(vals_h), len(vals_a)
    dH = np.tile(vals_h[:, None], (1, F)).astype(np.float32)
    a = np.tile(vals_a[None, :], (T, 1))
    ag = inputs.f32_to_bf16_bits(a)
    au = inputs.f32_to_bf16_bits(np.roll(a, 3, axis=1))
    ref_g, ref_u = sg.glue(dH, ag, au)
    for pad_h, pad_a in ((0, 0), (3, 5), (4, 8)):       # unaligned and aligned strides
        dHb = torch.zeros(T, F + pad_h, device=DEV)
        dHb[:, :F] = torch.from_numpy(dH)
        Ab = torch.zeros(2, T, F + pad_a, dtype=torch.bfloat16, device=DEV)
        Ab[0, :, :F] = _bf16_dev(ag)
        Ab[1, :, :F] = _bf16_dev(au)
        Gb = torch.full((2, T, F + pad_a), 7.0, dtype=torch.bfloat16, device=DEV)
        s3r.s3r_swiglu_backward(dHb[:, :F], Ab[0, :, :F], Ab[1, :, :F], Gb[0, :, :F], Gb[1, :, :F])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(Gb[0, :, :F]), ref_g)
        np.testing.assert_array_equal(_bits(Gb[1, :, :F]), ref_u)
        assert (host(Gb[:, :, F:].float()) == 7.0).all()


def test_glue_empty():
    z = torch.empty(0, 16, device=DEV)
    zb = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    s3r.s3r_swiglu_backward(z, zb, zb, zb.clone(), zb.clone())
    torch.cuda.synchronize()


def test_glue_ffn_block_size_sampled():
    # the FFN block's glue: 8192 tokens x d_ff 14336, rows sampled for the oracle
    T, F = 8192, 14336
    dH, ag, au = _draw(T, F, 77)
    gg, gu = s3r.swiglu_backward(torch.from_numpy(dH).to(DEV), _bf16_dev(ag), _bf16_dev(au))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 5000, 8190, 8191])
    ref_g, ref_u = sg.glue(dH[rows], ag[rows], au[rows])
    np.testing.assert_array_equal(_bits(gg)[rows], ref_g)
    np.testing.assert_array_equal(_bits(gu)[rows], ref_u)


# ------------------------------------------------------ glue + amax ----

def _amax_bits(g_bits, sx, sw):
    """The oracle quantizer's per-tensor amax of fold(G) as fp32 bits (NaN -> any NaN pattern)."""
    from oracle import quantize as oq
    x = oq.fold(oq.decode(g_bits, "bf16"), sx, sw)
    a = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    return int(np.array([a], np.float32).view(np.uint32)[0])


def _check_amax(got, exp):
    if exp > 0x7F800000:
        assert got > 0x7F800000, (hex(got), hex(exp))
    else:
        assert got == exp, (hex(got), hex(exp))


def _glue_amax(dH, ag, au, sx, swg, swu):
    T, F = dH.shape
    gg = torch.empty(T, F, dtype=torch.bfloat16, device=DEV)
    gu = torch.empty_like(gg)
    amax = torch.full((2,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    ws = torch.zeros(s3r.s3r_swiglu_amax_workspace(T, F), dtype=torch.uint8, device=DEV)
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    s3r.s3r_swiglu_backward_amax(torch.from_numpy(dH).to(DEV), _bf16_dev(ag), _bf16_dev(au), gg, gu, dev(sx),
                                 dev(swg), dev(swu), amax, ws)
    torch.cuda.synchronize()
    return _bits(gg), _bits(gu), host(amax).view(np.uint32)


@pytest.mark.parametrize("T,F,scaled", [(300, 1100, True), (64, 512, False), (1024, 14336, True), (7, 9, True)])
def test_glue_amax_matches_quantizer_amax(T, F, scaled):
    # the glue's results are bit-exact and its two amax values are the quantizer's own
    # max |fl(fl(G * s_x) * s_w)| of those results (ragged tiles; full d_ff at 1024 tokens)
    dH, ag, au = _draw(T, F, T + F)
    rng = np.random.default_rng(F)
    sx = rng.uniform(0.01, 0.05, T).astype(np.float32) if scaled else None
    swg = rng.uniform(1e-4, 1e-3, F).astype(np.float32) if scaled else None
    swu = rng.uniform(1e-4, 1e-3, F).astype(np.float32) if scaled else None
    gg, gu, amax = _glue_amax(dH, ag, au, sx, swg, swu)
    ref_g, ref_u = sg.glue(dH, ag, au)
    np.testing.assert_array_equal(gg, ref_g)
    np.testing.assert_array_equal(gu, ref_u)
    _check_amax(int(amax[0]), _amax_bits(ref_g, sx, swg))
    _check_amax(int(amax[1]), _amax_bits(ref_u, sx, swu))


def test_glue_amax_non_finite_and_strided():
    # a NaN or Inf result reaches the amax (NaN orders above Inf); unaligned layouts take the scalar path
    T, F = 6, 40
    dH, ag, au = _draw(T, F, 5)
    dH[2, 3] = np.inf
    ref_g, ref_u = sg.glue(dH, ag, au)
    for pad in (0, 3):
        dHb = torch.zeros(T, F + pad, device=DEV)
        dHb[:, :F] = torch.from_numpy(dH)
        Ab = torch.zeros(2, T, F + pad, dtype=torch.bfloat16, device=DEV)
        Ab[0, :, :F] = _bf16_dev(ag)
        Ab[1, :, :F] = _bf16_dev(au)
        Gb = torch.zeros(2, T, F + pad, dtype=torch.bfloat16, device=DEV)
        amax = torch.zeros(2, dtype=torch.int32, device=DEV)
        ws = torch.zeros(s3r.s3r_swiglu_amax_workspace(T, F), dtype=torch.uint8, device=DEV)
        s3r.s3r_swiglu_backward_amax(dHb[:, :F], Ab[0, :, :F], Ab[1, :, :F], Gb[0, :, :F], Gb[1, :, :F], None, None,
                                     None, amax, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(Gb[0, :, :F]), ref_g)
        np.testing.assert_array_equal(_bits(Gb[1, :, :F]), ref_u)
        got = host(amax).view(np.uint32)
        _check_amax(int(got[0]), _amax_bits(ref_g, None, None))
        _check_amax(int(got[1]), _amax_bits(ref_u, None, None))


def test_glue_amax_then_quantize_with_amax_equals_oracle_chain():
    # gate / up stage of the block: glue (with amax) -> quantize_with_amax equals the oracle's glue ->
    # quantize (its own amax) on codes, step and S3R-EC statistics
    from oracle import pipeline, quantize as oq
    T, F, S = 512, 1100, 128
    dH, ag, au = _draw(T, F, 99)
    rng = np.random.default_rng(4)
    sx = rng.uniform(0.01, 0.05, T).astype(np.float32)
    swg = rng.uniform(1e-4, 1e-3, F).astype(np.float32)
    gg, gu, amax = _glue_amax(dH, ag, au, sx, swg, None)
    ref_g, _ = sg.glue(dH, ag, au)
    np.testing.assert_array_equal(gg, ref_g)
    d = s3r.qdesc(T, F, S, s3r.S3R, s3r.EC_TWO_WAY, layer_id=1, seed=11)
    Q = s3r.q_buffer(T, F, DEV)
    delta = torch.empty(1, device=DEV)
    er, ecl, em = torch.empty(T, device=DEV), torch.empty(T // S, F, device=DEV), torch.empty(T // S, device=DEV)
    ws = torch.zeros(s3r.s3r_quantize_workspace(d), dtype=torch.uint8, device=DEV)
    amax_d = torch.from_numpy(amax[:1].view(np.int32).copy()).to(DEV)
    s3r.s3r_quantize_with_amax(d, _bf16_dev(gg), torch.from_numpy(sx).to(DEV), torch.from_numpy(swg).to(DEV), amax_d,
                               Q, delta, er, ecl, em, None, ws)
    torch.cuda.synchronize()
    fx, fw = {"scale": sx}, {"scale": swg}
    ref = pipeline.quantize_gradient(ref_g, "bf16", fx, fw, mode=oq.S3R, scale=oq.PER_TENSOR, seed=11, layer_id=1,
                                     rows_per_example=S)
    np.testing.assert_array_equal(host(Q), ref["Q"])
    np.testing.assert_array_equal(host(delta), ref["delta"])
    for got, exp in ((er, ref["eps"]), (ecl, ref["ebar"])):
        e = np.abs(host(got) - exp).max() / np.abs(exp).max()
        assert e <= 1e-5, e
