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


def test_glue_every_bf16_pre_activation():
    # A_gate takes every one of the 65536 bf16 bit patterns (zeros, subnormals, the clamp bounds of the
    # exponential and beyond, infinities, NaNs), so the exponential, the reciprocal and the bf16
    # rounding see every value they can see in the glue; bit-exact against the oracle
    T, F = 256, 256
    ag = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(T, F)
    rng = np.random.default_rng(65536)
    dH = (rng.standard_normal((T, F)) * np.float32(1e-3)).astype(np.float32)
    dH[0, :8] = np.float32([1.0, -1.0, 3e38, -3e38, 1e-40, 0.0, np.inf, np.nan])
    au = inputs.f32_to_bf16_bits(rng.standard_normal((T, F)).astype(np.float32))
    gg, gu = s3r.swiglu_backward(torch.from_numpy(dH).to(DEV), _bf16_dev(ag), _bf16_dev(au))
    torch.cuda.synchronize()
    ref_g, ref_u = sg.glue(dH, ag, au)
    np.testing.assert_array_equal(_bits(gg), ref_g)
    np.testing.assert_array_equal(_bits(gu), ref_u)


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


# ---------------------------------------- gate / up quantizers with the glue inside ----

def _scales(T, F, seed, scaled=True):
    rng = np.random.default_rng(seed + 7)
    if not scaled:
        return None, None, None
    return (rng.uniform(0.01, 0.05, T).astype(np.float32), rng.uniform(1e-4, 1e-3, F).astype(np.float32),
            rng.uniform(1e-4, 1e-3, F).astype(np.float32))


def _dev(a):
    return None if a is None else torch.from_numpy(a).to(DEV)


class _Out:
    """One projection's outputs on the device, pre-filled with garbage the call must overwrite."""

    def __init__(self, T, F, S, ld, ec):
        B = T // S
        self.Qb = torch.full((T, ld), 99, dtype=torch.int8, device=DEV)
        self.Q = self.Qb[:, :F]
        self.delta = torch.full((1,), -5.0, device=DEV)
        self.ec = ((torch.full((T,), 7.0, device=DEV), torch.full((B, F), 7.0, device=DEV),
                    torch.full((B,), 7.0, device=DEV)) if ec != s3r.EC_NONE else (None, None, None))

    def host(self):
        r = {"Q": host(self.Q), "delta": host(self.delta), "pad": host(self.Qb[:, self.Q.shape[1]:])}
        if self.ec[0] is not None:
            r["eps"], r["ebar"], r["mu"] = (host(t) for t in self.ec)
        return r


def _layout(dH, ag, au, ld):
    T, F = dH.shape
    dHb = torch.zeros(T, ld, device=DEV)
    dHb[:, :F] = torch.from_numpy(dH)
    Ab = torch.zeros(2, T, ld, dtype=torch.bfloat16, device=DEV)
    Ab[0, :, :F] = _bf16_dev(ag)
    Ab[1, :, :F] = _bf16_dev(au)
    return dHb[:, :F], Ab[0, :, :F], Ab[1, :, :F]


def _garbage_ws(n):
    return torch.full((max(n, 1),), 0x5A, dtype=torch.uint8, device=DEV)


def _fused(dH, ag, au, sc, descs, ld):
    """s3r_swiglu_quantize with every row at leading dimension ld: (gate outputs, up outputs, flags)."""
    T, F = dH.shape
    d_h, a_g, a_u = _layout(dH, ag, au, ld)
    outs = [_Out(T, F, descs[0].rows_per_example, ld, descs[0].ec) for _ in range(2)]
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = _garbage_ws(s3r.s3r_swiglu_quantize_workspace(descs[0]))
    s3r.s3r_swiglu_quantize(descs[0], descs[1], d_h, a_g, a_u, _dev(sc[0]), _dev(sc[1]), _dev(sc[2]), outs[0].Q,
                            outs[1].Q, outs[0].delta, outs[1].delta, outs[0].ec, outs[1].ec, flags, ws)
    torch.cuda.synchronize()
    return outs[0].host(), outs[1].host(), int(host(flags)[0])


def _separate(dH, ag, au, sc, descs, ld):
    """The same through s3r_swiglu_backward_amax (G_gate, G_up written) and two s3r_quantize_with_amax."""
    T, F = dH.shape
    d_h, a_g, a_u = _layout(dH, ag, au, ld)
    Gb = torch.zeros(2, T, ld, dtype=torch.bfloat16, device=DEV)
    amax = torch.zeros(2, dtype=torch.int32, device=DEV)
    s3r.s3r_swiglu_backward_amax(d_h, a_g, a_u, Gb[0, :, :F], Gb[1, :, :F], _dev(sc[0]), _dev(sc[1]), _dev(sc[2]),
                                 amax, _garbage_ws(s3r.s3r_swiglu_amax_workspace(T, F)))
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    res = []
    for k in range(2):
        o = _Out(T, F, descs[k].rows_per_example, ld, descs[k].ec)
        s3r.s3r_quantize_with_amax(descs[k], Gb[k, :, :F], _dev(sc[0]), _dev(sc[1 + k]), amax[k:k + 1], o.Q, o.delta,
                                   *o.ec, flags, _garbage_ws(s3r.s3r_quantize_workspace(descs[k])))
        res.append(o)
    torch.cuda.synchronize()
    return res[0].host(), res[1].host(), int(host(flags)[0])


def _assert_same(a, b):
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint8), b[k].view(np.uint8), err_msg=k)


def _descs(T, F, S, mode, ec, seeds=(11, 12), layers=(1, 2), streams=(0, 1)):
    return [s3r.qdesc(T, F, S, mode, ec, layer_id=layers[k], seed=seeds[k], stream=streams[k]) for k in range(2)]


SQ_CASES = [
    # T, F, S, mode, ec, leading-dim padding (None: to 16 elements, the vector path)
    (512, 1100, 128, s3r.S3R, s3r.EC_TWO_WAY, None),      # ragged column tile, full row tiles
    (512, 1100, 128, s3r.S3R, s3r.EC_TWO_WAY, 3),         # unaligned rows: the general path everywhere
    (200, 520, 50, s3r.S3R_BCAST, s3r.EC_DW_ONLY, None),  # ragged row tiles (S = 50), one threshold per example
    (256, 1024, 256, s3r.SR, s3r.EC_NONE, None),
    (96, 77, 32, s3r.SR, s3r.EC_NONE, None),              # D % 4 != 0: one Philox block per element
    (256, 1024, 128, s3r.RTNE, s3r.EC_NONE, None),
    (128, 2048, 128, s3r.S3R, s3r.EC_NONE, None),
    (1024, 14336, 256, s3r.S3R, s3r.EC_TWO_WAY, None),    # full d_ff
]


@pytest.mark.parametrize("T,F,S,mode,ec,pad", SQ_CASES)
def test_swiglu_quantize_equals_glue_then_quantizers_and_oracle(T, F, S, mode, ec, pad):
    # the fused call reproduces the unfused chain bit for bit (codes, steps, statistics, flags, untouched
    # padding), and the oracle's glue -> quantizer chain: codes and steps exactly, statistics within 1e-5
    from oracle import pipeline, quantize as oq
    from tests._gpu import assert_rows_close, rel_err
    print(f"[case] swiglu_quantize T={T} F={F} S={S} mode={mode} ec={ec} pad={pad}", flush=True)
    dH, ag, au = _draw(T, F, T + 3 * F)
    sc = _scales(T, F, F)
    ld = F + (-F) % 16 + (pad or 0)
    descs = _descs(T, F, S, mode, ec)
    fg, fu, ff = _fused(dH, ag, au, sc, descs, ld)
    sg_, su_, sf = _separate(dH, ag, au, sc, descs, ld)
    _assert_same(fg, sg_)
    _assert_same(fu, su_)
    assert ff == sf == 0
    assert (fg["pad"] == 99).all() and (fu["pad"] == 99).all()
    refs = sg.glue(dH, ag, au)
    for k, got in enumerate((fg, fu)):
        ref = pipeline.quantize_gradient(refs[k], "bf16", {"scale": sc[0]}, {"scale": sc[1 + k]}, mode=mode,
                                         scale=oq.PER_TENSOR, seed=descs[k].seed, layer_id=descs[k].layer_id,
                                         rows_per_example=S, stream=descs[k].stream)
        np.testing.assert_array_equal(got["Q"], ref["Q"])
        np.testing.assert_array_equal(got["delta"], ref["delta"])
        if ec != s3r.EC_NONE:
            assert rel_err(got["eps"], ref["eps"]) <= 1e-5
            assert_rows_close(got["ebar"], ref["ebar"], 1e-5, f"swiglu_quantize ebar[{k}]")
            assert rel_err(got["mu"], ref["mu"]) <= 1e-5


def test_swiglu_quantize_unscaled_and_non_finite():
    # no forward scales; then an Inf in dH: the non-finite amax flags the projections (their codes are
    # zero, their steps the amax over 127: Inf, or NaN where a NaN result wins), exactly as the unfused chain
    T, F, S = 128, 600, 64
    dH, ag, au = _draw(T, F, 21)
    descs = _descs(T, F, S, s3r.S3R, s3r.EC_TWO_WAY)
    for poison in (False, True):
        if poison:
            dH[3, 5] = np.inf
        fg, fu, ff = _fused(dH, ag, au, (None, None, None), descs, 608)
        sg_, su_, sf = _separate(dH, ag, au, (None, None, None), descs, 608)
        _assert_same(fg, sg_)
        _assert_same(fu, su_)
        assert ff == sf
        if poison:
            assert ff & 1 and (fg["Q"] == 0).all() and not np.isfinite(fg["delta"][0])


def test_swiglu_quantize_empty():
    for T, F in ((0, 64), (64, 0)):
        descs = _descs(T, F, max(T, 1), s3r.S3R, s3r.EC_TWO_WAY)
        dH = np.zeros((T, F), np.float32)
        a = np.zeros((T, F), np.uint16)
        fg, fu, ff = _fused(dH, a, a, (None, None, None), descs, 64)
        for o in (fg, fu):
            assert o["delta"][0] == 1.0 and ff == 0
            assert (o["eps"] == 0).all() and (o["mu"] == 0).all()


def test_swiglu_quantize_ffn_block_size():
    # the FFN block's gate / up stage: 8192 tokens x d_ff 14336 in 4 examples of 2048, S3R-EC.  Against the
    # unfused chain bit for bit; against the oracle: the steps from the whole tensor's amax (oracle glue in
    # row chunks), codes and token means of sampled 64-row tiles quantized with that amax
    from oracle import ec as ecm, quantize as oq
    T, F, S = 8192, 14336, 2048
    dH, ag, au = _draw(T, F, 1234)
    sc = _scales(T, F, 5)
    descs = _descs(T, F, S, s3r.S3R, s3r.EC_TWO_WAY)
    fg, fu, ff = _fused(dH, ag, au, sc, descs, F)
    for k, (f, s) in enumerate(zip((fg, fu), _separate(dH, ag, au, sc, descs, F)[:2])):
        _assert_same(f, s)
    amax = [np.float32(0), np.float32(0)]
    for r in range(0, T, 1024):
        g2 = sg.glue(dH[r:r + 1024], ag[r:r + 1024], au[r:r + 1024])
        for k in range(2):
            x = oq.fold(oq.decode(g2[k], "bf16"), sc[0][r:r + 1024], sc[1 + k])
            amax[k] = max(amax[k], np.abs(x).max())
    for k, got in enumerate((fg, fu)):
        assert got["delta"][0] == oq.step_from_amax(np.array([amax[k]], np.float32))[0][0]
        for r0 in (0, 2048, 5120, T - 64):
            rows = slice(r0, r0 + 64)
            g2 = sg.glue(dH[rows], ag[rows], au[rows])[k]
            ref = oq.quantize(g2, "bf16", mode=oq.S3R, row_scale=sc[0][rows], col_scale=sc[1 + k],
                              seed=descs[k].seed, layer_id=descs[k].layer_id, rows_per_example=S,
                              stream=descs[k].stream, row0=r0, amax=amax[k])
            np.testing.assert_array_equal(got["Q"][rows], ref["Q"])
            E = ecm.rounding_error(ref["Q"], ref["x"], ref["delta"])
            eps = E.mean(axis=1)
            assert np.abs(got["eps"][rows] - eps).max() <= 1e-5 * np.abs(eps).max()
