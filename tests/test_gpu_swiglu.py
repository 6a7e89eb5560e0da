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
