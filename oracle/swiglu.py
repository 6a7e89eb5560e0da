"""SwiGLU backward glue of the FFN block (oracle; test infrastructure only).

The S3R page times one SwiGLU FFN block forward and backward ("Setup", the
single-block FFN benchmarks, and Table III).  Between the down projection's
backward and the gate / up projections' backward sits the elementwise
derivative of H = silu(A_gate) * A_up with respect to the two pre-activations:

    G_up   = dH * silu(A_gate)
    G_gate = dH * A_up * silu'(A_gate)
    silu(a) = a * s,  silu'(a) = s * (1 + a * (1 - s)),  s = 1 / (1 + exp(-a))

This is not part of the method; the pages do not fix its arithmetic.  The
reading taken here: IEEE fp32 with one rounding per operation, in exactly the
order written in ``glue``, with the exponential ``exp32`` defined below (a
Cody-Waite reduction by ln 2 and the degree-7 Taylor polynomial of exp), and
the two results rounded to bfloat16 (nearest, ties to even).  The GPU kernel
follows the same definition, so both produce the same bf16 bits.

Pins (tests/test_oracle_pins.py): exp32 against math.exp, silu' against a
central difference of silu in float64, the closed forms at 0 and at large |a|,
and the bf16 rounding against exact rational rounding.
"""
from __future__ import annotations

import numpy as np

F = np.float32
LOG2E = F(1.4426950408889634)          # log2(e) rounded to fp32
LN2_HI = F(0.693145751953125)          # 0x3F317200: ln 2 with 15 significant bits (n * LN2_HI exact, |n| < 512)
LN2_LO = F(1.4286068203094173e-06)     # ln 2 - LN2_HI rounded to fp32
TAYLOR = [F(1.0), F(1.0), F(1 / 2), F(1 / 6), F(1 / 24), F(1 / 120), F(1 / 720), F(1 / 5040)]
X_MIN, X_MAX = F(-104.0), F(89.0)      # exp underflows / overflows fp32 beyond these


def exp32(x: np.ndarray) -> np.ndarray:
    """exp in fp32: clamp, n = rint(x log2 e), r = (x - n ln2_hi) - n ln2_lo, Taylor(r) * 2^n."""
    x = np.asarray(x, dtype=F)
    with np.errstate(all="ignore"):
        return _exp32(x)


def _exp32(x: np.ndarray) -> np.ndarray:
    xc = np.where(x < X_MIN, X_MIN, np.where(x > X_MAX, X_MAX, x)).astype(F)    # NaN passes through
    n = np.rint((xc * LOG2E).astype(F)).astype(F)
    r = ((xc - (n * LN2_HI).astype(F)).astype(F) - (n * LN2_LO).astype(F)).astype(F)
    p = TAYLOR[7]
    for c in TAYLOR[6::-1]:
        p = ((p * r).astype(F) + c).astype(F)
    ni = np.where(np.isnan(n), F(0), n).astype(np.int32)
    return np.ldexp(p, ni).astype(F)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, nearest with ties to even; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=F)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    b = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), b).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F)


def silu_parts(a: np.ndarray):
    """fp32 (s, silu(a), silu'(a)) in the fixed operation order."""
    a = np.asarray(a, dtype=F)
    with np.errstate(all="ignore"):
        return _silu_parts(a)


def _silu_parts(a: np.ndarray):
    e = exp32(-a)
    s = (F(1.0) / (F(1.0) + e).astype(F)).astype(F)
    silu = (a * s).astype(F)
    ds = (s * (F(1.0) + (a * (F(1.0) - s).astype(F)).astype(F)).astype(F)).astype(F)
    return s, silu, ds


def glue(dH: np.ndarray, A_gate_bits: np.ndarray, A_up_bits: np.ndarray):
    """(G_gate bits, G_up bits) of dH f32 [T x F] and the bf16 pre-activations A_gate, A_up."""
    dH = np.asarray(dH, dtype=F)
    a = bf16_to_f32(A_gate_bits)
    u = bf16_to_f32(A_up_bits)
    with np.errstate(all="ignore"):            # inf * 0 and the like give NaN, as in IEEE fp32
        _, silu, ds = silu_parts(a)
        g_up = (dH * silu).astype(F)
        g_gate = ((dH * u).astype(F) * ds).astype(F)
    return round_bf16(g_gate), round_bf16(g_up)
