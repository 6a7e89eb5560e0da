"""Seeded synthetic inputs for the quantized backward of one linear layer.

This module only draws random numbers and stores them as fp32 or bf16 bit
patterns.  It holds none of the quantizer's or the GEMMs' arithmetic, so both
the GPU path and the CPU oracle can be fed from it without sharing any of the
method.

Distributions follow the workloads of "Efficient Quantization Training with
Stochastic Rounding via Structured Subspace Randomness": heavy-tailed upstream
gradients (Introduction: backward gradients are heavy-tailed and span a wide
dynamic range), Gaussian activations and small Gaussian weights.  The pages
train on C4 and real checkpoints; these draws stand in for them.

Seeding: every tensor has its own ``numpy.random.default_rng`` stream with
seed ``1000 * workload_id + k`` (k: G = 1, X = 2, W = 3, A_gate = 4, A_up = 5).
Values are drawn in float64, rounded to float32, then (where a workload says
bf16) rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "student_t", "gaussian", "make_linear_inputs", "FfnBlock", "BLOCKS", "make_ffn_block_inputs",
    "MoeExperts", "MOE", "zipf_counts", "make_moe_inputs",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def student_t(seed: int, shape, nu: float, scale: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_t(nu, size=shape)).astype(np.float32)


def gaussian(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal(size=shape)).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """One linear layer's backward problem: G [T x D], X [T x d_in], W [D x d_in]."""
    name: str
    wid: int                 # seed base: 1000 * wid + k
    tokens: int              # T
    d_in: int
    d_out: int               # D, the hidden dimension of G
    rows_per_example: int    # S, tokens per example (T % S == 0)
    dtype: str               # "f32" or "bf16"
    g_nu: float
    g_scale: float
    outlier_frac: float = 0.0    # fraction of tokens scaled by outlier_mult
    outlier_mult: float = 1.0
    x_std: float = 1.0
    w_std: float = 0.02
    note: str = field(default="", compare=False)

    def scaled(self, tokens: int, d_in: int, d_out: int, rows_per_example: int | None = None,
               name: str | None = None) -> "Workload":
        """Same distributions at another shape (for small parity cases)."""
        return Workload(name or f"{self.name}@{tokens}x{d_in}x{d_out}", self.wid, tokens, d_in, d_out,
                        rows_per_example or tokens, self.dtype, self.g_nu, self.g_scale,
                        self.outlier_frac, self.outlier_mult, self.x_std, self.w_std, self.note)


WORKLOADS = {
    # single linear backward, fp32: T=256, d_in=512, d_out=1024
    "linear-256x512x1024-f32": Workload(
        "linear-256x512x1024-f32", 1, 256, 512, 1024, 256, "f32", 3.0, 1e-3),
    # Llama-style FFN down-projection, bf16: T=4096, 11008 -> 4096, 1% outlier tokens x100
    "down-4096x11008x4096-bf16": Workload(
        "down-4096x11008x4096-bf16", 2, 4096, 11008, 4096, 4096, "bf16", 2.5, 1e-4,
        outlier_frac=0.01, outlier_mult=100.0),
    # Llama-3-8B FFN down-projection, bf16: T=8192 (4 x 2048), 14336 -> 4096
    "down-8192x14336x4096-bf16": Workload(
        "down-8192x14336x4096-bf16", 3, 8192, 14336, 4096, 2048, "bf16", 3.0, 1e-4,
        note="X ~ N(0,1) stands in for the SwiGLU output feeding the down-projection"),
}


# The 4-bit (MXFP4) variant of the Llama-3-8B down-projection backward: the same shape with
# Student-t(nu=3) gradients; G is rounded to E2M1 with one E8M0 scale per 32 elements.
MX_WORKLOADS = {
    "mx-down-8192x14336x4096-bf16": Workload(
        "mx-down-8192x14336x4096-bf16", 6, 8192, 14336, 4096, 2048, "bf16", 3.0, 1e-4,
        note="MXFP4 operands; X ~ N(0,1) stands in for the SwiGLU output"),
}


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> storage: float32 array, or uint16 bf16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def make_linear_inputs(w: Workload, with_x: bool = True, with_w: bool = True) -> dict:
    """Draw G, X, W for workload ``w``.

    Returns storage arrays (float32, or uint16 bf16 bit patterns) under keys
    "G", "X", "W", plus "dtype".
    """
    base = 1000 * w.wid
    T, D, K = w.tokens, w.d_out, w.d_in
    g = student_t(base + 1, (T, D), w.g_nu, w.g_scale)
    if w.outlier_frac > 0 and T > 0:
        rng = np.random.default_rng(base + 6)
        n = int(round(w.outlier_frac * T))
        rows = rng.choice(T, n, replace=False)
        g[rows] *= np.float32(w.outlier_mult)
    out = {"G": _store(g, w.dtype), "dtype": w.dtype}
    if with_x:
        out["X"] = _store(gaussian(base + 2, (T, K), w.x_std), w.dtype)
    if with_w:
        out["W"] = _store(gaussian(base + 3, (D, K), w.w_std), w.dtype)
    return out


@dataclass(frozen=True)
class FfnBlock:
    """One SwiGLU FFN block: H = silu(X W_gate^T) * (X W_up^T), Y = H W_down^T.

    Its backward takes G_out = dY [T x d_model] and produces dX [T x d_model]
    and the three weight gradients.  The forward activations (A_gate, A_up and
    H) are synthetic inputs of the backward, drawn here.
    """
    name: str
    wid: int
    tokens: int              # T
    d_model: int
    d_ff: int
    rows_per_example: int    # S
    g_nu: float = 3.0
    g_scale: float = 1e-4
    w_std: float = 0.02

    def scaled(self, tokens: int, d_model: int, d_ff: int, rows_per_example: int | None = None) -> "FfnBlock":
        return FfnBlock(f"{self.name}@{tokens}x{d_model}x{d_ff}", self.wid, tokens, d_model, d_ff,
                        rows_per_example or tokens, self.g_nu, self.g_scale, self.w_std)


BLOCKS = {
    # Llama-3-8B-shaped FFN block, bf16: T=8192 (4 x 2048), d_model=4096, d_ff=14336
    "ffn-block-8192x4096x14336-bf16": FfnBlock("ffn-block-8192x4096x14336-bf16", 4, 8192, 4096, 14336, 2048),
}


def make_ffn_block_inputs(b: FfnBlock) -> dict:
    """bf16 bit patterns: G_out [T x d_model] = g_scale * t(g_nu); X [T x d_model], A_gate and
    A_up [T x d_ff] ~ N(0, 1); W_gate, W_up [d_ff x d_model] and W_down [d_model x d_ff] ~ N(0, w_std^2);
    H = silu(A_gate) * A_up evaluated in float64 from the bf16 values and rounded to bf16 (the
    forward activation the down projection consumed).  Seeds 1000 * wid + k, k: G_out 1, X 2,
    W_down 3, A_gate 4, A_up 5, W_gate 6, W_up 7."""
    base = 1000 * b.wid
    T, M, F = b.tokens, b.d_model, b.d_ff
    out = {"dtype": "bf16"}
    out["G"] = f32_to_bf16_bits(student_t(base + 1, (T, M), b.g_nu, b.g_scale))
    out["X"] = f32_to_bf16_bits(gaussian(base + 2, (T, M), 1.0))
    out["W_down"] = f32_to_bf16_bits(gaussian(base + 3, (M, F), b.w_std))
    out["A_gate"] = f32_to_bf16_bits(gaussian(base + 4, (T, F), 1.0))
    out["A_up"] = f32_to_bf16_bits(gaussian(base + 5, (T, F), 1.0))
    out["W_gate"] = f32_to_bf16_bits(gaussian(base + 6, (F, M), b.w_std))
    out["W_up"] = f32_to_bf16_bits(gaussian(base + 7, (F, M), b.w_std))
    h = np.empty((T, F), np.uint16)
    for r0 in range(0, T, 1024):                 # bounded float64 temporaries
        a = bf16_bits_to_f32(out["A_gate"][r0:r0 + 1024]).astype(np.float64)
        u = bf16_bits_to_f32(out["A_up"][r0:r0 + 1024]).astype(np.float64)
        h[r0:r0 + 1024] = f32_to_bf16_bits((a / (1.0 + np.exp(-a)) * u).astype(np.float32))
    out["H"] = h
    return out


@dataclass(frozen=True)
class MoeExperts:
    """The expert path of a mixture-of-experts FFN: top-k routing of ``tokens`` tokens over
    ``experts`` experts gives tokens * top_k rows, sorted by expert (expert e owns rows
    [offsets[e], offsets[e+1])).  Each expert is a linear layer; this is the backward of the
    experts' down projection: G [R x d_model], the expert inputs H [R x d_ff] and the weights
    W [experts x d_model x d_ff].  Rows per expert follow Zipf(zipf_s)."""
    name: str
    wid: int
    tokens: int
    top_k: int
    experts: int
    d_model: int
    d_ff: int
    zipf_s: float = 1.1
    g_nu: float = 3.0
    g_scale: float = 1e-4
    w_std: float = 0.02

    @property
    def rows(self) -> int:
        return self.tokens * self.top_k

    def scaled(self, tokens: int, experts: int, d_model: int, d_ff: int) -> "MoeExperts":
        return MoeExperts(f"{self.name}@{tokens}x{experts}x{d_model}x{d_ff}", self.wid, tokens, self.top_k,
                          experts, d_model, d_ff, self.zipf_s, self.g_nu, self.g_scale, self.w_std)


MOE = {
    # 64 experts, top-2 over 16384 tokens (32768 expert rows), d_model 2048, d_ff 1408
    "moe-64x16384-top2-2048x1408-bf16": MoeExperts("moe-64x16384-top2-2048x1408-bf16", 5, 16384, 2, 64, 2048, 1408),
}


def zipf_counts(rows: int, experts: int, s: float) -> np.ndarray:
    """Rows per expert proportional to k^-s (k = 1 .. experts), rounded by largest remainder so
    that they sum to ``rows`` (int64 [experts], largest first)."""
    w = np.arange(1, experts + 1, dtype=np.float64) ** -s
    share = rows * w / w.sum()
    base = np.floor(share).astype(np.int64)
    rest = rows - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rest]] += 1
    return base


def make_moe_inputs(m: MoeExperts) -> dict:
    """bf16 bit patterns G [R x d_model] = g_scale * t(g_nu), H [R x d_ff] ~ N(0, 1) and
    W [experts x d_model x d_ff] ~ N(0, w_std^2); "counts" (Zipf sizes dealt to the experts in a
    seeded random order, as a router would) and "offsets" int64 [experts + 1].  Seeds
    1000 * wid + k, k: G 1, H 2, W 3, expert order 8."""
    base = 1000 * m.wid
    R, E, M, F = m.rows, m.experts, m.d_model, m.d_ff
    counts = zipf_counts(R, E, m.zipf_s)
    counts = counts[np.random.default_rng(base + 8).permutation(E)]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return {"dtype": "bf16", "counts": counts, "offsets": offsets,
            "G": f32_to_bf16_bits(student_t(base + 1, (R, M), m.g_nu, m.g_scale)),
            "X": f32_to_bf16_bits(gaussian(base + 2, (R, F), 1.0)),
            "W": f32_to_bf16_bits(gaussian(base + 3, (E, M, F), m.w_std))}
