"""S3R-EC: the structured error correction.  (Oracle: test use only.)

S3R page, section "Structured Error Correction (S3R-EC)", "Two-Way
Correction": the quantizer knows the rounding error E = G~ - G exactly.  For
each example b it takes the mean error of every token over its channels and
the mean error of every channel over the tokens of the example; together they
form the orthogonal projection of E_b (S x D) onto the subspace of sums of
row-constant and column-constant matrices, {1_S a^T + c 1_D^T} (eqs. (3)-(4),
lost from the text).  That projection is

    P(E_b)[s, j] = ebar_b[j] + eps_{b,s} - mu_b,

with ebar_b the per-example channel means, eps the per-token means and mu_b
the example's grand mean (the grand mean is subtracted once, so that the
sum of a row-constant and a column-constant part is not counted twice).  What
remains after subtracting it sums to zero along every row and every column.

The error is taken in the folded space (G', with the fixed rescalings by
1/s_x and 1/s_w applied later): E'[t, j] = Delta_t * (q[t, j] - x[t, j]).
All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np


def rounding_error(q: np.ndarray, x: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """E' = Delta * (q - x) in float64; delta is [1] (per tensor) or [T] (per token)."""
    d = np.asarray(delta, dtype=np.float64)
    d = d[0] if d.size == 1 else d[:, None]
    return d * (q.astype(np.float64) - x.astype(np.float64))


def statistics(E: np.ndarray, rows_per_example: int):
    """(eps [T], ebar [B, D], mu [B]): token means, per-example channel means, grand means."""
    T, D = E.shape
    S = rows_per_example
    B = T // S if S else 0
    if D == 0 or T == 0:
        return np.zeros(T), np.zeros((B, D)), np.zeros(B)
    eps = E.mean(axis=1)
    Eb = E.reshape(B, S, D)
    ebar = Eb.mean(axis=1)
    mu = Eb.mean(axis=(1, 2))
    return eps, ebar, mu


def projection(eps: np.ndarray, ebar: np.ndarray, mu: np.ndarray, rows_per_example: int) -> np.ndarray:
    """Dense P(E) [T, D] from its factors: ebar_b[j] + eps_t - mu_b."""
    S = rows_per_example
    b_of_t = np.arange(eps.size) // S
    return ebar[b_of_t] + (eps - mu[b_of_t])[:, None]


def center(v: np.ndarray) -> np.ndarray:
    """Subtract the group mean (S3R page, "Subtracting the Mean Removes the Correlation")."""
    return v - v.mean(axis=-1, keepdims=True)
