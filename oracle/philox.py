"""Philox4x32-10 and the threshold maps built on it.  (Oracle: test use only.)

Generator: Philox4x32 with 10 rounds, the counter-based generator of Salmon,
Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
which the S3R page cites as its reference [16] beside Threefry (Related Work,
"The Cost of Randomness": each random word is a keyed function of a counter).
The pages use partitionable Threefry; this oracle (like the kernels) uses Philox4x32-10 with its
own counter layout, so thresholds are a pure function of (seed, layer, index)
and do not depend on how the work is split.

One Philox round maps the counter (c0, c1, c2, c3) with key (k0, k1) to
    (hi(B*c2) ^ c1 ^ k0,  lo(B*c2),  hi(A*c0) ^ c3 ^ k1,  lo(A*c0))
with the multipliers A = 0xD2511F53 and B = 0xCD9E8D57 and hi/lo the upper
and lower 32 bits of the 64-bit product.  Between rounds the key is bumped by
the Weyl constants (0x9E3779B9, 0xBB67AE85).

Counter layout used here (key = (low 32 bits of seed, high 32 bits of seed)):
  independent SR   element e = t*D + j:  counter (lo(e>>2), hi(e>>2), layer, 0),
                   word e & 3;  r = (2*(w >> 9) + 1) / 2**24
  S3R (per token)  token t:  counter (lo(t>>4), hi(t>>4), layer, 1),
                   word (t>>2) & 3, byte t & 3;  b = byte >> 1;  r = (2b + 1) / 256
  S3R (per example, the Phi_bcast ablation)  example b:  as S3R with the
                   example index b in place of t and tag 2
Word 3 of the counter is tag + 65536 * stream: stream 0 is the one threshold
tensor shared by both backward products; a second stream (1) gives the
independent draw R^RHS of a gradient quantized separately for the weight
gradient (the page's conventional, quantize-twice configuration).
The S3R map is the page's threshold slicing (Structured Subspace Randomness:
four 7-bit thresholds cut from each 32-bit word, on a grid shifted by half a
step, bias at most Delta/256).  The SR map is the same half-step grid with 23
bits (the page fixes one 32-bit word per element, Compared Configurations,
but not how it becomes a uniform).
"""
from __future__ import annotations

import numpy as np

PHILOX_A = np.uint64(0xD2511F53)
PHILOX_B = np.uint64(0xCD9E8D57)
WEYL_0 = 0x9E3779B9
WEYL_1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)

TAG_SR = 0
TAG_S3R = 1
TAG_BCAST = 2


def philox4x32_10(counter: np.ndarray, seed: int) -> np.ndarray:
    """Philox4x32-10 on an array of counters.

    counter: uint32-valued array of shape (N, 4).  seed: 64-bit key.
    Returns uint32 array (N, 4) of output words.
    """
    c = np.asarray(counter, dtype=np.uint64).reshape(-1, 4) & MASK32
    c0, c1, c2, c3 = (c[:, i].copy() for i in range(4))
    k0 = int(seed) & 0xFFFFFFFF
    k1 = (int(seed) >> 32) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + WEYL_0) & 0xFFFFFFFF
            k1 = (k1 + WEYL_1) & 0xFFFFFFFF
        p0 = PHILOX_A * c0          # exact: both factors < 2**32
        p1 = PHILOX_B * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n1 = p1 & MASK32
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        n3 = p0 & MASK32
        c0, c1, c2, c3 = n0, n1, n2, n3
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def _counters(block: np.ndarray, layer_id: int, tag: int, stream: int = 0) -> np.ndarray:
    block = np.asarray(block, dtype=np.uint64)
    ctr = np.empty((block.size, 4), dtype=np.uint64)
    ctr[:, 0] = block & MASK32
    ctr[:, 1] = block >> np.uint64(32)
    ctr[:, 2] = np.uint64(layer_id & 0xFFFFFFFF)
    ctr[:, 3] = np.uint64((tag + 65536 * stream) & 0xFFFFFFFF)
    return ctr


def sr_threshold_units(seed: int, layer_id: int, rows: int, cols: int,
                       row0: int = 0, stream: int = 0) -> np.ndarray:
    """Independent SR: one threshold per element, as the odd integer 2b+1 (r = value / 2**24).

    Element (t, j) of a [rows x cols] tensor has global index e = (row0 + t)*cols + j.
    Returns int64 array [rows, cols].
    """
    e = (np.arange(rows, dtype=np.uint64)[:, None] + np.uint64(row0)) * np.uint64(cols) \
        + np.arange(cols, dtype=np.uint64)[None, :]
    e = e.reshape(-1)
    if e.size == 0:
        return np.zeros((rows, cols), dtype=np.int64)
    first = int(e[0]) >> 2
    blocks = np.arange(first, (int(e[-1]) >> 2) + 1, dtype=np.uint64)
    words = philox4x32_10(_counters(blocks, layer_id, TAG_SR, stream), seed)
    inv = ((e >> np.uint64(2)) - np.uint64(first)).astype(np.int64)
    w = words[inv, (e & np.uint64(3)).astype(np.int64)].astype(np.int64)
    return (2 * (w >> 9) + 1).reshape(rows, cols)


def s3r_threshold_units(seed: int, layer_id: int, rows: int, row0: int = 0, stream: int = 0,
                        tag: int = TAG_S3R) -> np.ndarray:
    """S3R (Phi_2D): one threshold per token, as the odd integer 2b+1 (r = value / 256).

    Returns int64 array [rows] for tokens row0 .. row0+rows-1.  With tag=TAG_BCAST
    the index is an example's (Phi_bcast).
    """
    t = np.arange(rows, dtype=np.uint64) + np.uint64(row0)
    if t.size == 0:
        return np.zeros(0, dtype=np.int64)
    first = int(t[0]) >> 4
    blocks = np.arange(first, (int(t[-1]) >> 4) + 1, dtype=np.uint64)
    words = philox4x32_10(_counters(blocks, layer_id, tag, stream), seed)
    inv = ((t >> np.uint64(4)) - np.uint64(first)).astype(np.int64)
    w = words[inv, ((t >> np.uint64(2)) & np.uint64(3)).astype(np.int64)].astype(np.uint64)
    byte = (w >> (np.uint64(8) * (t & np.uint64(3)))) & np.uint64(0xFF)
    b = (byte >> np.uint64(1)).astype(np.int64)
    return 2 * b + 1


def sr_thresholds(seed: int, layer_id: int, rows: int, cols: int, row0: int = 0, stream: int = 0) -> np.ndarray:
    """Independent SR thresholds r in (0, 1) as exact float64 values [rows, cols]."""
    return sr_threshold_units(seed, layer_id, rows, cols, row0, stream).astype(np.float64) * 2.0 ** -24


def s3r_thresholds(seed: int, layer_id: int, rows: int, row0: int = 0, stream: int = 0) -> np.ndarray:
    """S3R per-token thresholds r in (0, 1) as exact float64 values [rows]."""
    return s3r_threshold_units(seed, layer_id, rows, row0, stream).astype(np.float64) / 256.0


def bcast_thresholds(seed: int, layer_id: int, rows: int, rows_per_example: int, row0: int = 0,
                     stream: int = 0) -> np.ndarray:
    """Phi_bcast: every token of example b = t // S takes that example's threshold; float64 [rows].

    S3R page, "Threshold Broadcasting": the per-example broadcast keeps each
    threshold marginally uniform but shares it across all tokens and channels
    of an example (an ablation).  Rows row0 .. row0+rows-1.
    """
    if rows == 0:
        return np.zeros(0)
    S = rows_per_example
    b = (np.arange(rows) + row0) // S
    b0 = int(b[0])
    units = s3r_threshold_units(seed, layer_id, int(b[-1]) - b0 + 1, row0=b0, stream=stream, tag=TAG_BCAST)
    return units[b - b0].astype(np.float64) / 256.0
