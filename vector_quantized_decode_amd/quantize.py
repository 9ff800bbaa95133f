"""Offline 3.125-bit quantizer for the rotated-residual decode path.

From a weight matrix W [N][K] it makes what vq_gemv_residual decodes: a 256 x 4
fp16 codebook, an 8-bit codeword per group of 4 consecutive rotated weights,
one sign bit per weight and one fp16 scale per 128 weights of a row, plus the
rotation (a random +-1 diagonal and a Hadamard block size).  The method is the
3.125-bit edge format of "Replacing MatMul with SRAM lookup: a 3-bit edge
inference architecture" (section details): rotate the weights by a randomized
Hadamard transform, cluster their 4-vectors into 256 centroids, and encode
what the centroids miss with one sign per weight and one scale per 128.  It
runs on the host in numpy, once per matrix, off the decode path.

Readings where that page is silent:
  * The rotation is the decode's own: the decode rotates x into
    x' = blockdiag(H_h) diag(s) x / sqrt(h), H_h the Sylvester Hadamard matrix
    of the largest power of two h dividing K.  Turning every row of W the
    same way keeps the product: W' x' = W x.
  * The page weighs the clustering by weight sensitivity; synthetic weights
    have none, so every coordinate weighs 1 unless a sensitivity array is
    given, which then weighs both the nearest-centroid search and the
    centroid updates (weighted Lloyd rounds).
  * A coordinate the centroid matches exactly gets sign bit 1 (+1).
  * Each group's scale is the one that minimizes its weighted squared error
    between the miss and scale * sign, i.e. the weighted mean of |miss|.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["Quantized", "rotate_rows", "quantize_rotated_residual"]

QUAD = 4            # weights per codeword
TABLE = 256         # codebook entries (8-bit codewords)
SCALE_GROUP = 128   # weights sharing one residual scale
_CHUNK = 8192       # 4-vectors per distance evaluation (bounds the temporary array)


@dataclass
class Quantized:
    wc: np.ndarray          # float16 [256][4] codebook
    idx: np.ndarray         # uint8 [N][K/4] codeword of each group of 4 rotated weights
    sign_bits: np.ndarray   # uint8 {0,1} [N][K], 1 means +1
    alpha: np.ndarray       # float16 [N][K/group] residual scales
    rht_sign: np.ndarray    # int8 {-1,+1} [K]
    had_block: int
    group: int
    objective: List[float] = field(default_factory=list)   # clustering error after each round


# ------------------------------------------------------------------ rotation
def _hadamard_blocks(a: np.ndarray, h: int) -> np.ndarray:
    """Each length-h block along the last axis of ``a`` multiplied by the
    (unnormalized) Sylvester Hadamard matrix H_h: log2 h rounds of pairwise
    sums and differences, pair distance 1, 2, 4, ..."""
    x = np.array(a, dtype=np.float64, copy=True)
    shape = x.shape
    span = 1
    while span < h:
        pairs = x.reshape(-1, 2, span)          # [..., first half, second half] of each 2*span run
        lo = pairs[:, 0, :].copy()
        pairs[:, 0, :] += pairs[:, 1, :]
        pairs[:, 1, :] = lo - pairs[:, 1, :]
        x = pairs.reshape(shape)
        span *= 2
    return x


def rotate_rows(W: np.ndarray, rht_sign: np.ndarray, h: int) -> np.ndarray:
    """Every row w of W turned to w' = blockdiag(H_h) diag(s) w / sqrt(h)."""
    flipped = np.asarray(W, dtype=np.float64) * rht_sign.astype(np.float64)[None, :]
    return _hadamard_blocks(flipped, h) / np.sqrt(h)


# ------------------------------------------------------------------ clustering
def _nearest(vecs: np.ndarray, weight: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table row with the least weighted squared distance, per row of vecs."""
    out = np.empty(vecs.shape[0], dtype=np.int64)
    for lo in range(0, vecs.shape[0], _CHUNK):
        v, w = vecs[lo:lo + _CHUNK], weight[lo:lo + _CHUNK]
        dist = np.einsum("nkd,nd->nk", (v[:, None, :] - table[None, :, :]) ** 2, w)
        out[lo:lo + _CHUNK] = dist.argmin(axis=1)
    return out


def _lloyd(vecs: np.ndarray, weight: np.ndarray, seeds: np.ndarray,
           rounds: int) -> Tuple[np.ndarray, np.ndarray, List[float]]:
    """Weighted Lloyd rounds from the initial table ``seeds``: each round
    assigns every vector its nearest entry, records the weighted error, and
    moves every used entry to the weighted mean of its vectors (an unused one
    stays put)."""
    table = seeds.copy()
    trace: List[float] = []
    code = np.zeros(vecs.shape[0], dtype=np.int64)
    for _ in range(rounds):
        code = _nearest(vecs, weight, table)
        trace.append(float((weight * (vecs - table[code]) ** 2).sum()))
        wsum = np.zeros_like(table)
        wvec = np.zeros_like(table)
        np.add.at(wsum, code, weight)
        np.add.at(wvec, code, weight * vecs)
        used = wsum > 0
        table[used] = wvec[used] / wsum[used]
    return table, code, trace


# ------------------------------------------------------------------ residual
def _sign_scale(miss: np.ndarray, weight: np.ndarray, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """One bit per weight (1 where the miss is >= 0) and, per group of
    ``group`` weights of a row, the scale minimizing the weighted error
    sum w (miss - a sign)^2: a = sum w |miss| / sum w."""
    N, K = miss.shape
    bits = (miss >= 0).astype(np.uint8)
    num = (weight * np.abs(miss)).reshape(N, K // group, group).sum(axis=2)
    den = weight.reshape(N, K // group, group).sum(axis=2)
    return bits, num / np.maximum(den, 1e-300)


# ------------------------------------------------------------------ the format
def quantize_rotated_residual(W: np.ndarray, *, seed: int = 0, iters: int = 12,
                              sensitivity: Optional[np.ndarray] = None, group: int = SCALE_GROUP,
                              d: int = QUAD, k: int = TABLE) -> Quantized:
    """Quantize W [N][K] to the 3.125-bit format the residual decode reads
    (d = 4, 256 codebook entries, one scale per 128 weights); ``iters``
    Lloyd rounds from ``k`` seed vectors drawn from the matrix."""
    if d != QUAD or k != TABLE or group != SCALE_GROUP:
        raise ValueError("the decode kernels take d = 4, 256 centroids and groups of 128")
    weights = np.asarray(W, dtype=np.float64)
    N, K = weights.shape
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    diag = np.where(rng.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)
    h = K & (-K)
    turned = rotate_rows(weights, diag, h)

    quads = turned.reshape(-1, QUAD)
    if sensitivity is None:
        wq = np.ones_like(quads)
    else:
        wq = np.asarray(sensitivity, dtype=np.float64).reshape(-1, QUAD)
    seeds = quads[rng.choice(quads.shape[0], size=TABLE, replace=quads.shape[0] < TABLE)]
    table, _, trace = _lloyd(quads, wq, seeds, iters)

    # the decode holds the table in fp16, so codewords are chosen against the
    # rounded table, and the residual encodes what that table misses
    table16 = table.astype(np.float16)
    code = _nearest(quads, wq, table16.astype(np.float64))
    miss = turned - table16.astype(np.float64)[code].reshape(N, K)
    bits, scale = _sign_scale(miss, wq.reshape(N, K), group)
    return Quantized(wc=table16, idx=code.reshape(N, K // QUAD).astype(np.uint8), sign_bits=bits,
                     alpha=scale.astype(np.float16), rht_sign=diag, had_block=h, group=group,
                     objective=trace)
