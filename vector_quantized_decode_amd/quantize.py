"""Offline 3.125-bit quantizer: rotated vector quantization plus a 1-bit residual.

Produces, from a weight matrix W [N][K], the inputs vq_gemv_residual decodes:
an fp16 codebook of 256 centroids of dimension 4, one 8-bit index per block of
4 rotated weights, one residual sign per weight and one fp16 scale per group of
128 weights, together with the rotation (a random +-1 diagonal and the
Hadamard block size).  It follows the pipeline of "Replacing MatMul with SRAM
lookup: a 3-bit edge inference architecture" (section details: randomized
Hadamard rotation of W, blocks of D = 4, K-means with K = 256, residual, its
signs, an optimal scale per group of G = 128, dense sign packing).  It runs on
the host in numpy, once per weight matrix; nothing of it is on the decode path.

Readings where that page is silent:
  * The rotation is the one the decode applies to x: x_rot = Q^T x with
    Q^T = blockdiag(H_h) diag(s) / sqrt(h), H_h the Sylvester Hadamard matrix
    of the largest power of two h dividing K; so W_rot = W Q and
    W_rot x_rot = W x.
  * "Sensitivity-aware" K-means weighs each weight's squared error by a
    sensitivity; none is known for synthetic weights, so the default weighs
    all weights equally (plain Lloyd iterations).  A sensitivity array can be
    passed; it weighs both the assignment distances and the centroid means.
  * A zero residual takes the sign +1 (bit 1).
  * The optimal scale of a group is the one minimizing its (weighted) squared
    error sum w (R - alpha s)^2 with s = sign(R): alpha = sum w |R| / sum w.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = ["Quantized", "rotate_rows", "quantize_rotated_residual"]


@dataclass
class Quantized:
    wc: np.ndarray          # float16 [256][4] codebook
    idx: np.ndarray         # uint8 [N][K/4] centroid of each block of 4 rotated weights
    sign_bits: np.ndarray   # uint8 {0,1} [N][K], 1 means +1
    alpha: np.ndarray       # float16 [N][K/group]
    rht_sign: np.ndarray    # int8 {-1,+1} [K]
    had_block: int
    group: int
    objective: List[float] = field(default_factory=list)   # K-means objective per iteration


def _fwht_last(a: np.ndarray, h: int) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform (Sylvester order) of every
    length-h block along the last axis, by radix-2 butterflies."""
    out = np.array(a, dtype=np.float64, copy=True)
    lead = out.shape[:-1]
    K = out.shape[-1]
    v = out.reshape(*lead, K // h, h)
    step = 1
    while step < h:
        v = v.reshape(*lead, K // h, h // (2 * step), 2, step)
        top = v[..., 0, :].copy()
        bot = v[..., 1, :].copy()
        v[..., 0, :] = top + bot
        v[..., 1, :] = top - bot
        step *= 2
    return v.reshape(*lead, K)


def rotate_rows(W: np.ndarray, rht_sign: np.ndarray, h: int) -> np.ndarray:
    """W_rot = W Q with Q = diag(s) blockdiag(H_h) / sqrt(h), row by row."""
    Ws = np.asarray(W, dtype=np.float64) * rht_sign.astype(np.float64)[None, :]
    return _fwht_last(Ws, h) / np.sqrt(h)


def _kmeans(blocks: np.ndarray, sens: np.ndarray, k: int, iters: int,
            rng: np.random.Generator):
    """Weighted Lloyd iterations on the rows of ``blocks`` (n x D); ``sens``
    (n x D) weighs each coordinate's squared error.  Returns centroids,
    assignments and the objective after each assignment step."""
    n = blocks.shape[0]
    cent = blocks[rng.choice(n, size=k, replace=n < k)].copy()
    hist: List[float] = []
    assign = np.zeros(n, dtype=np.int64)
    for _ in range(iters):
        # weighted distance sum_t w_t (v_t - c_t)^2, in chunks of rows
        for a in range(0, n, 8192):
            v, w = blocks[a:a + 8192], sens[a:a + 8192]
            d = (w[:, None, :] * (v[:, None, :] - cent[None, :, :]) ** 2).sum(axis=2)
            assign[a:a + 8192] = d.argmin(axis=1)
        err = (sens * (blocks - cent[assign]) ** 2).sum()
        hist.append(float(err))
        # weighted means; an empty centroid keeps its place
        num = np.zeros_like(cent)
        den = np.zeros_like(cent)
        np.add.at(num, assign, sens * blocks)
        np.add.at(den, assign, sens)
        filled = den > 0
        cent[filled] = num[filled] / den[filled]
    return cent, assign, hist


def quantize_rotated_residual(W: np.ndarray, *, seed: int = 0, iters: int = 12,
                              sensitivity: Optional[np.ndarray] = None, group: int = 128,
                              d: int = 4, k: int = 256) -> Quantized:
    """Quantize W [N][K] to the 3.125-bit format (d = 4, k = 256, group = 128)."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if d != 4 or k != 256 or group != 128:
        raise ValueError("the decode kernels take d = 4, 256 centroids and groups of 128")
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    rht_sign = np.where(rng.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)
    h = K & (-K)
    W_rot = rotate_rows(W, rht_sign, h)

    blocks = W_rot.reshape(N * (K // d), d)
    sens = (np.ones_like(blocks) if sensitivity is None
            else np.asarray(sensitivity, dtype=np.float64).reshape(N * (K // d), d))
    cent, assign, hist = _kmeans(blocks, sens, k, iters, rng)

    # the decode reads the codebook in fp16: each block takes its nearest fp16
    # centroid, and the residual is taken against it
    wc = cent.astype(np.float16)
    wc64 = wc.astype(np.float64)
    for a in range(0, blocks.shape[0], 8192):
        v, w = blocks[a:a + 8192], sens[a:a + 8192]
        assign[a:a + 8192] = (w[:, None, :] * (v[:, None, :] - wc64[None, :, :]) ** 2).sum(axis=2).argmin(axis=1)
    approx = wc64[assign].reshape(N, K)
    residual = W_rot - approx
    sign_bits = (residual >= 0).astype(np.uint8)
    sw = sens.reshape(N, K)
    g_abs = (sw * np.abs(residual)).reshape(N, K // group, group).sum(axis=2)
    g_w = sw.reshape(N, K // group, group).sum(axis=2)
    alpha = (g_abs / np.maximum(g_w, 1e-300)).astype(np.float16)
    return Quantized(wc=wc, idx=assign.reshape(N, K // d).astype(np.uint8), sign_bits=sign_bits,
                     alpha=alpha, rht_sign=rht_sign, had_block=h, group=group, objective=hist)
