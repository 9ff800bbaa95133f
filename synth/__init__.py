"""Seeded synthetic inputs for vector-quantized decode layers.

This module is shared by the CPU oracle and by the GPU path. It holds random
draws and the rounding of draws to fp16, nothing of the method's arithmetic:
no codebook product, no lookup, no packing, no rotation.

Workloads (matrix shapes follow LLaMA-7B / LLaMA-13B / Gemma-2-9B linears):

  1  one 512->512 matrix, d=4, n=8, B=1, seed 0
  2  four 4096->4096 matrices (q, k, v, o), d=4, n=8, B=1
  3  seven LLaMA-7B layer linears (q, k, v, o 4096->4096, gate/up 4096->11008,
     down 11008->4096), d=4, n=12, B=1
  4  5120->5120, 5120->13824, 13824->5120, d=8, n=16, B=16, 5% outlier
     input channels scaled by 20
  5  3584->14336, 14336->3584, d=4, n=8, B=1, plus randomized Hadamard
     rotation of x and a 1-bit sign residual with an fp16 scale per group of
     128 weights
  6  mixture-of-experts decode shaped like Qwen3-30B-A3B (hidden 2048, expert
     width 768, 8 routed experts per token): the gate and up projections of
     the 8 experts, 16 matrices 2048->768, each with its own codebook,
     d=4, n=8, B=1
  7  the same experts' down projections, 8 matrices 768->2048, d=4, n=8, B=1
  8  workload 2 for 4 tokens per call (batched or speculative decode), B=4
  9  LLaMA-7B MLP gate and up projections (2 x 4096->11008), d=4, n=8, B=1,
     called as one gate/up pair with the SiLU gating fused (both use the
     gate's x)
 10  workload 2 for 16 tokens per call, B=16
 11  workload 2 with one codebook shared by q, k and v, which also share
     their input x (the attention projections of one layer read the same
     hidden state); o keeps its own codebook and x

Distributions: x ~ N(0, 1), codebook ~ N(0, 0.02) (0.02 is the standard
deviation), indices uniform over [0, 2^n), residual sign bits Bernoulli(0.5),
alpha ~ U(0.001, 0.01), rotation diagonal uniform over {-1, +1}.  Every float
is drawn in float64 and rounded to fp16 with round-to-nearest-even.

Seeds: workload c, matrix m uses seed 1000*c + m, except workload 1 which uses
seed 0.  Each matrix spawns six independent PCG64 streams from that seed in
the fixed order x, codebook, indices, signs, alpha, rotation signs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = ["MatrixSpec", "Workload", "WORKLOADS", "workload", "matrix_inputs",
           "seed_for", "small_matrix", "shared_leader"]


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    K: int          # input features (length of x)
    N: int          # output features (rows of the index matrix)


@dataclass(frozen=True)
class Workload:
    number: int
    title: str
    d: int          # subvector / centroid dimension
    nbits: int      # index width n (2^n centroids)
    B: int          # tokens per call
    matrices: List[MatrixSpec]
    residual: bool = False      # rotation + 1-bit sign residual
    group: int = 128            # residual scale group (weights along K)
    outlier_frac: float = 0.0   # fraction of input channels scaled
    outlier_scale: float = 1.0
    gated_pairs: bool = False   # matrices 2i, 2i+1 are a gate/up pair (SiLU gating fused)
    shared: tuple = ()          # groups of matrices that share the first one's codebook and x

    @property
    def count(self) -> int:
        return len(self.matrices)


_LLAMA7B_ATTN = [MatrixSpec(n, 4096, 4096) for n in ("q", "k", "v", "o")]

WORKLOADS = {
    1: Workload(1, "single 512x512 VQ linear, 2 bits/weight", 4, 8, 1,
                [MatrixSpec("w", 512, 512)]),
    2: Workload(2, "LLaMA-7B attention projections q/k/v/o, 2 bits/weight",
                4, 8, 1, list(_LLAMA7B_ATTN)),
    3: Workload(3, "LLaMA-7B decoder-layer linears, 3 bits/weight", 4, 12, 1,
                list(_LLAMA7B_ATTN) + [MatrixSpec("gate", 4096, 11008),
                                       MatrixSpec("up", 4096, 11008),
                                       MatrixSpec("down", 11008, 4096)]),
    4: Workload(4, "LLaMA-13B-shaped batched decode, 16 tokens, 2 bits/weight",
                8, 16, 16, [MatrixSpec("attn", 5120, 5120),
                            MatrixSpec("up", 5120, 13824),
                            MatrixSpec("down", 13824, 5120)],
                outlier_frac=0.05, outlier_scale=20.0),
    5: Workload(5, "Gemma-2-9B-shaped rotated VQ + 1-bit residual, 3.125 bits/weight",
                4, 8, 1, [MatrixSpec("up", 3584, 14336),
                          MatrixSpec("down", 14336, 3584)],
                residual=True, group=128),
    6: Workload(6, "MoE decode (Qwen3-30B-A3B-shaped), gate+up of 8 routed experts, 2 bits/weight",
                4, 8, 1, [MatrixSpec(f"e{e}.{p}", 2048, 768) for e in range(8)
                          for p in ("gate", "up")]),
    7: Workload(7, "MoE decode (Qwen3-30B-A3B-shaped), down of 8 routed experts, 2 bits/weight",
                4, 8, 1, [MatrixSpec(f"e{e}.down", 768, 2048) for e in range(8)]),
    8: Workload(8, "LLaMA-7B attention projections q/k/v/o, 4 tokens, 2 bits/weight",
                4, 8, 4, list(_LLAMA7B_ATTN)),
    9: Workload(9, "LLaMA-7B MLP gate and up, SiLU gating fused, 2 bits/weight",
                4, 8, 1, [MatrixSpec("gate", 4096, 11008), MatrixSpec("up", 4096, 11008)],
                gated_pairs=True),
    10: Workload(10, "LLaMA-7B attention projections q/k/v/o, 16 tokens, 2 bits/weight",
                 4, 8, 16, list(_LLAMA7B_ATTN)),
    11: Workload(11, "LLaMA-7B attention projections, q/k/v sharing one codebook and x, "
                     "2 bits/weight", 4, 8, 1, list(_LLAMA7B_ATTN), shared=((0, 1, 2),)),
}


def workload(number: int) -> Workload:
    return WORKLOADS[number]


def seed_for(number: int, matrix: int) -> int:
    return 0 if number == 1 else 1000 * number + matrix


def _streams(seed: int):
    kids = np.random.SeedSequence(seed).spawn(6)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids]


def _fp16(a: np.ndarray) -> np.ndarray:
    # numpy's float64 -> float16 cast rounds to nearest, ties to even
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _largest_pow2_divisor(k: int) -> int:
    return k & (-k)


@dataclass
class MatrixInputs:
    """Unpacked inputs of one matrix.  Packed forms are made by each side."""
    K: int
    N: int
    d: int
    nbits: int
    B: int
    x: np.ndarray                    # float16 [B][K]
    wc: np.ndarray                   # float16 [2^n][d]
    idx: np.ndarray                  # uint16 (n<=16) [N][K/d], values < 2^n
    sign_bits: Optional[np.ndarray] = None   # uint8 {0,1} [N][K]; 1 means +1
    alpha: Optional[np.ndarray] = None       # float16 [N][K/group]
    rht_sign: Optional[np.ndarray] = None    # int8 {-1,+1} [K]
    had_block: int = 0
    group: int = 0
    outlier_channels: Optional[np.ndarray] = field(default=None)


def draw(K: int, N: int, d: int, nbits: int, B: int, seed: int, *,
         residual: bool = False, group: int = 128, outlier_frac: float = 0.0,
         outlier_scale: float = 1.0, had_block: Optional[int] = None,
         rows: Optional[int] = None) -> MatrixInputs:
    """Draw the inputs of one matrix from ``seed``.

    ``rows`` limits how many index rows are drawn (the first ``rows`` rows of
    the full draw, used for sampled checks at large N); the draw order makes
    those rows identical to the full draw's.
    """
    if K % d:
        raise ValueError("K must be a multiple of d")
    J = K // d
    s_x, s_wc, s_wi, s_sg, s_al, s_rh = _streams(seed)

    xf = s_x.standard_normal((B, K))
    outl = None
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        outl = np.sort(s_x.choice(K, size=n_out, replace=False))
        xf[:, outl] *= outlier_scale
    x = _fp16(xf)

    wc = _fp16(s_wc.normal(0.0, 0.02, size=(1 << nbits, d)))

    n_rows = N if rows is None else min(rows, N)
    # rows are drawn one after another, so a prefix of rows is a prefix draw
    idx = s_wi.integers(0, 1 << nbits, size=(n_rows, J), dtype=np.uint32)
    idx = idx.astype(np.uint16 if nbits <= 16 else np.uint32)

    out = MatrixInputs(K=K, N=N, d=d, nbits=nbits, B=B, x=x, wc=wc, idx=idx,
                       outlier_channels=outl)
    if residual:
        out.sign_bits = s_sg.integers(0, 2, size=(n_rows, K), dtype=np.uint8)
        out.alpha = _fp16(s_al.uniform(0.001, 0.01, size=(n_rows, K // group)))
        out.rht_sign = np.where(s_rh.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)
        out.had_block = had_block if had_block else _largest_pow2_divisor(K)
        out.group = group
    return out


def shared_leader(number: int, m: int) -> int:
    """The matrix whose codebook and x matrix ``m`` uses (``m`` itself unless
    it belongs to a shared group of the workload)."""
    for g in WORKLOADS[number].shared:
        if m in g:
            return g[0]
    return m


def matrix_inputs(number: int, m: int, rows: Optional[int] = None) -> MatrixInputs:
    """Inputs of matrix ``m`` of workload ``number`` (see module docstring).
    A member of a shared group draws its own indices and takes the group's
    first matrix's codebook and x."""
    w = WORKLOADS[number]
    spec = w.matrices[m]
    out = draw(spec.K, spec.N, w.d, w.nbits, w.B, seed_for(number, m),
               residual=w.residual, group=w.group,
               outlier_frac=w.outlier_frac, outlier_scale=w.outlier_scale,
               rows=rows)
    lead = shared_leader(number, m)
    if lead != m:
        ls = w.matrices[lead]
        src = draw(ls.K, ls.N, w.d, w.nbits, w.B, seed_for(number, lead), rows=1,
                   outlier_frac=w.outlier_frac, outlier_scale=w.outlier_scale)
        out.x, out.wc = src.x, src.wc
    return out


def small_matrix(K: int, N: int, d: int, nbits: int, B: int = 1, seed: int = 7,
                 **kw) -> MatrixInputs:
    """A small seeded matrix for parity tests (same distributions)."""
    return draw(K, N, d, nbits, B, seed, **kw)


def weight_bytes(number: int) -> int:
    """Algorithmic weight bytes of one layer of workload ``number``: packed
    indices + codebooks (+ packed signs + fp16 alpha)."""
    w = WORKLOADS[number]
    total = 0
    for m, s in enumerate(w.matrices):
        J = s.K // w.d
        total += (s.N * J * w.nbits + 7) // 8
        if shared_leader(number, m) == m:               # a shared codebook counts once
            total += (1 << w.nbits) * w.d * 2
        if w.residual:
            total += s.N * s.K // 8 + s.N * (s.K // w.group) * 2
    return total
