"""Plain float64 CPU oracle of the VQ decode hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use this module.  It shares no code with the HIP library.

Sources (cited by page title and section):

  [EVA]  "EVA: Accelerating LLM Decoding via an Efficient Vector Quantization
         Architecture" -- explainer page, technical summary: section 1 (the
         problem), section 2.A (algorithmic reformulation: input-codebook
         inner products, conflict-free lookup), section 2.B (epilogue unit,
         weight-stationary tiling).
  [EDGE] "Replacing MatMul with SRAM lookup: a 3-bit edge inference
         architecture" -- article page, section details: the 3.125-bit
         quantization pipeline sketch (Hadamard rotation, blocks of 4, K-means
         codebook of 256, residual signs, one fp16 scale per group of 128,
         dense sign packing) and the LUT-inference paragraph.

What the path computes.  A weight matrix W (N x K) is stored as a codebook WC
of 2^n centroids of dimension d and an index matrix WI (N x K/d) [EVA 2.A].
The decode output is y = W_hat x where W_hat[r, j*d + t] = WC[WI[r, j], t].
EVA reaches the same y by (a) splitting x into K/d contiguous subvectors and
multiplying them with the codebook, giving the output codebook
OC[j, c] = <x_j, WC[c]>, then (b) y[r] = sum_j OC[j, WI[r, j]] [EVA 2.A].
The reformulation is a reassociation of the same sum, so the plain
definition is exact up to rounding; this oracle computes (a) and (b)
literally, in float64.  [EDGE] adds, before the lookup, a randomized Hadamard
rotation of x (the weights were rotated offline) and after it a 1-bit
residual: y[r] += sum_g alpha[r, g] * sum_{k in g} s[r, k] * x_rot[k], with
s = +-1 from the packed sign bits and one alpha per group of 128 weights.

Readings where the pages are silent (each is tested by the pins in
``tests/test_oracle_*.py``):
  * subvector j is x[j*d : (j+1)*d] (contiguous along K);
  * OC row for token b, subvector j is b*(K/d) + j; column is the centroid;
  * WI is [N][K/d] row-major; n-bit indices are a little-endian bit stream,
    index t in stream bits [n*t, n*t + n), each row starting on a byte;
  * sign bit 1 means +1, weight k of a row is bit (k mod 8) of byte k // 8;
  * residual group g covers weights [128 g, 128 g + 128) of a row;
  * rotation: x_rot = blockdiag(H_h, ..., H_h) (s * x) / sqrt(h) with H_h the
    Sylvester Hadamard matrix and h the largest power of two dividing K;
    both the lookup and the residual use x_rot.

Parity status: every function here is pinned by an independent check
(brute-force dequantize-then-GEMV, closed forms, hand-packed vectors,
Hadamard identities).  The pages print no numeric example, so no end-to-end
output value is pinned to the pages themselves.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "pack_bits", "unpack_bits", "pack_rows", "unpack_rows",
    "sylvester_hadamard", "rht", "output_codebook", "lookup_sum",
    "vq_gemv", "dequant_gemv", "residual_term", "vq_gemv_residual", "silu_gated", "compare",
    "within_tolerance", "REL_L2_TOL", "MAX_ERR_RMS_TOL",
]

# acceptance bar for float outputs against this oracle
REL_L2_TOL = 2e-3
MAX_ERR_RMS_TOL = 1e-2


# --------------------------------------------------------------------------
# index / sign packing  [EVA 2.A: WI holds n-bit indices; EDGE: signs are
# packed densely into bytes]
# --------------------------------------------------------------------------
def pack_bits(values: np.ndarray, nbits: int) -> np.ndarray:
    """Pack unsigned ``values`` (each < 2^nbits) into a little-endian bit
    stream: value t occupies stream bits [nbits*t, nbits*t + nbits), stream
    bit q is bit (q mod 8) of byte q // 8.  Returns ceil(count*nbits/8) bytes.
    """
    v = np.asarray(values, dtype=np.int64).reshape(-1)
    if not 1 <= nbits <= 32:
        raise ValueError("nbits out of range")
    if v.size and (v.min() < 0 or v.max() >= (1 << nbits)):
        raise ValueError("value does not fit in nbits")
    shifts = np.arange(nbits, dtype=np.int64)[None, :]
    out = []
    step = 1 << 20                     # values per chunk; a multiple of 8
    for i in range(0, max(v.size, 1), step):
        bits = ((v[i:i + step, None] >> shifts) & 1).astype(np.uint8)
        out.append(bits.reshape(-1))
    return np.packbits(np.concatenate(out), bitorder="little")


def unpack_bits(packed: np.ndarray, count: int, nbits: int) -> np.ndarray:
    """Inverse of :func:`pack_bits`: the first ``count`` values (int64)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    need = (count * nbits + 7) // 8
    if p.size < need:
        raise ValueError("packed buffer too short")
    weights = (np.int64(1) << np.arange(nbits, dtype=np.int64))
    out = np.empty(count, dtype=np.int64)
    step = 1 << 20                     # values per chunk; a multiple of 8
    for i in range(0, count, step):
        c = min(step, count - i)
        b0, b1 = i * nbits // 8, ((i + c) * nbits + 7) // 8
        bits = np.unpackbits(p[b0:b1], bitorder="little")[: c * nbits]
        out[i:i + c] = bits.reshape(c, nbits).astype(np.int64) @ weights
    return out


def pack_rows(mat: np.ndarray, nbits: int) -> np.ndarray:
    """Pack a [rows][cols] matrix row by row (each row starts on a byte)."""
    m = np.asarray(mat)
    rows, cols = m.shape
    if (cols * nbits) % 8:
        raise ValueError("a packed row must be a whole number of bytes")
    return np.stack([pack_bits(m[r], nbits) for r in range(rows)]) if rows else \
        np.zeros((0, cols * nbits // 8), np.uint8)


def unpack_rows(packed: np.ndarray, rows: int, cols: int, nbits: int) -> np.ndarray:
    """Inverse of :func:`pack_rows` -> int64 [rows][cols]."""
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, -1)
    rb = cols * nbits // 8
    if p.shape[1] != rb:
        raise ValueError("row byte count mismatch")
    flat = unpack_bits(p.reshape(-1), rows * cols, nbits)
    return flat.reshape(rows, cols)


# --------------------------------------------------------------------------
# randomized Hadamard rotation  [EDGE: section details, rotation of the
# weights by a randomized Hadamard transform before quantization; the input
# is rotated the same way at inference so that W_rot x_rot = W x]
# --------------------------------------------------------------------------
def sylvester_hadamard(h: int) -> np.ndarray:
    """Dense +-1 Sylvester matrix of order h (power of two), by the doubling
    recursion H_2m = [[H_m, H_m], [H_m, -H_m]], H_1 = [1]."""
    if h < 1 or h & (h - 1):
        raise ValueError("Hadamard order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < h:
        H = np.block([[H, H], [H, -H]])
    return H


def rht(x: np.ndarray, sign: np.ndarray, had_block: int) -> np.ndarray:
    """x_rot[b] = blockdiag(H_h, ...) (sign * x[b]) / sqrt(h), float64 [B][K]."""
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B, K = xf.shape
    h = int(had_block)
    if K % h:
        raise ValueError("had_block must divide K")
    s = np.asarray(sign, dtype=np.float64).reshape(K)
    H = sylvester_hadamard(h).astype(np.float64)
    xs = (xf * s[None, :]).reshape(B, K // h, h)
    # block i of the output is H_h applied to block i of the signed input
    out = np.einsum("pq,bnq->bnp", H, xs)
    return out.reshape(B, K) / math.sqrt(h)


# --------------------------------------------------------------------------
# output codebook and lookup  [EVA 2.A]
# --------------------------------------------------------------------------
def output_codebook(x: np.ndarray, wc: np.ndarray, d: int) -> np.ndarray:
    """OC[b, j, c] = sum_t x[b, j*d + t] * WC[c, t]  (float64 [B][K/d][2^n]).

    The input is reshaped into K/d contiguous subvectors of length d and each
    is multiplied with every centroid: the (B*K/d x d) by (d x 2^n) product.
    """
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B, K = xf.shape
    if K % d:
        raise ValueError("K must be a multiple of d")
    w = np.asarray(wc, dtype=np.float64)
    if w.shape[1] != d:
        raise ValueError("codebook dimension differs from d")
    X = xf.reshape(B, K // d, d)
    return X @ w.T


def lookup_sum(oc: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """y[b, r] = sum_j OC[b, j, idx[r, j]]  (float64 [B][N])."""
    B, J, _ = oc.shape
    ii = np.asarray(idx, dtype=np.int64)
    if ii.shape[1] != J:
        raise ValueError("index matrix width differs from K/d")
    jj = np.arange(J)[None, :]
    return np.stack([oc[b][jj, ii].sum(axis=1) for b in range(B)])


def _oc_chunk_cols(B: int, ncent: int, budget_bytes: int = 256 << 20) -> int:
    return max(1, budget_bytes // (8 * B * ncent))


def vq_gemv(x: np.ndarray, wc: np.ndarray, wi_packed: np.ndarray, N: int,
            K: int, d: int, nbits: int) -> np.ndarray:
    """y = sum_j OC[j, WI[r, j]] for a canonical packed WI ([N] rows of
    K/d n-bit indices).  Returns float64 [B][N].

    The OC is formed in column chunks of subvectors so that the B=16,
    65536-centroid case stays within a few hundred MB; chunking changes only
    the order of the float64 additions.
    """
    J = K // d
    idx = unpack_rows(wi_packed, N, J, nbits)
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B = xf.shape[0]
    y = np.zeros((B, N), dtype=np.float64)
    step = _oc_chunk_cols(B, 1 << nbits)
    for j0 in range(0, J, step):
        j1 = min(J, j0 + step)
        oc = output_codebook(xf[:, j0 * d:j1 * d], wc, d)
        y += lookup_sum(oc, idx[:, j0:j1])
    return y


def dequant_gemv(x: np.ndarray, wc: np.ndarray, wi_packed: np.ndarray, N: int,
                 K: int, d: int, nbits: int) -> np.ndarray:
    """The plain definition the lookup form reassociates: dequantize the
    weights, W_hat[r, j*d + t] = WC[WI[r, j], t], then y = X W_hat^T
    [EVA 1, 2.A].  float64 [B][N].  Cheap for a few rows of a matrix whose
    output codebook would be huge (2^n >> N)."""
    J = K // d
    idx = unpack_rows(wi_packed, N, J, nbits)
    w = np.asarray(wc, dtype=np.float64)
    w_hat = w[idx].reshape(N, K)
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return xf @ w_hat.T


# --------------------------------------------------------------------------
# 1-bit residual  [EDGE: section details -- sign of the residual, one fp16
# scale per group of 128 weights, signs packed into bytes; at inference the
# residual needs only pointer references and bit operations]
# --------------------------------------------------------------------------
def residual_term(x_rot: np.ndarray, signs_packed: np.ndarray,
                  alpha: np.ndarray, N: int, K: int, group: int) -> np.ndarray:
    """sum_g alpha[r, g] * sum_{k in group g} s[r, k] * x_rot[b, k],
    s = +1 for a set bit, -1 for a clear bit.  float64 [B][N]."""
    xr = np.atleast_2d(np.asarray(x_rot, dtype=np.float64))
    B = xr.shape[0]
    if K % group:
        raise ValueError("group must divide K")
    bits = unpack_rows(signs_packed, N, K, 1)
    s = np.where(bits == 1, 1.0, -1.0)                      # [N][K]
    G = K // group
    a = np.asarray(alpha, dtype=np.float64).reshape(N, G)
    sg = s.reshape(N, G, group)
    xg = xr.reshape(B, G, group)
    per_group = np.einsum("ngk,bgk->bng", sg, xg)           # [B][N][G]
    return np.einsum("bng,ng->bn", per_group, a)


def vq_gemv_residual(x: np.ndarray, wc: np.ndarray, wi_packed: np.ndarray,
                     signs_packed: np.ndarray, alpha: np.ndarray,
                     rht_sign: Optional[np.ndarray], had_block: int, N: int,
                     K: int, d: int, nbits: int, group: int) -> np.ndarray:
    """Rotated VQ lookup plus 1-bit residual.  With ``rht_sign`` None the
    input is taken as already rotated."""
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    xr = xf if rht_sign is None else rht(xf, rht_sign, had_block)
    y = vq_gemv(xr, wc, wi_packed, N, K, d, nbits)
    return y + residual_term(xr, signs_packed, alpha, N, K, group)


def silu_gated(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u with silu(z) = z / (1 + exp(-z)): the gating of a SiLU-
    gated MLP (the LLaMA, Mixtral and Qwen3 models the EVA page evaluates)
    applied to the gate and up projections' outputs, in float64."""
    gf = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return gf / (1.0 + np.exp(-gf)) * np.asarray(u, dtype=np.float64)


# --------------------------------------------------------------------------
# comparison against the acceptance bar (per matrix, over all B*N outputs)
# --------------------------------------------------------------------------
def compare(y: np.ndarray, y_ref: np.ndarray) -> Tuple[float, float, float]:
    """(relative L2 error, max abs error, rms of the reference)."""
    a = np.asarray(y, dtype=np.float64).reshape(-1)
    b = np.asarray(y_ref, dtype=np.float64).reshape(-1)
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    nrm = float(np.linalg.norm(b))
    rel = float(np.linalg.norm(a - b)) / nrm if nrm > 0 else float(np.linalg.norm(a))
    mx = float(np.max(np.abs(a - b))) if a.size else 0.0
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    return rel, mx, rms


def within_tolerance(y: np.ndarray, y_ref: np.ndarray,
                     rel_tol: float = REL_L2_TOL,
                     max_rms_tol: float = MAX_ERR_RMS_TOL) -> bool:
    rel, mx, rms = compare(y, y_ref)
    return rel <= rel_tol and mx <= max_rms_tol * rms
