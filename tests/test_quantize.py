"""The offline 3.125-bit quantizer (host, numpy) against the decode's definition.

Pins: its rotation is the decode's (W_rot x_rot = W x with x_rot from the
oracle), its outputs decode through the oracle to exactly the dense product of
their own reconstruction, K-means never increases its objective, the residual
and its per-group scale reduce the error, and the scale is the group optimum.
"""
import numpy as np
import pytest

import oracle
from vector_quantized_decode_amd import quantize as qz


def _weights(N=48, K=512, seed=3):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02
    W[:, rng.choice(K, 8, replace=False)] *= 15.0          # outlier input channels
    return W


def _reconstruct_rot(q, N, K):
    approx = q.wc.astype(np.float64)[q.idx.astype(np.int64)].reshape(N, K)
    s = np.where(q.sign_bits == 1, 1.0, -1.0)
    a = np.repeat(q.alpha.astype(np.float64), q.group, axis=1)
    return approx, approx + a * s


def test_rotation_is_the_decodes():
    W = _weights()
    K = W.shape[1]
    rng = np.random.default_rng(5)
    s = np.where(rng.integers(0, 2, K) == 1, 1, -1).astype(np.int8)
    x = rng.standard_normal((2, K))
    for h in (1, 2, 64, 512):
        x_rot = oracle.rht(x, s, h)
        W_rot = qz.rotate_rows(W, s, h)
        assert np.allclose(x_rot @ W_rot.T, x @ W.T, rtol=0, atol=1e-12)


def test_quantized_outputs_decode_to_their_reconstruction():
    N, K = 48, 512
    W = _weights(N, K)
    q = qz.quantize_rotated_residual(W, seed=1, iters=6)
    assert q.wc.shape == (256, 4) and q.wc.dtype == np.float16
    assert q.idx.shape == (N, K // 4) and q.idx.dtype == np.uint8
    assert q.sign_bits.shape == (N, K) and set(np.unique(q.sign_bits)) <= {0, 1}
    assert q.alpha.shape == (N, K // 128) and q.had_block == 512
    x = np.random.default_rng(9).standard_normal((1, K)).astype(np.float16)
    y = oracle.vq_gemv_residual(x, q.wc, oracle.pack_rows(q.idx, 8), oracle.pack_rows(q.sign_bits, 1),
                                q.alpha, q.rht_sign, q.had_block, N, K, 4, 8, 128)
    _, full = _reconstruct_rot(q, N, K)
    x_rot = oracle.rht(x.astype(np.float64), q.rht_sign, q.had_block)
    assert np.allclose(y, x_rot @ full.T, rtol=1e-12, atol=1e-12)
    # and it approximates W x (3.125 bits per weight)
    ref = x.astype(np.float64) @ W.T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.5


def test_kmeans_objective_never_increases():
    q = qz.quantize_rotated_residual(_weights(64, 256, seed=4), seed=2, iters=10)
    h = np.array(q.objective)
    assert len(h) == 10 and np.all(np.diff(h) <= 1e-9 * h[0])


def test_residual_and_its_scale_reduce_the_error():
    N, K = 32, 512
    W = _weights(N, K, seed=6)
    q = qz.quantize_rotated_residual(W, seed=3, iters=6)
    W_rot = qz.rotate_rows(W, q.rht_sign, q.had_block)
    approx, full = _reconstruct_rot(q, N, K)
    e_vq = np.linalg.norm(W_rot - approx)
    e_res = np.linalg.norm(W_rot - full)
    assert e_res < e_vq
    # the scale is the group optimum: scaling any group's alpha up or down
    # (computed in float64 here) does not lower that group's error
    R = W_rot - approx
    s = np.where(q.sign_bits == 1, 1.0, -1.0)
    for r, g in [(0, 0), (5, 3), (31, 2)]:
        sl = slice(128 * g, 128 * g + 128)
        a = np.abs(R[r, sl]).mean()
        best = np.sum((R[r, sl] - a * s[r, sl]) ** 2)
        for f in (0.9, 1.1):
            assert np.sum((R[r, sl] - f * a * s[r, sl]) ** 2) > best
        assert abs(float(q.alpha[r, g]) - a) <= 1e-3 * a


def test_sensitivity_weights_the_fit():
    # with all sensitivity on one column of every block, that coordinate is
    # fitted better than without weighting
    N, K = 32, 256
    W = _weights(N, K, seed=8)
    sens = np.full((N, K), 1e-3)
    sens[:, 0::4] = 1.0
    q1 = qz.quantize_rotated_residual(W, seed=4, iters=8)
    q2 = qz.quantize_rotated_residual(W, seed=4, iters=8, sensitivity=sens)
    W_rot = qz.rotate_rows(W, q1.rht_sign, q1.had_block)
    e1 = np.linalg.norm((W_rot - _reconstruct_rot(q1, N, K)[0])[:, 0::4])
    e2 = np.linalg.norm((W_rot - _reconstruct_rot(q2, N, K)[0])[:, 0::4])
    assert e2 < e1


def test_rejects_other_formats():
    with pytest.raises(ValueError):
        qz.quantize_rotated_residual(np.zeros((4, 200)))
    with pytest.raises(ValueError):
        qz.quantize_rotated_residual(np.zeros((4, 256)), d=8)
