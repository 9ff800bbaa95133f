"""Pins of the float64 oracle against facts fixed outside the oracle itself:
hand-packed vectors, hand-worked examples, brute-force dequantize-then-GEMV
in plain Python loops, closed forms and the Walsh-function definition of the
Hadamard matrix.  No GPU.

Passages: EVA explainer, technical summary section 2.A (output codebook and
lookup reformulation of the VQ GEMV); edge-LUT article, section details
(rotation, sign residual with per-group scale, dense sign packing).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- packing
def test_pack_hand_vectors():
    for case in _load("pack_vectors.json")["cases"]:
        got = o.pack_bits(np.array(case["values"]), case["nbits"])
        assert got.tobytes().hex() == case["bytes_hex"], case["note"]
        back = o.unpack_bits(np.frombuffer(bytes.fromhex(case["bytes_hex"]), np.uint8),
                             len(case["values"]), case["nbits"])
        assert list(back) == case["values"]


@pytest.mark.parametrize("nbits", list(range(1, 17)))
def test_pack_roundtrip_and_size(nbits):
    rng = np.random.default_rng(100 + nbits)
    for count in (0, 1, 7, 8, 9, 1000, 4099):
        v = rng.integers(0, 1 << nbits, size=count)
        p = o.pack_bits(v, nbits) if count else np.zeros(0, np.uint8)
        assert p.size == (count * nbits + 7) // 8
        assert np.array_equal(o.unpack_bits(p, count, nbits), v)


def test_pack_bit_positions_by_definition():
    # value t, bit i sits in stream bit q = n*t + i, i.e. bit q%8 of byte q//8
    rng = np.random.default_rng(5)
    for nbits in (1, 3, 8, 12, 16):
        v = rng.integers(0, 1 << nbits, size=37)
        p = o.pack_bits(v, nbits)
        for t in range(v.size):
            for i in range(nbits):
                q = nbits * t + i
                assert ((p[q // 8] >> (q % 8)) & 1) == ((int(v[t]) >> i) & 1)


def test_pack_rows_rows_start_on_bytes():
    rng = np.random.default_rng(3)
    m = rng.integers(0, 4096, size=(5, 6))          # 6 * 12 bits = 9 bytes
    p = o.pack_rows(m, 12)
    assert p.shape == (5, 9)
    for r in range(5):
        assert np.array_equal(p[r], o.pack_bits(m[r], 12))
    assert np.array_equal(o.unpack_rows(p, 5, 6, 12), m)


def test_uint16_indices_are_little_endian_words():
    rng = np.random.default_rng(4)
    v = rng.integers(0, 1 << 16, size=64).astype(np.uint16)
    assert o.pack_bits(v, 16).tobytes() == v.astype("<u2").tobytes()


def test_8bit_indices_are_plain_bytes():
    v = np.arange(256, dtype=np.uint8)
    assert o.pack_bits(v, 8).tobytes() == v.tobytes()


# ---------------------------------------------------------- OC and lookup
def test_hand_worked_vq_example():
    g = _load("tiny_vq_example.json")
    x = np.array([g["x"]])
    oc = o.output_codebook(x, np.array(g["wc"]), g["d"])
    assert np.array_equal(oc[0], np.array(g["oc"]))
    y = o.lookup_sum(oc, np.array(g["wi"]))
    assert np.array_equal(y[0], np.array(g["y"]))
    # the dequantized matrix printed by hand gives the same y
    assert np.array_equal(np.array(g["w_hat"]) @ np.array(g["x"]), np.array(g["y"]))


def test_oc_entries_by_scalar_loop():
    rng = np.random.default_rng(11)
    for d, nb in ((4, 3), (8, 2), (1, 4), (2, 5)):
        B, J = 3, 5
        x = rng.standard_normal((B, J * d))
        wc = rng.standard_normal((1 << nb, d))
        oc = o.output_codebook(x, wc, d)
        assert oc.shape == (B, J, 1 << nb)
        for b in range(B):
            for j in range(J):
                for c in range(1 << nb):
                    s = 0.0
                    for t in range(d):
                        s += float(x[b, j * d + t]) * float(wc[c, t])
                    assert abs(oc[b, j, c] - s) <= 1e-12 * (1 + abs(s))


def _brute_force_y(x, wc, idx, d):
    """Dequantize W_hat[r, j*d+t] = WC[idx[r, j], t] then dense y = W_hat x,
    in plain Python loops."""
    B, K = x.shape
    N, J = idx.shape
    y = [[0.0] * N for _ in range(B)]
    for r in range(N):
        w_row = [0.0] * K
        for j in range(J):
            for t in range(d):
                w_row[j * d + t] = float(wc[int(idx[r, j]), t])
        for b in range(B):
            acc = 0.0
            for k in range(K):
                acc += w_row[k] * float(x[b, k])
            y[b][r] = acc
    return np.array(y)


@pytest.mark.parametrize("K,N,d,nb,B", [(16, 5, 4, 3, 1), (64, 16, 4, 6, 1),
                                         (32, 9, 8, 4, 2), (48, 7, 2, 5, 3),
                                         (64, 16, 4, 8, 1), (24, 3, 1, 6, 1)])
def test_gemv_equals_bruteforce_dequant(K, N, d, nb, B):
    rng = np.random.default_rng(K * 131 + N)
    J = K // d
    x = rng.standard_normal((B, K))
    wc = rng.standard_normal((1 << nb, d))
    idx = rng.integers(0, 1 << nb, size=(N, J))
    y_bf = _brute_force_y(x, wc, idx, d)
    if (J * nb) % 8 == 0:
        y = o.vq_gemv(x, wc, o.pack_rows(idx, nb), N, K, d, nb)
    else:
        y = o.lookup_sum(o.output_codebook(x, wc, d), idx)
    scale = np.abs(y_bf).max() + 1.0
    assert np.max(np.abs(y - y_bf)) <= 1e-12 * scale


def test_exhaustive_two_subvectors_two_bits():
    # N=1, J=2, n=2: all 16 index pairs
    rng = np.random.default_rng(21)
    d = 3
    x = rng.standard_normal((1, 2 * d))
    wc = rng.standard_normal((4, d))
    for a, b in itertools.product(range(4), range(4)):
        idx = np.array([[a, b]])
        y = o.lookup_sum(o.output_codebook(x, wc, d), idx)[0, 0]
        want = float(np.dot(x[0, :d], wc[a]) + np.dot(x[0, d:], wc[b]))
        assert abs(y - want) <= 1e-13 * (1 + abs(want))


def test_constant_index_closed_form():
    rng = np.random.default_rng(8)
    K, N, d, nb = 64, 4, 4, 8
    x = rng.standard_normal((1, K))
    wc = rng.standard_normal((1 << nb, d))
    c = 77
    idx = np.full((N, K // d), c)
    y = o.vq_gemv(x, wc, o.pack_rows(idx, nb), N, K, d, nb)
    want = x[0].reshape(-1, d).sum(axis=0) @ wc[c]
    assert np.allclose(y, want, rtol=0, atol=1e-12)


def test_one_hot_input_reads_a_weight_column():
    # x = e_k -> y[r] = W_hat[r, k] = WC[idx[r, k // d], k % d]
    rng = np.random.default_rng(9)
    K, N, d, nb = 32, 6, 4, 8
    wc = rng.standard_normal((1 << nb, d))
    idx = rng.integers(0, 1 << nb, size=(N, K // d))
    packed = o.pack_rows(idx, nb)
    for k in (0, 1, 3, 4, 17, 31):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y = o.vq_gemv(x, wc, packed, N, K, d, nb)[0]
        assert np.array_equal(y, wc[idx[:, k // d], k % d])


def test_scalar_quantization_special_case():
    # d=1: a scalar LUT GEMV, y[r] = sum_k levels[idx[r,k]] * x[k]
    rng = np.random.default_rng(10)
    K, N = 40, 5
    levels = rng.standard_normal((16, 1))
    idx = rng.integers(0, 16, size=(N, K))
    x = rng.standard_normal((1, K))
    y = o.vq_gemv(x, levels, o.pack_rows(idx, 4), N, K, 1, 4)[0]
    assert np.allclose(y, levels[idx, 0] @ x[0], rtol=0, atol=1e-12)


def test_fp16_inputs_decode_exactly():
    rng = np.random.default_rng(12)
    x16 = rng.standard_normal((1, 64)).astype(np.float16)
    wc16 = (0.02 * rng.standard_normal((256, 4))).astype(np.float16)
    idx = rng.integers(0, 256, size=(8, 16))
    y = o.vq_gemv(x16, wc16, o.pack_rows(idx, 8), 8, 64, 4, 8)
    y_bf = _brute_force_y(x16.astype(np.float64), wc16.astype(np.float64), idx, 4)
    assert np.max(np.abs(y - y_bf)) <= 1e-15 * 64


def test_chunked_oc_matches_single_chunk(monkeypatch):
    rng = np.random.default_rng(13)
    K, N, d, nb, B = 256, 10, 8, 16, 2
    x = rng.standard_normal((B, K))
    wc = rng.standard_normal((1 << nb, d))
    idx = rng.integers(0, 1 << nb, size=(N, K // d))
    packed = o.pack_rows(idx, nb)
    y_ref = _brute_force_y(x, wc, idx, d)
    monkeypatch.setattr(o.vq, "_oc_chunk_cols", lambda B, n, budget_bytes=0: 3)
    y3 = o.vq_gemv(x, wc, packed, N, K, d, nb)
    assert np.max(np.abs(y3 - y_ref)) <= 1e-12 * (1 + np.abs(y_ref).max())


# ---------------------------------------------------------------- Hadamard
def test_hadamard_matches_walsh_definition():
    # H[i, j] = (-1)^popcount(i & j) for the Sylvester order
    for h in (1, 2, 4, 8, 32, 256):
        H = o.sylvester_hadamard(h)
        ii, jj = np.meshgrid(np.arange(h), np.arange(h), indexing="ij")
        pop = np.vectorize(lambda v: bin(int(v)).count("1"))(ii & jj)
        assert np.array_equal(H, np.where(pop % 2 == 0, 1, -1))


def test_hadamard_textbook_h4():
    H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    assert np.array_equal(o.sylvester_hadamard(4), H4)


@pytest.mark.parametrize("h", [2 ** k for k in range(12)])
def test_hadamard_orthogonal(h):
    H = o.sylvester_hadamard(h).astype(np.float64)   # integer sums < 2^53: exact
    assert np.array_equal(H @ H.T, h * np.eye(h))


def test_rht_hand_worked_and_norm():
    g = _load("tiny_residual_example.json")
    xr = o.rht(np.array([g["x"]]), np.array(g["rht_sign"]), g["had_block"])
    assert np.allclose(xr[0] * 2.0, g["x_rot_times_2"], rtol=0, atol=1e-13)
    rng = np.random.default_rng(14)
    for K, h in ((3584, 512), (14336, 2048), (64, 64)):
        x = rng.standard_normal((2, K))
        s = np.where(rng.integers(0, 2, K) == 1, 1, -1)
        xr = o.rht(x, s, h)
        assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1),
                           rtol=1e-12, atol=0)


def test_rht_one_hot_and_involution():
    K, h = 32, 8
    rng = np.random.default_rng(15)
    s = np.where(rng.integers(0, 2, K) == 1, 1, -1)
    H = o.sylvester_hadamard(h)
    for k in (0, 5, 9, 31):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        xr = o.rht(e, s, h)[0]
        blk = k // h
        want = np.zeros(K)
        want[blk * h:(blk + 1) * h] = s[k] * H[:, k % h] / math.sqrt(h)
        assert np.allclose(xr, want, rtol=0, atol=1e-15)
    x = rng.standard_normal((1, K))
    ones = np.ones(K)
    assert np.allclose(o.rht(o.rht(x, ones, h), ones, h), x, rtol=0, atol=1e-13)


def test_rht_rotation_preserves_product():
    # x_rot = R x with R orthogonal, so rotating W offline by R^T keeps W x
    rng = np.random.default_rng(16)
    K, N, h = 64, 5, 16
    s = np.where(rng.integers(0, 2, K) == 1, 1, -1)
    R = o.rht(np.eye(K), s, h).T            # column k = rht(e_k)
    assert np.allclose(R @ R.T, np.eye(K), atol=1e-12)
    x = rng.standard_normal((1, K))
    assert np.allclose(R @ x[0], o.rht(x, s, h)[0], atol=1e-12)
    W = rng.standard_normal((N, K))
    assert np.allclose((W @ R.T) @ o.rht(x, s, h)[0], W @ x[0], atol=1e-12)


# ---------------------------------------------------------------- residual
def test_residual_hand_worked():
    g = _load("tiny_residual_example.json")
    xr = o.rht(np.array([g["x"]]), np.array(g["rht_sign"]), g["had_block"])
    sp = o.pack_rows(np.array(g["sign_bits"]), 1)
    assert [r.tobytes().hex() for r in sp] == g["signs_packed_hex"]
    res = o.residual_term(xr, sp, np.array(g["alpha"]), 3, g["K"], g["group"])
    assert np.allclose(res[0] * 2.0, g["residual_times_2"], rtol=0, atol=1e-12)


def test_residual_bruteforce_dense():
    rng = np.random.default_rng(17)
    K, N, G, B = 256, 6, 128, 2
    bits = rng.integers(0, 2, size=(N, K))
    alpha = rng.uniform(0.001, 0.01, size=(N, K // G))
    xr = rng.standard_normal((B, K))
    res = o.residual_term(xr, o.pack_rows(bits, 1), alpha, N, K, G)
    want = np.zeros((B, N))
    for b in range(B):
        for r in range(N):
            acc = 0.0
            for k in range(K):
                w = alpha[r, k // G] * (1.0 if bits[r, k] else -1.0)
                acc += w * xr[b, k]
            want[b, r] = acc
    assert np.max(np.abs(res - want)) <= 1e-13


def test_residual_all_ones_closed_form():
    rng = np.random.default_rng(18)
    K, N, G = 512, 3, 128
    xr = rng.standard_normal((1, K))
    a = 0.0037
    bits = np.ones((N, K), dtype=np.int64)
    res = o.residual_term(xr, o.pack_rows(bits, 1), np.full((N, K // G), a), N, K, G)
    assert np.allclose(res, a * xr.sum(), rtol=1e-13, atol=0)
    res0 = o.residual_term(xr, o.pack_rows(0 * bits, 1), np.full((N, K // G), a), N, K, G)
    assert np.allclose(res0, -a * xr.sum(), rtol=1e-13, atol=0)


def test_gemv_residual_composes_parts():
    rng = np.random.default_rng(19)
    K, N, d, nb, G = 256, 8, 4, 8, 128
    x = rng.standard_normal((1, K)).astype(np.float16)
    wc = (0.02 * rng.standard_normal((256, d))).astype(np.float16)
    idx = rng.integers(0, 256, size=(N, K // d))
    bits = rng.integers(0, 2, size=(N, K))
    alpha = rng.uniform(0.001, 0.01, size=(N, K // G)).astype(np.float16)
    s = np.where(rng.integers(0, 2, K) == 1, 1, -1)
    y = o.vq_gemv_residual(x, wc, o.pack_rows(idx, nb), o.pack_rows(bits, 1), alpha,
                           s, 256, N, K, d, nb, G)
    xr = o.rht(x, s, 256)
    w_hat = np.zeros((N, K))
    for r in range(N):
        for j in range(K // d):
            w_hat[r, j * d:(j + 1) * d] = wc[idx[r, j]]
        w_hat[r] += np.repeat(alpha[r].astype(np.float64), G) * np.where(bits[r] == 1, 1.0, -1.0)
    assert np.allclose(y[0], w_hat @ xr[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- budgets
def test_bit_budgets():
    # 2 bits per weight at d=4, n=8; 3.125 = 2 (VQ) + 1 (sign) + 16/128 (alpha)
    import synth
    assert synth.weight_bytes(2) == 4 * (4096 * 1024 + 2048)
    K, N = 3584, 14336
    per = K * N * 2 // 8 + K * N // 8 + K * N // 128 * 2
    assert per * 8 / (K * N) == 3.125
    assert synth.weight_bytes(5) == 2 * (per + 2048) == 2 * 20072448
    assert 16 / 3.125 == 5.12            # the edge-LUT page's stated ratio is the bit ratio
    # OC build multiplies vs dense: K*2^n vs N*K -> 1 - 256/3584 = 92.9 %
    assert abs((1 - 256 / 3584) - 0.929) < 1e-3


def test_compare_metrics():
    y_ref = np.array([3.0, 4.0])
    rel, mx, rms = o.compare(np.array([3.0, 4.5]), y_ref)
    assert abs(rel - 0.1) < 1e-15 and mx == 0.5 and abs(rms - math.sqrt(12.5)) < 1e-15


def test_dequant_form_matches_lookup_form_and_a_loop():
    # the two definitions agree (reassociation of one sum), and the dequant
    # form agrees with an explicit triple loop on a tiny case
    rng = np.random.default_rng(31)
    for (K, N, d, nb, B) in [(16, 5, 4, 2, 1), (32, 7, 8, 6, 3), (64, 9, 4, 12, 2), (32, 4, 8, 16, 2)]:
        J = K // d
        x = rng.standard_normal((B, K)).astype(np.float16)
        wc = rng.normal(0, 0.02, size=(1 << nb, d)).astype(np.float16)
        idx = rng.integers(0, 1 << nb, size=(N, J))
        packed = o.pack_rows(idx, nb)
        a = o.dequant_gemv(x, wc, packed, N, K, d, nb)
        b = o.vq_gemv(x, wc, packed, N, K, d, nb)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    x = np.array([[1.0, -2.0, 0.5, 4.0]], dtype=np.float16)
    wc = np.array([[0.25, 1.0], [-0.5, 2.0], [1.5, -1.0], [0.0, 0.75]], dtype=np.float16)
    idx = np.array([[2, 1], [0, 3], [3, 3]])
    y = o.dequant_gemv(x, wc, o.pack_rows(idx, 4), 3, 4, 2, 4)
    ref = np.zeros((1, 3))
    for r in range(3):
        for j in range(2):
            for t in range(2):
                ref[0, r] += float(x[0, 2 * j + t]) * float(wc[idx[r, j], t])
    assert np.array_equal(y, ref)


def test_silu_gating_closed_forms():
    # silu(0) = 0; silu(1) = 1 / (1 + 1/e); silu(z) - silu(-z) = z; silu(z)
    # tends to z for large z and to 0 for very negative z; u scales linearly
    e = np.e
    g = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 40.0, -800.0])
    u = np.array([3.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0])
    y = o.silu_gated(g, u)
    assert y[0] == 0.0
    assert abs(y[1] - 1.0 / (1.0 + 1.0 / e)) < 1e-15
    assert abs(y[2] - (-1.0 / (1.0 + e))) < 1e-15
    assert abs((y[3] - y[4]) - 2.5) < 1e-14
    assert abs(y[5] - 40.0) < 1e-12
    assert y[6] == 0.0 or abs(y[6]) < 1e-300
    assert np.allclose(o.silu_gated(g[:6], 2.0 * u[:6]), 2.0 * y[:6], rtol=0, atol=1e-15)
