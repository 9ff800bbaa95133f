"""Seeded synthetic inputs: determinism, prefix draws, shapes and ranges."""
import hashlib

import numpy as np

import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes():
    a = synth.matrix_inputs(1, 0)
    b = synth.matrix_inputs(1, 0)
    for f in ("x", "wc", "idx"):
        assert _h(getattr(a, f)) == _h(getattr(b, f))


def test_seeds_per_workload_and_matrix():
    assert synth.seed_for(1, 0) == 0
    assert [synth.seed_for(2, m) for m in range(4)] == [2000, 2001, 2002, 2003]
    a = synth.matrix_inputs(2, 0, rows=8)
    b = synth.matrix_inputs(2, 1, rows=8)
    assert _h(a.idx) != _h(b.idx) and _h(a.wc) != _h(b.wc)


def test_row_prefix_equals_full_draw():
    full = synth.small_matrix(64, 40, 4, 12, residual=True)
    part = synth.small_matrix(64, 40, 4, 12, residual=True, rows=9)
    assert np.array_equal(full.idx[:9], part.idx)
    assert np.array_equal(full.sign_bits[:9], part.sign_bits)
    assert np.array_equal(full.alpha[:9], part.alpha)
    assert np.array_equal(full.x, part.x) and np.array_equal(full.wc, part.wc)


def test_shapes_and_ranges():
    m = synth.matrix_inputs(1, 0)
    assert m.x.shape == (1, 512) and m.x.dtype == np.float16
    assert m.wc.shape == (256, 4) and m.wc.dtype == np.float16
    assert m.idx.shape == (512, 128) and int(m.idx.max()) < 256
    assert abs(float(m.wc.astype(np.float64).std()) - 0.02) < 0.003
    w4 = synth.matrix_inputs(4, 0, rows=4)
    assert w4.x.shape == (16, 5120) and w4.wc.shape == (65536, 8)
    assert w4.outlier_channels.size == 256
    big = np.abs(w4.x[:, w4.outlier_channels].astype(np.float64)).mean()
    small = np.abs(np.delete(w4.x, w4.outlier_channels, axis=1).astype(np.float64)).mean()
    assert 15 < big / small < 25
    w5 = synth.matrix_inputs(5, 1, rows=4)
    assert w5.had_block == 2048 and w5.alpha.shape == (4, 112)
    assert set(np.unique(w5.rht_sign)) == {-1, 1}
    a = w5.alpha.astype(np.float64)
    assert a.min() >= 0.00099 and a.max() <= 0.01001
    assert synth.matrix_inputs(5, 0, rows=1).had_block == 512


def test_weight_bytes_per_layer():
    assert synth.weight_bytes(1) == 67584
    assert synth.weight_bytes(2) == 16785408
    assert synth.weight_bytes(3) == 76120064
    assert synth.weight_bytes(4) == 45088768
    assert synth.weight_bytes(5) == 40144896
    # MoE experts: 16 x (768 rows x 512 subvectors + 2 KiB), 8 x (2048 x 192 + 2 KiB)
    assert synth.weight_bytes(6) == 16 * (768 * 512 + 2048)
    assert synth.weight_bytes(7) == 8 * (2048 * 192 + 2048)
    assert synth.workload(6).count == 16 and synth.workload(7).count == 8
    assert synth.weight_bytes(8) == synth.weight_bytes(2) and synth.workload(8).B == 4
    assert synth.weight_bytes(9) == 2 * (11008 * 1024 + 2048) and synth.workload(9).gated_pairs
    assert synth.weight_bytes(10) == synth.weight_bytes(2) and synth.workload(10).B == 16
    # a codebook shared by q, k and v counts once
    assert synth.weight_bytes(11) == 4 * 4096 * 1024 + 2 * 2048


def test_shared_group_inputs():
    # members of a shared group take the first matrix's codebook and x and
    # keep indices of their own; matrices outside the group keep their own
    import numpy as np
    q, k, o = (synth.matrix_inputs(11, m, rows=4) for m in (0, 1, 3))
    assert synth.shared_leader(11, 2) == 0 and synth.shared_leader(11, 3) == 3
    assert np.array_equal(q.x, k.x) and np.array_equal(q.wc, k.wc)
    assert not np.array_equal(q.idx, k.idx)
    assert not np.array_equal(q.wc, o.wc) and not np.array_equal(q.x, o.x)
