"""GPU parity of the large-codebook formats against the float64 CPU oracle:
12-bit indices (d=4, 4096 centroids, one token) and 16-bit indices (d=8,
65536 centroids, up to 16 tokens).

Bars: device layouts bit-exact; outputs within relative L2 2e-3 and max
error 1e-2 * rms(y) per matrix; repeated calls bitwise identical.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import synth  # noqa: E402
import vector_quantized_decode_amd as vq  # noqa: E402

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _assert_close(y, y_ref, what):
    rel, mx, rms = oracle.compare(y, y_ref)
    _say(f"{what}: rel_l2={rel:.3e} max_err={mx:.3e} rms={rms:.3e}")
    assert rel <= oracle.REL_L2_TOL, what
    assert mx <= oracle.MAX_ERR_RMS_TOL * rms, what


# ------------------------------------------------------------------ layouts
def _host_wi12(idx, N, J):
    """tile-16x64-12: chunk (rg, jt), lane l: 24 bytes holding the indices of
    rows 16 rg + i at subvector 64 jt + l, index i at bits [12 i, 12 i + 12)."""
    NG, JT = (N + 15) // 16, J // 64
    out = np.zeros((NG, JT, 64, 24), dtype=np.uint8)
    pad = np.zeros((NG * 16, J), dtype=np.int64)
    pad[:N] = idx
    for rg in range(NG):
        for j in range(J):
            v = 0
            for i in range(16):
                v |= int(pad[rg * 16 + i, j]) << (12 * i)
            out[rg, j // 64, j % 64] = np.frombuffer(v.to_bytes(24, "little"), dtype=np.uint8)
    return out.reshape(-1)


def _host_wi16(idx, N, J):
    """tile-16x32-16: chunk (rg, jb), lane l: 8 uint16, the q-th of row
    16 rg + l%16 at subvector 32 jb + l/16 + 4 q."""
    NG, JB = (N + 15) // 16, J // 32
    pad = np.zeros((NG * 16, J), dtype=np.uint16)
    pad[:N] = idx
    out = np.zeros((NG, JB, 64, 8), dtype=np.uint16)
    for l in range(64):
        for q in range(8):
            out[:, :, l, q] = pad.reshape(NG, 16, JB, 32)[:, l % 16, :, l // 16 + 4 * q]
    return out.reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 256), (100, 512), (33, 1024)])
def test_repack_wi12_bitexact(N, K):
    _say(f"repack 12-bit N={N} K={K}")
    rng = np.random.default_rng(N * K)
    J = K // 4
    idx = rng.integers(0, 4096, size=(N, J))
    canon = torch.from_numpy(oracle.pack_rows(idx, 12).reshape(-1)).to(DEV)
    dev = torch.full((vq.vq_wi_device_bytes(N, K, 4, 12),), 0xA5, dtype=torch.uint8, device=DEV)
    vq.vq_repack_wi(canon, N, K, 4, 12, dev)
    torch.cuda.synchronize()
    assert np.array_equal(dev.cpu().numpy(), _host_wi12(idx, N, J))


@pytest.mark.parametrize("N,K", [(16, 256), (100, 512), (40, 2048)])
def test_repack_wi16_bitexact(N, K):
    _say(f"repack 16-bit N={N} K={K}")
    rng = np.random.default_rng(N + K)
    J = K // 8
    idx = rng.integers(0, 65536, size=(N, J)).astype(np.uint16)
    canon = torch.from_numpy(oracle.pack_rows(idx, 16).reshape(-1)).to(DEV)
    dev = torch.full((vq.vq_wi_device_bytes(N, K, 8, 16),), 0xA5, dtype=torch.uint8, device=DEV)
    vq.vq_repack_wi(canon, N, K, 8, 16, dev)
    torch.cuda.synchronize()
    assert np.array_equal(dev.cpu().numpy().view(np.uint16), _host_wi16(idx, N, J))


@pytest.mark.parametrize("d,nbits", [(8, 16), (4, 8), (4, 12)])
def test_repack_wc_bitexact(d, nbits):
    # (8, 16): dimension-major, element t * 65536 + c = WC[c][t]; the other
    # formats keep the canonical layout
    _say(f"repack codebook d={d} n={nbits}")
    rng = np.random.default_rng(d * 100 + nbits)
    wc = rng.integers(0, 65536, size=(1 << nbits, d), dtype=np.uint16)
    dev = torch.full((vq.vq_wc_device_bytes(d, nbits) // 2,), 0x5A5A, dtype=torch.int16, device=DEV)
    vq.vq_repack_wc(torch.from_numpy(wc.view(np.int16)).to(DEV), d, nbits, dev)
    torch.cuda.synchronize()
    want = wc.T.reshape(-1) if (d, nbits) == (8, 16) else wc.reshape(-1)
    assert np.array_equal(dev.cpu().numpy().view(np.uint16), want)


# ------------------------------------------------------------------ GEMV
def _run(mats, xs, B):
    ys = [torch.full((B, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    ws = vq.alloc_workspace(mats, B, device=DEV)
    xt = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in xs]
    vq.vq_gemv(mats, xt, B, ys, ws, ws.numel())
    torch.cuda.synchronize()
    out = [y.cpu().numpy() for y in ys]
    vq.vq_gemv(mats, xt, B, ys, ws, ws.numel())           # again: bitwise identical
    torch.cuda.synchronize()
    for a, y in zip(out, ys):
        assert np.array_equal(a.view(np.uint32), y.cpu().numpy().view(np.uint32))
    return out


def _up(mi):
    return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, device=DEV)


@pytest.mark.parametrize("K,N", [(256, 1), (256, 40), (1024, 100), (4096, 333), (11008, 64),
                                 (16384, 50), (6400, 17)])
def test_gemv_12bit_shapes(K, N):
    _say(f"gemv 12-bit K={K} N={N}")
    mi = synth.small_matrix(K, N, 4, 12, seed=K + 3 * N)
    (y,) = _run([_up(mi)], [mi.x], 1)
    ref = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx, 12), N, K, 4, 12)
    _assert_close(y, ref, f"12-bit K={K} N={N}")


@pytest.mark.parametrize("K,N,B", [(256, 20, 1), (256, 16, 16), (512, 100, 3), (2048, 33, 16), (3072, 40, 16),
                                   (5120, 24, 2),
                                   (1024, 7, 5)])
def test_gemv_16bit_shapes(K, N, B):
    _say(f"gemv 16-bit K={K} N={N} B={B}")
    mi = synth.small_matrix(K, N, 8, 16, B=B, seed=K + N + B)
    (y,) = _run([_up(mi)], [mi.x], B)
    ref = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx, 16), N, K, 8, 16)
    _assert_close(y, ref, f"16-bit K={K} N={N} B={B}")


def test_gemv_16bit_mixed_group_flat_grid():
    # the 16-bit lookup kernel takes a flat grid of the call's workgroups and
    # each workgroup finds its matrix by a scan; a group of eight matrices of
    # different row lengths (splits of 1, 2, 3, 5, 10 and 16 waves, so
    # some workgroups leave waves without rows), tiny and ragged row counts,
    # and in an order the launcher sorts: every row against the oracle and
    # each matrix bitwise its result alone
    shapes = [(256, 1), (5120, 37), (13824, 100), (2048, 16), (1024, 333), (30720, 20),
              (65536, 17), (8192, 700)]
    _say(f"gemv 16-bit mixed group of {len(shapes)}")
    mis = [synth.small_matrix(K, N, 8, 16, B=5, seed=900 + i) for i, (K, N) in enumerate(shapes)]
    mats = [_up(mi) for mi in mis]
    ys = _run(mats, [mi.x for mi in mis], 5)
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _dequant_rows(mi), f"16-bit group matrix {i} K={mi.K} N={mi.N}")
    for i in (0, 2, 6):
        (y1,) = _run([mats[i]], [mis[i].x], 5)
        assert np.array_equal(y1.view(np.uint32), ys[i].view(np.uint32)), f"matrix {i} alone"


@pytest.mark.parametrize("d,nbits,B", [(4, 8, 1), (4, 8, 4), (4, 12, 1), (8, 16, 1), (8, 16, 16)])
def test_gemv_longest_supported_rows(d, nbits, B):
    # K = 65536, the longest row each 16-bit call takes (16 waves x 16 blocks
    # of 32 subvectors); the 8- and 12-bit kernels stream it
    K, N = 65536, 24
    _say(f"gemv K={K} N={N} d={d} n={nbits} B={B}")
    mi = synth.small_matrix(K, N, d, nbits, B=B, seed=4242 + nbits + B)
    (y,) = _run([_up(mi)], [mi.x], B)
    # the dequantize-then-GEMV form (pinned equal to the lookup form by the
    # oracle tests): the lookup form would build a 65536-column codebook
    # product for every subvector
    ref = oracle.dequant_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx, nbits), N, K, d, nbits)
    _assert_close(y, ref, f"K={K} d={d} n={nbits} B={B}")


def _dequant_rows(mi, chunk=1024):
    """The dequantize-then-GEMV definition over every row, in row chunks so
    the dense float64 weights stay small (pinned equal to the lookup form by
    the oracle tests)."""
    packed = oracle.pack_rows(mi.idx, mi.nbits)
    out = [oracle.dequant_gemv(mi.x, mi.wc, packed[r0:r0 + chunk], min(chunk, mi.N - r0), mi.K,
                               mi.d, mi.nbits) for r0 in range(0, mi.N, chunk)]
    return np.concatenate(out, axis=1)


def test_gemv_workload3_grouped():
    # the seven LLaMA-7B decoder linears at 3 bits/weight in one launch, the
    # launch bench.py times; every row of every matrix against the oracle's
    # output-codebook form (the tolerance is per matrix over all outputs)
    _say("gemv workload 3 (7 linears, 12-bit, one launch)")
    wl = synth.workload(3)
    mis = [synth.matrix_inputs(3, m) for m in range(wl.count)]
    ys = _run([_up(mi) for mi in mis], [mi.x for mi in mis], 1)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        ref = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx, 12), mi.N, mi.K, 4, 12)
        _assert_close(y, ref, f"workload3 matrix {m} ({wl.matrices[m].name})")


def test_gemv_workload4_grouped():
    # LLaMA-13B-shaped batched decode, 16 tokens with 5% outlier channels,
    # 65536 centroids of dimension 8, in the launch bench.py times: all
    # 16 x N outputs of every matrix against the dequantize-then-GEMV
    # definition
    _say("gemv workload 4 (3 matrices, 16-bit, B=16, one launch)")
    wl = synth.workload(4)
    mis = [synth.matrix_inputs(4, m) for m in range(wl.count)]
    ys = _run([_up(mi) for mi in mis], [mi.x for mi in mis], wl.B)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _dequant_rows(mi), f"workload4 matrix {m} ({wl.matrices[m].name})")
    # one matrix also through the output-codebook form of the oracle, on a few rows
    mi, y = mis[0], ys[0]
    rows = np.arange(0, mi.N, 640)
    ref = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx[rows], 16), rows.size, mi.K, 8, 16)
    _assert_close(y[:, rows], ref, "workload4 matrix 0 via OC")
