"""GPU parity tests: the HIP library (through its C ABI) against the float64
CPU oracle on the same seeded inputs.

Bars: packing, unpacking and device layouts bit-exact; float outputs within
relative L2 error 2e-3 and max error 1e-2 * rms(y) per matrix; the output
codebook within relative L2 error 1e-3.
"""
import os
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


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("nbits", [1, 3, 8, 12, 16])
@pytest.mark.parametrize("count", [1, 5, 8, 1001, 65536 + 3])
def test_pack_unpack_bitexact(nbits, count):
    _say(f"pack nbits={nbits} count={count}")
    rng = np.random.default_rng(nbits * 1000 + count)
    idx = rng.integers(0, 1 << nbits, size=count).astype(np.uint32)
    nbytes = (count * nbits + 7) // 8
    out = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    vq.vq_pack_indices(_i32(idx), count, nbits, out)
    back = torch.zeros(count, dtype=torch.int32, device=DEV)
    ref_packed = oracle.pack_bits(idx, nbits)
    vq.vq_unpack_indices(torch.from_numpy(ref_packed).to(DEV), count, nbits, back)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref_packed)
    assert np.array_equal(back.cpu().numpy().view(np.uint32), idx)


def test_pack_hand_vectors_on_gpu():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_vectors.json")))
    for case in g["cases"]:
        v = np.array(case["values"], dtype=np.uint32)
        out = torch.zeros((v.size * case["nbits"] + 7) // 8, dtype=torch.uint8, device=DEV)
        vq.vq_pack_indices(_i32(v), v.size, case["nbits"], out)
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes().hex() == case["bytes_hex"], case["note"]


def _host_wi_layout(canon, N, J):
    NG = (N + 15) // 16
    out = np.zeros((J // 64, NG, 64, 16), dtype=np.uint8)
    for r in range(N):
        for j in range(J):
            out[j // 64, r // 16, j % 64, r % 16] = canon[r, j]
    return out.reshape(-1)


def _host_sign_layout(canon, N, P):
    """chunk (tile pt, row pair rp), lane 2r + g: 16 sign bytes of row
    32 rp + r, byte j at position 32 pt + 16 g + (j ^ (r % 16))."""
    NP = (N + 31) // 32
    out = np.zeros((P // 32, NP, 32, 2, 16), dtype=np.uint8)
    for r in range(N):
        rr = r % 32
        for g in range(2):
            for j in range(16):
                out[:, r // 32, rr, g, j] = canon[r].reshape(P // 32, 32)[:, 16 * g + (j ^ (rr % 16))]
    return out.reshape(-1)


def _host_alpha_layout(canon, N, G):
    """chunk (group pair, row pair rp), lane 2r + g: the scale of row
    32 rp + r, group 2 (group pair) + g."""
    NP = (N + 31) // 32
    out = np.zeros((G // 2, NP, 32, 2), dtype=np.uint16)
    for r in range(N):
        for g in range(G):
            out[g // 2, r // 32, r % 32, g % 2] = canon[r, g]
    return out.reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 256), (100, 512), (33, 768)])
def test_repack_layouts_bitexact(N, K):
    _say(f"repack N={N} K={K}")
    rng = np.random.default_rng(N + K)
    J, P, G = K // 4, K // 8, K // 128
    canon = rng.integers(0, 256, size=(N, J), dtype=np.uint8)
    dev = torch.full((vq.vq_wi_device_bytes(N, K, 4, 8),), 0x5A, dtype=torch.uint8, device=DEV)
    vq.vq_repack_wi(torch.from_numpy(canon).to(DEV), N, K, 4, 8, dev)
    scanon = rng.integers(0, 256, size=(N, P), dtype=np.uint8)
    sdev = torch.full((vq.vq_signs_device_bytes(N, K),), 0x5A, dtype=torch.uint8, device=DEV)
    vq.vq_repack_signs(torch.from_numpy(scanon).to(DEV), N, K, sdev)
    acanon = rng.integers(0, 65536, size=(N, G), dtype=np.uint16)
    adev = torch.full((vq.vq_alpha_device_bytes(N, K, 128) // 2,), 7, dtype=torch.int16, device=DEV)
    vq.vq_repack_alpha(torch.from_numpy(acanon.view(np.int16)).to(DEV), N, K, 128, adev)
    torch.cuda.synchronize()
    assert np.array_equal(dev.cpu().numpy(), _host_wi_layout(canon, N, J))
    assert np.array_equal(sdev.cpu().numpy(), _host_sign_layout(scanon, N, P))
    body = _host_alpha_layout(acanon, N, G)
    got = adev.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:body.size], body)
    # header after the tiled scales: the largest fp16 magnitude, as bits
    assert got[body.size:body.size + 2].view(np.uint32)[0] == int((acanon & 0x7FFF).max())


# ------------------------------------------------------------------ OC build
@pytest.mark.parametrize("dtype", [vq.VQ_F32, vq.VQ_F16])
@pytest.mark.parametrize("cfg,m", [(1, 0), (2, 1), (5, 0)])
def test_build_oc_full(cfg, m, dtype):
    _say(f"build_oc workload={cfg} matrix={m} dtype={dtype}")
    mi = synth.matrix_inputs(cfg, m, rows=1)
    B, K, d, n = mi.B, mi.K, mi.d, mi.nbits
    J = K // d
    oc = torch.empty((B * J, 1 << n), dtype=torch.float32 if dtype == vq.VQ_F32 else torch.float16,
                     device=DEV)
    vq.vq_build_oc(torch.from_numpy(mi.x).to(DEV), B, K, d, n,
                   torch.from_numpy(mi.wc).to(DEV), oc, dtype)
    torch.cuda.synchronize()
    ref = oracle.output_codebook(mi.x, mi.wc, d).reshape(B * J, 1 << n)
    got = oc.float().cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _say(f"  rel_l2={rel:.3e}")
    assert rel <= 1e-3


def test_build_oc_sampled_16bit_codebook():
    # 16 tokens x 5120 inputs, d=8, n=16: OC is 10240 x 65536 (fp16, 1.34 GB)
    _say("build_oc workload=4 matrix=0 fp16 sampled rows")
    mi = synth.matrix_inputs(4, 0, rows=1)
    B, K, d, n = mi.B, mi.K, mi.d, mi.nbits
    J = K // d
    oc = torch.empty((B * J, 1 << n), dtype=torch.float16, device=DEV)
    vq.vq_build_oc(torch.from_numpy(mi.x).to(DEV), B, K, d, n,
                   torch.from_numpy(mi.wc).to(DEV), oc, vq.VQ_F16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(B * J, size=64, replace=False))
    got = oc[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    del oc
    xr = mi.x.astype(np.float64).reshape(B * J, d)[rows]
    ref = xr @ mi.wc.astype(np.float64).T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _say(f"  rel_l2={rel:.3e}")
    assert rel <= 1e-3


# ------------------------------------------------------------------ rotation
@pytest.mark.parametrize("K,h,B", [(3584, 512, 1), (14336, 2048, 1), (1024, 1024, 3), (256, 1, 1),
                                   (8192, 8192, 1)])
def test_rht_matches_oracle(K, h, B):
    _say(f"rht K={K} h={h} B={B}")
    rng = np.random.default_rng(K + h)
    x = rng.standard_normal((B, K)).astype(np.float16)
    s = np.where(rng.integers(0, 2, K) == 1, 1, -1).astype(np.int8)
    out = torch.empty((B, K), dtype=torch.float32, device=DEV)
    vq.vq_rht(torch.from_numpy(x).to(DEV), torch.from_numpy(s).to(DEV), B, K, h, out)
    torch.cuda.synchronize()
    ref = oracle.rht(x, s, h)
    err = np.abs(out.cpu().numpy() - ref).max()
    _say(f"  max_err={err:.3e}")
    assert err <= 1e-5 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------------ VQ GEMV
def _upload(mi, residual=False):
    if residual:
        return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits,
                                sign_bits=mi.sign_bits, alpha=mi.alpha, group=mi.group,
                                rht_sign=mi.rht_sign, had_block=mi.had_block, device=DEV)
    return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, device=DEV)


def _run_gemv(mats, xs, B=1, residual=False):
    ys = [torch.full((B, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    ws = vq.alloc_workspace(mats, B, residual=residual, device=DEV)
    xt = [torch.from_numpy(x).to(DEV) for x in xs]
    fn = vq.vq_gemv_residual if residual else vq.vq_gemv
    fn(mats, xt, B, ys, ws, ws.numel())
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], (mats, xt, ys, ws)


def _oracle_plain(mi, rows=None):
    idx = mi.idx if rows is None else mi.idx[rows]
    return oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(idx, mi.nbits), idx.shape[0], mi.K,
                          mi.d, mi.nbits)


def _oracle_res(mi, rows=None, rotate=True):
    sel = slice(None) if rows is None else rows
    idx, bits, alpha = mi.idx[sel], mi.sign_bits[sel], mi.alpha[sel]
    return oracle.vq_gemv_residual(mi.x, mi.wc, oracle.pack_rows(idx, 8),
                                   oracle.pack_rows(bits, 1), alpha,
                                   mi.rht_sign if rotate else None, mi.had_block,
                                   idx.shape[0], mi.K, mi.d, mi.nbits, mi.group)


def test_gemv_workload1_single_matrix():
    _say("gemv workload 1 (512x512)")
    mi = synth.matrix_inputs(1, 0)
    (y,), _ = _run_gemv([_upload(mi)], [mi.x])
    _assert_close(y, _oracle_plain(mi), "workload1")


@pytest.mark.parametrize("K,N", [(256, 1), (256, 17), (512, 100), (768, 333), (1024, 4103),
                                 (2048, 48), (4096, 513), (8192, 77), (8448, 50)])
def test_gemv_shapes_with_ragged_rows(K, N):
    _say(f"gemv K={K} N={N}")
    mi = synth.small_matrix(K, N, 4, 8, seed=K + N)
    (y,), _ = _run_gemv([_upload(mi)], [mi.x])
    _assert_close(y, _oracle_plain(mi), f"K={K} N={N}")


def test_gemv_workload2_grouped_and_deterministic():
    _say("gemv workload 2 (4 x 4096x4096, one launch)")
    mis = [synth.matrix_inputs(2, m) for m in range(4)]
    mats = [_upload(mi) for mi in mis]
    ys, keep = _run_gemv(mats, [mi.x for mi in mis])
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"workload2 matrix {m}")
    # bitwise reproducible, and the same per matrix whether grouped or not
    ys2, _ = _run_gemv(mats, [mi.x for mi in mis])
    for a, b in zip(ys, ys2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    (y1,), _ = _run_gemv([mats[2]], [mis[2].x])
    assert np.array_equal(y1.view(np.uint32), ys[2].view(np.uint32))


def test_gemv_long_rows_share_the_short_row_sums():
    # rows of more than 32 chunks of 64 subvectors are streamed; a short-row
    # matrix grouped with them is streamed too and must give bitwise the
    # result it gets alone (where all of its chunks are requested at once)
    _say("gemv long and short rows in one launch")
    mis = [synth.small_matrix(12288, 100, 4, 8, seed=21), synth.small_matrix(4096, 700, 4, 8, seed=22)]
    mats = [_upload(mi) for mi in mis]
    ys, _ = _run_gemv(mats, [mi.x for mi in mis])
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"long/short {i}")
    (y1,), _ = _run_gemv([mats[1]], [mis[1].x])
    assert np.array_equal(y1.view(np.uint32), ys[1].view(np.uint32))


def test_gemv_small_call_matches_its_grouped_sums():
    # alone, a 512 x 512 matrix is a call of few indices (4-wave workgroups);
    # grouped with a 4096 x 4096 matrix it takes the 8-wave burst kernel: the
    # same sums in the same order either way
    _say("gemv small matrix alone and in a group")
    mis = [synth.matrix_inputs(1, 0), synth.small_matrix(4096, 4096, 4, 8, seed=23)]
    mats = [_upload(mi) for mi in mis]
    ys, _ = _run_gemv(mats, [mi.x for mi in mis])
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"small/large {i}")
    (y0,), _ = _run_gemv([mats[0]], [mis[0].x])
    assert np.array_equal(y0.view(np.uint32), ys[0].view(np.uint32))


def test_gemv_largest_group():
    # VQ_MAX_GROUP matrices of mixed shapes in one launch, each checked against
    # the oracle and against its own single-matrix call
    _say("gemv 16 matrices in one launch")
    shapes = [(256, 7), (512, 300), (768, 64), (1024, 1000), (1280, 33), (2048, 515),
              (2304, 128), (4096, 256), (3072, 96), (512, 2049), (1536, 17), (256, 4000),
              (1024, 1), (2560, 200), (8192, 40), (9216, 24)]
    assert len(shapes) == vq.VQ_MAX_GROUP
    mis = [synth.small_matrix(K, N, 4, 8, seed=100 + i) for i, (K, N) in enumerate(shapes)]
    mats = [_upload(mi) for mi in mis]
    ys, _ = _run_gemv(mats, [mi.x for mi in mis])
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"group of 16, matrix {i}")
        (y1,), _ = _run_gemv([mats[i]], [mi.x])
        assert np.array_equal(y1.view(np.uint32), y.view(np.uint32)), f"matrix {i}"


@pytest.mark.parametrize("wl", [6, 7])
def test_gemv_moe_expert_groups(wl):
    # mixture-of-experts decode: the routed experts' projections (16 gate/up
    # matrices, or 8 down matrices), each with its own codebook, in one
    # launch; every matrix in full against the oracle, and grouped equal to
    # alone bitwise
    _say(f"gemv MoE expert group (workload {wl}) in one launch")
    w = synth.workload(wl)
    mis = [synth.matrix_inputs(wl, m) for m in range(w.count)]
    mats = [_upload(mi) for mi in mis]
    ys, _ = _run_gemv(mats, [mi.x for mi in mis])
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"workload {wl} matrix {i}")
    (y1,), _ = _run_gemv([mats[3]], [mis[3].x])
    assert np.array_equal(y1.view(np.uint32), ys[3].view(np.uint32))


@pytest.mark.parametrize("K,N,B", [(256, 17, 2), (1024, 333, 3), (2048, 1000, 4), (4096, 513, 2),
                                   (8192, 77, 4), (768, 2048, 3), (8448, 50, 2), (12288, 100, 3)])
def test_gemv_several_tokens(K, N, B):
    # 2 to 4 tokens per call: each codebook entry looked up once serves every
    # token; every token within tolerance, bitwise equal alone and grouped
    # (rows of more than 32 chunks are streamed, with their group)
    _say(f"gemv K={K} N={N} B={B}")
    mi = synth.small_matrix(K, N, 4, 8, B=B, seed=K + N + B)
    other = synth.small_matrix(1024, 700, 4, 8, B=B, seed=99)
    mats = [_upload(mi), _upload(other)]
    ys, _ = _run_gemv(mats, [mi.x, other.x], B=B)
    _assert_close(ys[0], _oracle_plain(mi), f"K={K} N={N} B={B}")
    _assert_close(ys[1], _oracle_plain(other), f"grouped companion B={B}")
    (y1,), _ = _run_gemv([mats[0]], [mi.x], B=B)
    assert np.array_equal(y1.view(np.uint32), ys[0].view(np.uint32))


def _dequant_all_rows(mi, chunk=1024):
    """Every row through the dequantize-then-GEMV definition (pinned equal to
    the lookup form by the oracle tests), in row chunks."""
    packed = oracle.pack_rows(mi.idx, mi.nbits)
    out = [oracle.dequant_gemv(mi.x, mi.wc, packed[r0:r0 + chunk], min(chunk, mi.N - r0), mi.K,
                               mi.d, mi.nbits) for r0 in range(0, mi.N, chunk)]
    return np.concatenate(out, axis=1)


def test_gemv_workload8_four_tokens():
    # LLaMA-7B q/k/v/o for 4 tokens in one launch, in the launch bench.py
    # times: all 4 x 4096 outputs of every matrix
    _say("gemv workload 8 (4 x 4096x4096, 4 tokens, one launch)")
    w = synth.workload(8)
    mis = [synth.matrix_inputs(8, m) for m in range(w.count)]
    ys, _ = _run_gemv([_upload(mi) for mi in mis], [mi.x for mi in mis], B=4)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _dequant_all_rows(mi), f"workload 8 matrix {m}")


def _upload_rows(mi):
    return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, tokens=True, device=DEV)


@pytest.mark.parametrize("N,K", [(1, 256), (17, 256), (1000, 1024), (4103, 512), (48, 16384)])
def test_repack_rows_bitexact(N, K):
    # row tiles against a host construction from the canonical indices
    _say(f"repack rows N={N} K={K}")
    rng = np.random.default_rng(N * 31 + K)
    J = K // 4
    idx = rng.integers(0, 256, size=(N, J), dtype=np.uint8)
    canon = torch.from_numpy(oracle.pack_rows(idx, 8)).to(DEV)
    dev = torch.full((vq.vq_wi_device_bytes(N, K, 4, 8),), 0xA5, dtype=torch.uint8, device=DEV)
    vq.vq_repack_wi_rows(canon, N, K, dev)
    torch.cuda.synchronize()
    NG = (N + 15) // 16
    pad = np.zeros((NG * 16, J), dtype=np.uint8)
    pad[:N] = idx
    # [column k][row group][lane l = 16 (l // 16) + l % 16 ... ] -> row 16 rg + l % 16, bytes 16 (l // 16)
    ref = pad.reshape(NG, 16, J // 64, 4, 16).transpose(2, 0, 3, 1, 4).reshape(-1)
    assert np.array_equal(dev.cpu().numpy(), ref)


def _run_tokens(mats, xs, B):
    ys = [torch.full((B, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    xt = [torch.from_numpy(x).to(DEV) for x in xs]
    vq.vq_gemv_tokens(mats, xt, B, ys)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


@pytest.mark.parametrize("K,N,B", [(256, 1, 16), (256, 17, 5), (512, 4103, 3), (1024, 333, 16),
                                   (2048, 64, 1), (4096, 700, 8), (4096, 1000, 13),
                                   (11008, 100, 16), (16384, 48, 16), (65536, 40, 16),
                                   (65536, 33, 3)])
def test_gemv_tokens_shapes(K, N, B):
    # 1 to 16 tokens on the matrix cores from row tiles: every
    # token within tolerance; ragged row tails, one to 256 columns of 64
    # subvectors per row (K = 65536: 32 columns per wave); bitwise equal
    # alone and grouped
    _say(f"gemv_tokens K={K} N={N} B={B}")
    mi = synth.small_matrix(K, N, 4, 8, B=B, seed=K + 3 * N + B)
    other = synth.small_matrix(2048, 1500, 4, 8, B=B, seed=98)
    mats = [_upload_rows(mi), _upload_rows(other)]
    ys = _run_tokens(mats, [mi.x, other.x], B)
    _assert_close(ys[0], _oracle_plain(mi), f"tokens K={K} N={N} B={B}")
    _assert_close(ys[1], _oracle_plain(other), f"tokens grouped companion B={B}")
    (y1,) = _run_tokens(mats[:1], [mi.x], B)
    assert np.array_equal(y1.view(np.uint32), ys[0].view(np.uint32))


@pytest.mark.parametrize("K,N,d,nbits,B", [(4096, 700, 4, 8, 1), (512, 17, 4, 8, 2),
                                           (12288, 100, 4, 8, 3), (1024, 300, 4, 12, 1),
                                           (1024, 100, 8, 16, 4)])
def test_gemv_f16_epilogue(K, N, d, nbits, B):
    # fp16 outputs: bitwise the fp32 call's sums rounded to nearest even (the
    # same kernels, burst and streaming 8-bit, 12- and 16-bit), and within
    # tolerance of the oracle
    _say(f"gemv_f16 K={K} N={N} d={d} n={nbits} B={B}")
    mi = synth.small_matrix(K, N, d, nbits, B=B, seed=K + N + 5 * B)
    m = _upload(mi)
    (y32,), (mats, xt, _, ws) = _run_gemv([m], [mi.x], B=B)
    y16 = torch.full((B, N), float("nan"), dtype=torch.float16, device=DEV)
    vq.vq_gemv_f16(mats, xt, B, [y16], ws, ws.numel())
    torch.cuda.synchronize()
    want = torch.from_numpy(y32).to(DEV).half()
    assert torch.equal(y16.view(torch.int16), want.view(torch.int16))
    _assert_close(y16.float().cpu().numpy(), _oracle_plain(mi), f"f16 K={K} N={N}")


def test_gemv_tokens_moe_expert_group():
    # 8 routed experts' gate and up matrices (16 x 2048 -> 768, MoE-shaped),
    # each with its own codebook and its own 8 tokens, in one launch
    _say("gemv_tokens MoE group: 16 x 2048x768, 8 tokens")
    mis = [synth.small_matrix(2048, 768, 4, 8, B=8, seed=700 + e) for e in range(16)]
    ys = _run_tokens([_upload_rows(mi) for mi in mis], [mi.x for mi in mis], 8)
    for e, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"expert matrix {e}")


def test_gemv_tokens_agrees_with_plain_call():
    # the same 4-token product through both 8-bit entry points, each within
    # tolerance of the oracle and of the other
    _say("gemv_tokens against vq_gemv, 4 tokens")
    mi = synth.small_matrix(4096, 2000, 4, 8, B=4, seed=4242)
    (yt,) = _run_tokens([_upload_rows(mi)], [mi.x], 4)
    (yp,), _ = _run_gemv([_upload(mi)], [mi.x], B=4)
    ref = _oracle_plain(mi)
    _assert_close(yt, ref, "tokens call")
    _assert_close(yp, ref, "plain call")
    _assert_close(yt, yp.astype(np.float64), "tokens against plain")


def test_gemv_tokens_workload8_four_tokens():
    # LLaMA-7B q/k/v/o for 4 tokens through the matrix-core call, the launch
    # bench.py times for 4 tokens: every output of every matrix
    _say("gemv_tokens workload 8 (4 x 4096x4096, 4 tokens, one launch)")
    w = synth.workload(8)
    mis = [synth.matrix_inputs(8, m) for m in range(w.count)]
    ys = _run_tokens([_upload_rows(mi) for mi in mis], [mi.x for mi in mis], 4)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _dequant_all_rows(mi), f"workload 8 (tokens) matrix {m}")


def test_gemv_workload10_sixteen_tokens():
    # LLaMA-7B q/k/v/o for 16 tokens in one launch, in the launch bench.py
    # times: all 16 x 4096 outputs of every matrix
    _say("gemv_tokens workload 10 (4 x 4096x4096, 16 tokens, one launch)")
    w = synth.workload(10)
    mis = [synth.matrix_inputs(10, m) for m in range(w.count)]
    ys = _run_tokens([_upload_rows(mi) for mi in mis], [mi.x for mi in mis], 16)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _dequant_all_rows(mi), f"workload 10 matrix {m}")


@pytest.mark.parametrize("K,N,B,pairs", [(256, 17, 1, 1), (1024, 333, 2, 2), (4096, 700, 1, 3),
                                         (2048, 768, 2, 4), (8192, 77, 1, 1)])
def test_gemv_swiglu_pairs(K, N, B, pairs):
    # silu(gate x) * (up x) for gate/up pairs sharing x, against the oracle's
    # two GEMVs and its gating
    _say(f"swiglu K={K} N={N} B={B} pairs={pairs}")
    gates = [synth.small_matrix(K, N, 4, 8, B=B, seed=500 + 2 * p) for p in range(pairs)]
    ups = [synth.small_matrix(K, N, 4, 8, B=B, seed=501 + 2 * p) for p in range(pairs)]
    xs = [torch.from_numpy(g.x).to(DEV) for g in gates]       # each pair uses its gate's x
    ys = [torch.full((B, N), float("nan"), dtype=torch.float32, device=DEV) for _ in range(pairs)]
    gm = [_upload(g) for g in gates]
    um = [_upload(u) for u in ups]
    ws = vq.alloc_workspace(gm, B, device=DEV)
    vq.vq_gemv_swiglu(gm, um, xs, B, ys, ws, ws.numel())
    torch.cuda.synchronize()
    for p, (g, u, y) in enumerate(zip(gates, ups, ys)):
        gy = oracle.vq_gemv(g.x, g.wc, oracle.pack_rows(g.idx, 8), N, K, 4, 8)
        uy = oracle.vq_gemv(g.x, u.wc, oracle.pack_rows(u.idx, 8), N, K, 4, 8)
        _assert_close(y.cpu().numpy(), oracle.silu_gated(gy, uy), f"swiglu pair {p}")


def test_gemv_swiglu_f16_epilogue():
    # fp16 gated products: bitwise the fp32 call's output rounded to nearest even
    _say("swiglu f16 K=4096 N=700 B=2 pairs=2")
    gates = [synth.small_matrix(4096, 700, 4, 8, B=2, seed=520 + 2 * p) for p in range(2)]
    ups = [synth.small_matrix(4096, 700, 4, 8, B=2, seed=521 + 2 * p) for p in range(2)]
    xs = [torch.from_numpy(g.x).to(DEV) for g in gates]
    gm = [_upload(g) for g in gates]
    um = [_upload(u) for u in ups]
    y32 = [torch.full((2, 700), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    y16 = [torch.full((2, 700), float("nan"), dtype=torch.float16, device=DEV) for _ in range(2)]
    ws = vq.alloc_workspace(gm, 2, device=DEV)
    vq.vq_gemv_swiglu(gm, um, xs, 2, y32, ws, ws.numel())
    vq.vq_gemv_swiglu_f16(gm, um, xs, 2, y16, ws, ws.numel())
    torch.cuda.synchronize()
    for p in range(2):
        assert torch.equal(y16[p].view(torch.int16), y32[p].half().view(torch.int16)), f"pair {p}"


@pytest.mark.parametrize("B", [1, 2, 4])
def test_gemv_shared_codebook_units(B):
    # vq_gemv_shared: matrices that pass the same codebook and x and have the
    # same shape are served as one unit (their row groups laid end to end,
    # one staged codebook per workgroup): each within tolerance of the
    # oracle and bitwise equal to its vq_gemv call alone; a same-shape matrix
    # with its own codebook, and one of another shape sharing the codebook,
    # stay apart
    _say(f"gemv shared-codebook units B={B}")
    base = synth.small_matrix(2048, 1000, 4, 8, B=B, seed=61)
    mis = [base] + [synth.small_matrix(2048, 1000, 4, 8, B=B, seed=62 + i) for i in range(2)]
    for mi in mis[1:]:
        mi.x, mi.wc = base.x, base.wc
    own = synth.small_matrix(2048, 1000, 4, 8, B=B, seed=70)
    other = synth.small_matrix(2048, 333, 4, 8, B=B, seed=71)
    other.x, other.wc = base.x, base.wc
    mats = [_upload(mi) for mi in mis] + [_upload(own), _upload(other)]
    for m in (mats[1], mats[2], mats[4]):
        m.wc = mats[0].wc
    x0 = torch.from_numpy(base.x).to(DEV)
    xt = [x0, x0, x0, torch.from_numpy(own.x).to(DEV), x0]
    ys = [torch.full((B, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    vq.vq_gemv_shared(mats, xt, B, ys)
    torch.cuda.synchronize()
    for i, (mi, y) in enumerate(zip(mis + [own, other], ys)):
        got = y.cpu().numpy()
        _assert_close(got, _oracle_plain(mi), f"shared unit matrix {i} B={B}")
        alone = torch.full((B, mi.N), float("nan"), dtype=torch.float32, device=DEV)
        vq.vq_gemv([mats[i]], [xt[i]], B, [alone], None, 0)
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy().view(np.uint32), got.view(np.uint32)), f"matrix {i}"


def test_gemv_workload11_shared_codebook():
    # LLaMA-7B q/k/v sharing one codebook and x with o alone: every row
    # against the oracle through vq_gemv (the launch bench.py times) and
    # through vq_gemv_shared (q/k/v one unit), both bitwise equal to the four
    # matrices called one by one
    _say("gemv workload 11 (q/k/v share a codebook and x)")
    w = synth.workload(11)
    mis = [synth.matrix_inputs(11, m) for m in range(w.count)]
    mats = [_upload(mi) for mi in mis]
    xt = [torch.from_numpy(mi.x).to(DEV) for mi in mis]
    for m in range(w.count):
        l = synth.shared_leader(11, m)
        if l != m:
            mats[m].wc, xt[m] = mats[l].wc, xt[l]
    ys = [torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    yu = [torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    vq.vq_gemv(mats, xt, 1, ys, None, 0)
    vq.vq_gemv_shared(mats, xt, 1, yu)
    torch.cuda.synchronize()
    for m, (mi, y, u) in enumerate(zip(mis, ys, yu)):
        got = y.cpu().numpy()
        _assert_close(got, _oracle_plain(mi), f"workload 11 matrix {m}")
        alone = torch.empty((1, mi.N), dtype=torch.float32, device=DEV)
        vq.vq_gemv([mats[m]], [xt[m]], 1, [alone], None, 0)
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy().view(np.uint32), got.view(np.uint32))
        assert np.array_equal(u.cpu().numpy().view(np.uint32), got.view(np.uint32))


def test_gemv_mixed_group():
    _say("gemv mixed shapes in one launch")
    mis = [synth.small_matrix(1024, 300, 4, 8, seed=1), synth.small_matrix(512, 2000, 4, 8, seed=2),
           synth.small_matrix(2304, 64, 4, 8, seed=3)]
    ys, _ = _run_gemv([_upload(mi) for mi in mis], [mi.x for mi in mis])
    for i, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_plain(mi), f"mixed {i}")


def test_plain_8bit_call_is_stateless():
    # the 8-bit plain kernels keep no state between calls (no workspace, no
    # counters): repeated calls give bitwise the first call's result
    _say("8-bit plain call repeated: bitwise identical, no state")
    mi = synth.small_matrix(2048, 1500, 4, 8, seed=9)
    m = _upload(mi)
    ys, (mats, xt, yt, ws) = _run_gemv([m], [mi.x])
    ref = _oracle_plain(mi)
    for _ in range(3):
        vq.vq_gemv(mats, xt, 1, yt, None, 0)
    torch.cuda.synchronize()
    _assert_close(yt[0].cpu().numpy(), ref, "after repeats")
    assert np.array_equal(yt[0].cpu().numpy().view(np.uint32), ys[0].view(np.uint32))


def test_workspace_shared_by_call_kinds_after_init():
    # one buffer serves a 16-bit call (which rewrites its codebook and x
    # planes from offset 0), then residual calls on two different groups of
    # matrices; each change of call kind or group is preceded by
    # vq_workspace_init, as the header requires, and repeated calls on one
    # group need none
    _say("workspace: 16-bit call, then residual groups A and B, one buffer")
    w16 = synth.small_matrix(2048, 300, 8, 16, B=4, seed=31)
    ra = [synth.small_matrix(3584, 700, 4, 8, seed=32, residual=True)]
    rb = [synth.small_matrix(1024, 2000, 4, 8, seed=33, residual=True),
          synth.small_matrix(4096, 90, 4, 8, seed=34, residual=True)]
    m16 = _upload(w16)
    ma = [_upload(mi, residual=True) for mi in ra]
    mb = [_upload(mi, residual=True) for mi in rb]
    need = max(vq.vq_workspace_bytes([m16], 4), vq.vq_workspace_bytes(ma, 1, residual=True),
               vq.vq_workspace_bytes(mb, 1, residual=True))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    vq.vq_workspace_init(ws, need)
    y16 = torch.empty((4, w16.N), dtype=torch.float32, device=DEV)
    vq.vq_gemv([m16], [torch.from_numpy(w16.x).to(DEV)], 4, [y16], ws, need)
    torch.cuda.synchronize()
    _assert_close(y16.cpu().numpy(), _oracle_plain(w16), "16-bit call")
    for tag, mats, mis in (("A", ma, ra), ("B", mb, rb), ("A again", ma, ra)):
        vq.vq_workspace_init(ws, need)                   # another call kind or group
        xs = [torch.from_numpy(mi.x).to(DEV) for mi in mis]
        for rep in range(2):                             # same group: no re-init needed
            ys = [torch.full((1, mi.N), float("nan"), dtype=torch.float32, device=DEV)
                  for mi in mis]
            vq.vq_gemv_residual(mats, xs, 1, ys, ws, need)
            torch.cuda.synchronize()
            for i, (mi, y) in enumerate(zip(mis, ys)):
                _assert_close(y.cpu().numpy(), _oracle_res(mi), f"residual group {tag} "
                              f"matrix {i} call {rep}")


# ------------------------------------------------------------------ residual
@pytest.mark.parametrize("K,N,rotate,h", [(256, 40, True, 0), (1024, 200, True, 0), (1024, 200, False, 0),
                                          (3584, 300, True, 0), (2048, 1031, True, 0), (768, 50, True, 0),
                                          (1024, 64, True, 64), (512, 33, True, 1), (1024, 96, True, 2),
                                          (4096, 80, True, 4096), (8192, 100, True, 8192),
                                          (1024, 3000, True, 0), (2048, 4500, True, 0),
                                          (20480, 64, True, 0), (33024, 64, True, 0)])
def test_gemv_residual_shapes(K, N, rotate, h):
    # h = 0: the largest power of two dividing K.  Blocks up to 2048 are
    # rotated inside the lookup kernel (h < 256: whole blocks per tile);
    # 4096 and 8192 go through the separate rotation kernel.  K = 20480 takes
    # the wider bound loads; above 127 splits (K = 33024) partial sums are
    # handed off in float.
    _say(f"gemv_residual K={K} N={N} rotate={rotate} h={h}")
    mi = synth.small_matrix(K, N, 4, 8, seed=K * 7 + N, residual=True, had_block=h or None)
    m = _upload(mi, residual=True)
    if not rotate:
        m.rht_sign = None
    (y,), _ = _run_gemv([m], [mi.x], residual=True)
    _assert_close(y, _oracle_res(mi, rotate=rotate), f"residual K={K} N={N}")


@pytest.mark.parametrize("K,N", [(4096, 9000), (20480, 6144)])
def test_gemv_residual_tall_sampled_rows(K, N):
    # tall layers take 2 and 4 row steps per wave (1024 and 2048 rows per
    # workgroup); K = 20480 also takes the wider bound loads
    _say(f"gemv_residual K={K} N={N}, sampled rows")
    mi = synth.small_matrix(K, N, 4, 8, seed=K + N, residual=True)
    (y,), _ = _run_gemv([_upload(mi, residual=True)], [mi.x], residual=True)
    rng = np.random.default_rng(K)
    rows = np.unique(np.concatenate([np.arange(64), rng.choice(N, 192, replace=False), np.arange(N - 64, N)]))
    _assert_close(y[:, rows], _oracle_res(mi, rows=rows), f"residual K={K} N={N} sampled")


def test_gemv_residual_workload5():
    # both Gemma-2-9B-shaped matrices in one launch, the launch bench.py
    # times: every row against the oracle (rotation, lookup sum, residual)
    _say("gemv_residual workload 5 (3584->14336, 14336->3584)")
    mis = [synth.matrix_inputs(5, m) for m in range(2)]
    mats = [_upload(mi, residual=True) for mi in mis]
    ys, _ = _run_gemv(mats, [mi.x for mi in mis], residual=True)
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle_res(mi), f"workload5 matrix {m}")


# ------------------------------------------------------------------ edge cases: magnitudes, zeros, non-finite inputs
def _scaled_matrix(K, N, seed, x_scale=1.0, wc_scale=1.0):
    mi = synth.small_matrix(K, N, 4, 8, seed=seed)
    mi.x = (mi.x.astype(np.float64) * x_scale).astype(np.float16)
    mi.wc = (mi.wc.astype(np.float64) * wc_scale).astype(np.float16)
    return mi


@pytest.mark.parametrize("x_scale,wc_scale", [(1000.0, 100.0), (1e-3, 1e-2), (60.0, 1.0)])
def test_gemv_across_magnitudes(x_scale, wc_scale):
    # K = 4096: the 8-bit kernel splits each row over four waves of one
    # workgroup whose fp32 segment sums meet in LDS; fp16 products with fp32
    # sums keep the relative accuracy at large and small magnitudes
    _say(f"gemv magnitudes x*{x_scale} wc*{wc_scale}")
    mi = _scaled_matrix(4096, 700, seed=21, x_scale=x_scale, wc_scale=wc_scale)
    (y,), _ = _run_gemv([_upload(mi)], [mi.x])
    _assert_close(y, _oracle_plain(mi), "scaled")


def test_gemv_zero_input_gives_exact_zero():
    _say("gemv x = 0")
    mi = synth.small_matrix(4096, 300, 4, 8, seed=22)
    mi.x = np.zeros_like(mi.x)
    (y,), _ = _run_gemv([_upload(mi)], [mi.x])
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("bad", ["inf", "nan"])
def test_gemv_nonfinite_input_propagates_like_oracle(bad):
    # a non-finite input flows through the fp32 products and sums of every
    # row that looks it up: the class of every output (NaN, +inf, -inf,
    # finite) matches the oracle's, and the next call on finite inputs is
    # unaffected (the plain kernels keep no state)
    _say(f"gemv non-finite input: {bad}")
    mi = synth.small_matrix(4096, 200, 4, 8, seed=23)
    x = mi.x.copy()
    x[0, 1234] = np.float16(np.inf if bad == "inf" else np.nan)
    mi.x = x
    (y,), _ = _run_gemv([_upload(mi)], [mi.x])
    with np.errstate(invalid="ignore", over="ignore"):
        ref = _oracle_plain(mi)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        _assert_close(y[fin], ref[fin], "finite rows")
    mi2 = synth.small_matrix(4096, 200, 4, 8, seed=24)
    (y2,), _ = _run_gemv([_upload(mi2)], [mi2.x])
    _assert_close(y2, _oracle_plain(mi2), "after non-finite call")


def test_gemv_residual_on_quantizer_output():
    # the offline quantizer's artifacts (non-uniform, K-means indices; signs
    # and scales of a real residual) decoded on the GPU against the oracle
    from vector_quantized_decode_amd import quantize
    _say("residual GEMV on quantizer output")
    N, K = 96, 1024
    rng = np.random.default_rng(12)
    W = rng.standard_normal((N, K)) * 0.02
    q = quantize.quantize_rotated_residual(W, seed=2, iters=6)
    x = rng.standard_normal((1, K)).astype(np.float16)
    m = vq.upload_matrix(q.idx, q.wc, K, N, 4, 8, sign_bits=q.sign_bits, alpha=q.alpha, group=128,
                         rht_sign=q.rht_sign, had_block=q.had_block, device=DEV)
    (y,), _ = _run_gemv([m], [x], residual=True)
    ref = oracle.vq_gemv_residual(x, q.wc, oracle.pack_rows(q.idx, 8), oracle.pack_rows(q.sign_bits, 1),
                                  q.alpha, q.rht_sign, q.had_block, N, K, 4, 8, 128)
    _assert_close(y, ref, "quantizer output")


def test_gemv_residual_zero_input_gives_exact_zero():
    # K = 3584 splits each row over 14 workgroups (fixed-point hand-off)
    _say("gemv_residual x = 0")
    mi = synth.small_matrix(3584, 300, 4, 8, seed=78, residual=True)
    mi.x = np.zeros_like(mi.x)
    (y,), _ = _run_gemv([_upload(mi, residual=True)], [mi.x], residual=True)
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("bad", ["inf", "nan"])
@pytest.mark.parametrize("rotate", [False, True])
def test_gemv_residual_nonfinite_input_propagates_like_oracle(bad, rotate):
    # a non-finite input makes the hand-off bound non-finite: float partials
    # and the last-workgroup sum instead; every output's class (NaN, +inf,
    # -inf, finite) matches the oracle, and the workspace is left ready
    _say(f"gemv_residual non-finite input: {bad}, rotate={rotate}")
    mi = synth.small_matrix(3584, 200, 4, 8, seed=79, residual=True)
    x = mi.x.copy()
    x[0, 1234] = np.float16(np.inf if bad == "inf" else np.nan)
    mi.x = x
    m = _upload(mi, residual=True)
    if not rotate:
        m.rht_sign = None
    (y,), _ = _run_gemv([m], [mi.x], residual=True)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = _oracle_res(mi, rotate=rotate)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        _assert_close(y[fin], ref[fin], "finite rows")
    mi2 = synth.small_matrix(3584, 200, 4, 8, seed=80, residual=True)
    (y2,), _ = _run_gemv([_upload(mi2, residual=True)], [mi2.x], residual=True)
    _assert_close(y2, _oracle_res(mi2), "after non-finite call")


def test_gemv_residual_large_magnitudes():
    _say("gemv_residual with large x and alpha")
    mi = synth.small_matrix(3584, 200, 4, 8, seed=77, residual=True)
    mi.x = (mi.x.astype(np.float64) * 300.0).astype(np.float16)
    mi.alpha = (mi.alpha.astype(np.float64) * 50.0).astype(np.float16)
    (y,), _ = _run_gemv([_upload(mi, residual=True)], [mi.x], residual=True)
    _assert_close(y, _oracle_res(mi), "residual large magnitudes")


# ------------------------------------------------------------------ the read floor
def test_stream_read_reads_every_word():
    # the measurement kernel must read every byte it is timed on: each
    # wavefront stores the XOR of what it read, so the XOR of the sink equals
    # the XOR of every 32-bit word of the buffers (loads past a buffer's end
    # return zeros, which leave it unchanged)
    _say("vq_stream_read XOR check")
    sizes = [16, (1 << 20) + 48, (4 << 20) + 1024]
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    bufs = [torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV, generator=g) for n in sizes]
    words = vq.vq_stream_read_sink_words(sizes)
    sink = torch.zeros(words, dtype=torch.int32, device=DEV)
    vq.vq_stream_read(bufs, sizes, sink, words)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    exp = 0
    for b in bufs:
        exp ^= int(np.bitwise_xor.reduce(b.cpu().numpy().view(np.uint32)))
    assert got == exp
