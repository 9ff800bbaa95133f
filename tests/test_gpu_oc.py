"""GPU parity of vq_gemv_oc, the plain 8-bit GEMV in the output-codebook
form ("EVA: Accelerating LLM Decoding via an Efficient Vector Quantization
Architecture", technical summary 2.A and 2.B): an OC tile of 64 subvectors x
256 centroids per workgroup in LDS, one lookup per index from the lane's own
bank, rows split along K and joined by a fixed-point atomic per row.

Against the float64 oracle (relative L2 <= 2e-3 and max error <= 1e-2 *
rms(y) per matrix, over every output), against vq_gemv (the same y by
another summation order: the same bar), and bitwise against itself:
repeated calls, graph-free reuse of one workspace, a matrix alone and in a
group (integer adds of the per-split partials do not depend on their order).
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
import synth  # noqa: E402
import vector_quantized_decode_amd as vq  # noqa: E402

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _assert_close(y, y_ref, what):
    rel, mx, rms = oracle.compare(y, y_ref)
    _say(f"{what}: rel_l2={rel:.3e} max_err={mx:.3e} rms={rms:.3e}")
    assert rel <= oracle.REL_L2_TOL, what
    assert mx <= oracle.MAX_ERR_RMS_TOL * rms, what


def _upload(mi):
    return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, device=DEV)


def _oracle(mi):
    return oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx, mi.nbits), mi.N, mi.K, mi.d,
                          mi.nbits)


def _run(mats, xs, ws=None, fn=None):
    ys = [torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
    if ws is None:
        ws = vq.alloc_workspace(mats, 1, residual=True, device=DEV)
    xt = [torch.from_numpy(x).to(DEV) for x in xs]
    (fn or vq.vq_gemv_oc)(mats, xt, 1, ys, ws, ws.numel())
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], ws


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("K,N", [(256, 1), (256, 17), (512, 100), (768, 333), (1024, 4103),
                                 (4096, 513), (8192, 77), (11008, 300), (33024, 40)])
def test_gemv_oc_shapes(K, N):
    # K = 256: one tile, no hand-off; K = 33024: 129 tiles, past the
    # fixed-point hand-off's 127, so float partials and a last-workgroup sum
    _say(f"gemv_oc K={K} N={N}")
    mi = synth.small_matrix(K, N, 4, 8, seed=3 * K + N)
    m = _upload(mi)
    (y,), _ = _run([m], [mi.x])
    _assert_close(y, _oracle(mi), f"oc K={K} N={N}")
    (yp,), _ = _run([m], [mi.x], ws=vq.alloc_workspace([m], 1, device=DEV), fn=vq.vq_gemv)
    _assert_close(y, yp.astype(np.float64), f"oc against vq_gemv K={K} N={N}")


@pytest.mark.parametrize("wl", [1, 2, 6, 7, 11])
def test_gemv_oc_workloads_every_row(wl):
    _say(f"gemv_oc workload {wl}, every row")
    w = synth.workload(wl)
    mis = [synth.matrix_inputs(wl, m) for m in range(w.count)]
    mats = [_upload(mi) for mi in mis]
    ys, ws = _run(mats, [mi.x for mi in mis])
    for m, (mi, y) in enumerate(zip(mis, ys)):
        _assert_close(y, _oracle(mi), f"oc workload {wl} matrix {m}")
    # the same workspace again (every call leaves its counters and
    # accumulators at zero): bitwise the same outputs
    ys2, _ = _run(mats, [mi.x for mi in mis], ws=ws)
    for a, b in zip(ys, ys2):
        assert np.array_equal(_bits(a), _bits(b))
    # a matrix alone gives bitwise its grouped result
    (y1,), _ = _run([mats[-1]], [mis[-1].x])
    assert np.array_equal(_bits(y1), _bits(ys[-1]))


@pytest.mark.parametrize("x_scale,wc_scale", [(1000.0, 100.0), (1e-3, 1e-2), (60.0, 1.0)])
def test_gemv_oc_across_magnitudes(x_scale, wc_scale):
    # the hand-off's fixed-point step follows a bound on each partial that
    # scales with |x| and max |WC|, so the relative accuracy holds at any scale
    _say(f"gemv_oc magnitudes x*{x_scale} wc*{wc_scale}")
    mi = synth.small_matrix(4096, 700, 4, 8, seed=91)
    mi.x = (mi.x.astype(np.float64) * x_scale).astype(np.float16)
    mi.wc = (mi.wc.astype(np.float64) * wc_scale).astype(np.float16)
    (y,), _ = _run([_upload(mi)], [mi.x])
    _assert_close(y, _oracle(mi), "oc scaled")


def test_gemv_oc_zero_input_gives_exact_zero():
    _say("gemv_oc x = 0")
    mi = synth.small_matrix(4096, 300, 4, 8, seed=92)
    mi.x = np.zeros_like(mi.x)
    (y,), _ = _run([_upload(mi)], [mi.x])
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("bad", ["inf", "nan"])
def test_gemv_oc_nonfinite_input_propagates_like_oracle(bad):
    # a non-finite input makes the hand-off bound non-finite: float partials
    # and a last-workgroup sum instead; every output's class (NaN, +inf,
    # -inf, finite) matches the oracle's, and the workspace is left ready for
    # the next call
    _say(f"gemv_oc non-finite input: {bad}")
    mi = synth.small_matrix(4096, 200, 4, 8, seed=93)
    x = mi.x.copy()
    x[0, 1234] = np.float16(np.inf if bad == "inf" else np.nan)
    mi.x = x
    m = _upload(mi)
    (y,), ws = _run([m], [mi.x])
    with np.errstate(invalid="ignore", over="ignore"):
        ref = _oracle(mi)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        _assert_close(y[fin], ref[fin], "finite rows")
    mi2 = synth.small_matrix(4096, 200, 4, 8, seed=94)
    (y2,), _ = _run([_upload(mi2)], [mi2.x], ws=ws)
    _assert_close(y2, _oracle(mi2), "after non-finite call")
