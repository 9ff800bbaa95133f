"""GPU test of vq_gemv_residual_noalloc, the residual call that allocates
nothing (its workspace is the library's fixed per-GPU device scratch),
through the C ABI: bitwise equal to vq_gemv_residual with a workspace of its
own, on calls in a row whose groups differ (the second call smaller, the
third the first again), and within tolerance of the float64 oracle."""
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


def _up(mi, rotate=True):
    m = vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, sign_bits=mi.sign_bits,
                         alpha=mi.alpha, group=mi.group, rht_sign=mi.rht_sign,
                         had_block=mi.had_block, device=DEV)
    if not rotate:
        m.rht_sign = None
    return m


def _both(mis, rotate):
    mats = [_up(mi, r) for mi, r in zip(mis, rotate)]
    xs = [torch.from_numpy(mi.x).to(DEV) for mi in mis]
    ref = [torch.full((1, mi.N), float("nan"), dtype=torch.float32, device=DEV) for mi in mis]
    got = [torch.full((1, mi.N), float("nan"), dtype=torch.float32, device=DEV) for mi in mis]
    ws = vq.alloc_workspace(mats, 1, residual=True, device=DEV)
    vq.vq_gemv_residual(mats, xs, 1, ref, ws, ws.numel())
    vq.vq_gemv_residual_noalloc(mats, xs, 1, got)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in ref], [g.cpu().numpy() for g in got]


def _oracle(mi, rotate):
    return oracle.vq_gemv_residual(mi.x, mi.wc, oracle.pack_rows(mi.idx, 8),
                                   oracle.pack_rows(mi.sign_bits, 1), mi.alpha,
                                   mi.rht_sign if rotate else None, mi.had_block, mi.N, mi.K,
                                   mi.d, mi.nbits, mi.group)


def _check(tag, mis, rotate):
    ref, got = _both(mis, rotate)
    for i, (mi, r, g, rot) in enumerate(zip(mis, ref, got, rotate)):
        assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), f"{tag} matrix {i}"
        rel, mx, rms = oracle.compare(g, _oracle(mi, rot))
        _say(f"{tag} matrix {i}: bitwise equal to the workspace call; rel_l2={rel:.3e}")
        assert rel <= oracle.REL_L2_TOL and mx <= oracle.MAX_ERR_RMS_TOL * rms


def test_noalloc_equals_the_workspace_call_on_calls_in_a_row():
    big = [synth.matrix_inputs(5, m) for m in range(2)]          # 3584 <-> 14336, rotated
    small = [synth.small_matrix(1024, 300, 4, 8, seed=91, residual=True),
             synth.small_matrix(2048, 100, 4, 8, seed=92, residual=True, had_block=256),
             synth.small_matrix(8192, 64, 4, 8, seed=93, residual=True)]   # h = 8192: rht kernel
    _say("call 1: the Gemma-2-9B-shaped pair")
    _check("call 1", big, [True, True])
    _say("call 2: a smaller group of three (one unrotated, one with its rotation in the scratch)")
    _check("call 2", small, [True, False, True])
    _say("call 3: the first group again")
    _check("call 3", big, [True, True])


def test_noalloc_rejects_a_group_beyond_its_scratch():
    # partials of 56 splits x 16384 rows need 3.7 MB, beyond the scratch
    mi = synth.small_matrix(14336, 16384, 4, 8, seed=94, residual=True, rows=1)
    m = vq.DeviceMatrix(mi.K, mi.N, 4, 8, torch.empty(16, dtype=torch.uint8, device=DEV),
                        torch.empty(1024, dtype=torch.float16, device=DEV),
                        torch.empty(16, dtype=torch.uint8, device=DEV),
                        torch.empty(16, dtype=torch.float16, device=DEV), 128)
    y = torch.empty((1, mi.N), dtype=torch.float32, device=DEV)
    x = torch.zeros((1, mi.K), dtype=torch.float16, device=DEV)
    with pytest.raises(vq.VQError) as e:
        vq.vq_gemv_residual_noalloc([m], [x], 1, [y])
    assert e.value.status == vq.VQ_EWORKSPACE
