"""Graph replay of the library's calls (the way bench.py times them).

A HIP graph captured from vq_gemv / vq_gemv_oc / vq_gemv_residual / vq_gemv_swiglu must give, on every
replay, bitwise the result of the same call made eagerly: the calls record
only kernels (no memset nodes), the residual and output-codebook calls'
counters and accumulators are left at zero by every call, and the 16-bit call rewrites
its workspace each time.  Each replay follows eager work of its own (the
outputs poisoned with NaN, an unrelated eager call) and a synchronization.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import synth  # noqa: E402
import vector_quantized_decode_amd as vq  # noqa: E402

DEV = torch.device("cuda:0")


def _case(kind):
    if kind == "lut8":
        mis = [synth.small_matrix(4096, 700, 4, 8, seed=31), synth.small_matrix(2048, 300, 4, 8, seed=32)]
        return mis, 1, False
    if kind == "lut8_tokens":
        return [synth.small_matrix(2048, 515, 4, 8, B=3, seed=33)], 3, False
    if kind == "residual":
        mis = [synth.small_matrix(1024, 200, 4, 8, seed=34, residual=True),
               synth.small_matrix(3584, 96, 4, 8, seed=35, residual=True)]
        return mis, 1, True
    if kind == "oc":
        mis = [synth.small_matrix(4096, 700, 4, 8, seed=47), synth.small_matrix(768, 300, 4, 8, seed=48)]
        return mis, 1, True
    if kind == "wc12":
        return [synth.small_matrix(1024, 300, 4, 12, seed=36)], 1, False
    if kind == "swiglu":
        mis = [synth.small_matrix(2048, 300, 4, 8, seed=39), synth.small_matrix(2048, 300, 4, 8, seed=40)]
        return mis, 1, False
    if kind == "f16":
        mis = [synth.small_matrix(4096, 700, 4, 8, seed=45), synth.small_matrix(2048, 300, 4, 8, seed=46)]
        return mis, 1, False
    if kind == "tokens16":
        return [synth.small_matrix(4096, 300, 4, 8, B=16, seed=41),
                synth.small_matrix(1024, 77, 4, 8, B=16, seed=42)], 16, False
    if kind == "tokens5":
        return [synth.small_matrix(4096, 300, 4, 8, B=5, seed=43),
                synth.small_matrix(1024, 77, 4, 8, B=5, seed=44)], 5, False
    if kind == "wc16":
        return [synth.small_matrix(1024, 100, 8, 16, B=4, seed=37),
                synth.small_matrix(2048, 40, 8, 16, B=4, seed=38)], 4, False
    raise ValueError(kind)


def _upload(mi, residual, tokens=False):
    if tokens:
        return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, tokens=True, device=DEV)
    if residual:
        return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits,
                                sign_bits=mi.sign_bits, alpha=mi.alpha, group=mi.group,
                                rht_sign=mi.rht_sign, had_block=mi.had_block, device=DEV)
    return vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits, device=DEV)


@pytest.mark.parametrize("kind", ["lut8", "lut8_tokens", "residual", "oc", "wc12", "wc16", "swiglu",
                                  "tokens16", "tokens5", "f16"])
def test_graph_replays_match_eager(kind):
    print(f"[graph] {kind}", flush=True)
    mis, B, residual = _case(kind)
    # the output-codebook call takes the residual call's workspace, not its inputs
    mats = [_upload(mi, residual and kind != "oc", tokens=kind.startswith("tokens")) for mi in mis]
    xs = [torch.from_numpy(mi.x).to(DEV) for mi in mis]
    ydt = torch.float16 if kind == "f16" else torch.float32
    ys = [torch.full((B, m.N), float("nan"), dtype=ydt, device=DEV) for m in mats]
    ws = vq.alloc_workspace(mats, B, residual=residual, device=DEV)
    call = vq.vq_gemv_residual if residual else (vq.vq_gemv_f16 if kind == "f16" else vq.vq_gemv)
    if kind.startswith("tokens"):
        def call(ms, xs_, B_, ys_, ws_, n_, stream=None):
            vq.vq_gemv_tokens(ms, xs_, B_, ys_, stream=stream)
    if kind == "oc":
        call = vq.vq_gemv_oc
    if kind == "swiglu":
        def call(ms, xs_, B_, ys_, ws_, n_, stream=None):
            vq.vq_gemv_swiglu(ms[0::2], ms[1::2], xs_[0::2], B_, ys_[0::2], ws_, n_, stream=stream)

    # eager reference
    call(mats, xs, B, ys, ws, ws.numel())
    torch.cuda.synchronize()
    ref = [y.cpu().numpy().copy() for y in ys]
    if kind == "swiglu":
        ref = ref[:1]            # one gated output per pair; the up matrix's slot is not written
    assert all(np.isfinite(r).all() for r in ref)

    # an unrelated eager call between replays, on its own outputs and workspace
    ys2 = [torch.empty_like(y) for y in ys]
    ws2 = vq.alloc_workspace(mats, B, residual=residual, device=DEV)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call(mats, xs, B, ys, ws, ws.numel(), stream=stream)      # warm the launch path
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call(mats, xs, B, ys, ws, ws.numel(), stream=torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        call(mats, xs, B, ys2, ws2, ws2.numel())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for m, (y, r) in enumerate(zip(ys, ref)):
            got = y.cpu().numpy()
            assert np.array_equal(got.view(np.uint8), r.view(np.uint8)), f"{kind} replay {rep} matrix {m}"
