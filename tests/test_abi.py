"""The C-ABI library loads without a GPU, exports every function that
include/vqd.h declares, and rejects invalid calls on the host before any
HIP call (no compute runs here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vqd.h")

vq = pytest.importorskip("vector_quantized_decode_amd",
                         reason="libvqd.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(vq_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(vq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(vq.EXPORTED) == names


def test_status_strings():
    assert vq.vq_status_str(0) == "VQ_OK"
    for s in (-1, -2, -3, -4, -5):
        assert vq.vq_status_str(s).startswith("VQ_E")
    assert vq.vq_status_str(7) == "unknown"


def test_device_layout_sizes():
    assert vq.vq_wi_device_bytes(4096, 4096, 4, 8) == 4096 * 1024
    assert vq.vq_wi_device_bytes(100, 1024, 4, 8) == 112 * 256      # rows padded to 16
    assert vq.vq_wi_device_bytes(64, 1000, 4, 8) == 0                # J not a multiple of 64
    assert vq.vq_wi_device_bytes(4096, 4096, 4, 12) == 4096 * 1024 * 3 // 2
    assert vq.vq_wi_device_bytes(11008, 4096, 4, 12) == 11008 * 1024 * 3 // 2
    assert vq.vq_wi_device_bytes(100, 1024, 4, 12) == 112 * 256 * 3 // 2   # rows padded to 16
    assert vq.vq_wi_device_bytes(5120, 13824, 8, 16) == 5120 * 1728 * 2
    assert vq.vq_wi_device_bytes(20, 256, 8, 16) == 32 * 32 * 2
    assert vq.vq_wi_device_bytes(16, 128, 8, 16) == 0                 # J not a multiple of 32
    assert vq.vq_wi_device_bytes(16, 1024, 4, 10) == 0                # no kernel for (4, 10)
    assert vq.vq_wc_device_bytes(4, 8) == 2048
    assert vq.vq_wc_device_bytes(4, 12) == 32768
    assert vq.vq_wc_device_bytes(8, 16) == 1 << 20
    assert vq.vq_wc_device_bytes(4, 10) == 0                      # no kernel for (4, 10)
    assert vq.vq_signs_device_bytes(14336, 3584) == 14336 * 448
    assert vq.vq_signs_device_bytes(100, 512) == 128 * 64            # rows padded to 32
    assert vq.vq_alpha_device_bytes(3584, 14336, 128) == 3584 * 112 * 2 + 256   # + header
    assert vq.vq_alpha_device_bytes(10, 256, 64) == 0


FAKE = 0x7f0000000000   # never dereferenced: every call below fails validation first


def _m(**kw):
    a = dict(K=1024, N=64, d=4, nbits=8, wi=FAKE, wc=FAKE, signs=FAKE, alpha=FAKE,
             group=128, rht_sign=None, had_block=0)
    a.update(kw)
    return vq.vq_matrix(**a)


def _gemv(mats, xs, B, ys, ws, nbytes, residual=False):
    f = vq._c["vq_gemv_residual" if residual else "vq_gemv"]
    arr = (vq.vq_matrix * max(1, len(mats)))(*mats) if mats else None
    xp = (ctypes.c_void_p * max(1, len(xs)))(*xs) if xs is not None else None
    yp = (ctypes.c_void_p * max(1, len(ys)))(*ys) if ys is not None else None
    return f(arr, len(mats), xp, B, yp, ws, nbytes, None)


def test_gemv_validation_errors():
    ok_x, ok_y = [FAKE], [FAKE]
    assert _gemv([], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL                   # count 0
    assert _gemv([_m()], None, 1, ok_y, None, 0) == vq.VQ_EINVAL               # x missing
    assert _gemv([_m()], ok_x, 0, ok_y, None, 0) == vq.VQ_EINVAL               # B < 1
    assert _gemv([_m(K=1022)], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL         # K % d
    assert _gemv([_m(d=3)], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL
    assert _gemv([_m(nbits=17)], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL
    assert _gemv([_m(wi=None)], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL
    assert _gemv([_m(N=0)], ok_x, 1, ok_y, None, 0) == vq.VQ_EINVAL
    assert _gemv([_m(d=2, nbits=8)], ok_x, 1, ok_y, None, 0) == vq.VQ_EUNSUPPORTED   # no kernel
    assert _gemv([_m(d=4, nbits=12)], ok_x, 2, ok_y, None, 0) == vq.VQ_EUNSUPPORTED  # one token
    assert _gemv([_m(d=8, nbits=16)], ok_x, 17, ok_y, None, 0) == vq.VQ_EUNSUPPORTED  # <= 16 tokens
    # one kernel per call: every matrix of a group has the same (d, nbits)
    assert _gemv([_m(), _m(d=4, nbits=12)], ok_x * 2, 1, ok_y * 2, None, 0) == vq.VQ_EUNSUPPORTED
    # the 12-bit format takes no workspace; the 16-bit one B*K*2 bytes (x by
    # dimension) per matrix, each rounded up to 256
    assert vq.vq_workspace_bytes([_m(d=4, nbits=12)], 1) == 0
    assert vq.vq_workspace_bytes([_m(d=8, nbits=16)], 16) == 16 * 1024 * 2
    assert vq.vq_workspace_bytes([_m(d=8, nbits=16, K=1280)] * 2, 3) == 2 * 7680
    assert vq.vq_workspace_bytes([_m(d=8, nbits=16, K=1280)], 1) == 2560
    need16 = vq.vq_workspace_bytes([_m(d=8, nbits=16)], 4)
    assert _gemv([_m(d=8, nbits=16)], ok_x, 4, ok_y, None, 0) == vq.VQ_EWORKSPACE
    assert _gemv([_m(d=8, nbits=16)], ok_x, 4, ok_y, FAKE, need16 - 1) == vq.VQ_EWORKSPACE
    assert _gemv([_m(d=8, nbits=16)], ok_x, 4, ok_y, FAKE + 16, need16) == vq.VQ_EALIGN
    assert _gemv([_m(d=8, nbits=16, K=65792)], ok_x, 1, ok_y, FAKE, 1 << 30) == vq.VQ_EUNSUPPORTED
    assert _gemv([_m(K=1088)], ok_x, 1, ok_y, None, 0) == vq.VQ_EUNSUPPORTED  # K % 256
    assert _gemv([_m()], ok_x, 5, ok_y, None, 0) == vq.VQ_EUNSUPPORTED        # 8-bit: B <= 4
    assert _gemv([_m(wi=FAKE + 8)], ok_x, 1, ok_y, None, 0) == vq.VQ_EALIGN
    assert _gemv([_m()], [FAKE + 2], 1, ok_y, None, 0) == vq.VQ_EALIGN
    assert _gemv([_m()], ok_x, 1, [FAKE + 1], None, 0) == vq.VQ_EALIGN
    # the plain kernels take no workspace; the residual kernel checks its own
    assert vq.vq_workspace_bytes([_m()], 1) == 0
    need = vq.vq_workspace_bytes([_m()], 1, residual=True)
    assert need > 0
    assert _gemv([_m()], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EWORKSPACE
    assert _gemv([_m()], ok_x, 1, ok_y, FAKE, need - 1, True) == vq.VQ_EWORKSPACE
    assert _gemv([_m()], ok_x, 1, ok_y, FAKE + 16, need, True) == vq.VQ_EALIGN
    assert _gemv([_m()] * 17, ok_x * 17, 1, ok_y * 17, FAKE, 1 << 30) == vq.VQ_EINVAL


def test_gemv_swiglu_validation_errors():
    c = vq._c["vq_gemv_swiglu"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    assert c(arr([_m()]), None, 1, ptrs(1), 1, ptrs(1), None, 0, None) == vq.VQ_EINVAL       # no up
    assert c(arr([_m()]), arr([_m(N=65)]), 1, ptrs(1), 1, ptrs(1), None, 0, None) == vq.VQ_EINVAL
    assert c(arr([_m()]), arr([_m()]), 1, ptrs(1), 3, ptrs(1), None, 0, None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m(K=12288)]), arr([_m(K=12288)]), 1, ptrs(1), 1, ptrs(1), None, 0,
             None) == vq.VQ_EUNSUPPORTED                                                   # long rows
    assert c(arr([_m(d=4, nbits=12)]), arr([_m(d=4, nbits=12)]), 1, ptrs(1), 1, ptrs(1), None, 0,
             None) == vq.VQ_EUNSUPPORTED


def test_gemv_swiglu_f16_validation_errors():
    c = vq._c["vq_gemv_swiglu_f16"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    assert c(arr([_m()]), None, 1, ptrs(1), 1, ptrs(1), None, 0, None) == vq.VQ_EINVAL       # no up
    assert c(arr([_m()]), arr([_m()]), 1, ptrs(1), 3, ptrs(1), None, 0, None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m()]), arr([_m()]), 1, ptrs(1), 1, ptrs(1, FAKE + 1), None, 0,
             None) == vq.VQ_EALIGN


def test_gemv_f16_validation_errors():
    c = vq._c["vq_gemv_f16"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    assert c(arr([_m()]), 1, ptrs(1), 0, ptrs(1), None, 0, None) == vq.VQ_EINVAL
    assert c(arr([_m()]), 1, ptrs(1), 5, ptrs(1), None, 0, None) == vq.VQ_EUNSUPPORTED   # B <= 4
    assert c(arr([_m()]), 1, ptrs(1), 1, ptrs(1, FAKE + 1), None, 0, None) == vq.VQ_EALIGN
    assert c(arr([_m()]), 1, ptrs(1, FAKE + 2), 1, ptrs(1), None, 0, None) == vq.VQ_EALIGN
    assert c(arr([_m(d=8, nbits=16)]), 1, ptrs(1), 1, ptrs(1, FAKE + 2), None, 0,
             None) == vq.VQ_EWORKSPACE                                      # 2-byte y passes
    assert c(arr([_m(d=3)]), 1, ptrs(1), 1, ptrs(1), None, 0, None) == vq.VQ_EINVAL


def test_gemv_tokens_validation_errors():
    c = vq._c["vq_gemv_tokens"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    assert c(arr([_m()]), 1, ptrs(1), 0, ptrs(1), None) == vq.VQ_EINVAL            # no token
    assert c(arr([_m()]), 1, ptrs(1), 17, ptrs(1), None) == vq.VQ_EUNSUPPORTED      # at most 16
    assert c(None, 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EINVAL
    assert c(arr([_m()]), 0, ptrs(1), 4, ptrs(1), None) == vq.VQ_EINVAL
    assert c(arr([_m()] * 17), 17, ptrs(17), 4, ptrs(17), None) == vq.VQ_EINVAL
    assert c(arr([_m(d=4, nbits=12)]), 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m(d=8, nbits=16)]), 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m(K=1088)]), 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EUNSUPPORTED   # K % 256
    # indices of 2 GiB or more: past 32-bit buffer offsets
    assert c(arr([_m(K=65536, N=131072)]), 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m(wi=FAKE + 8)]), 1, ptrs(1), 4, ptrs(1), None) == vq.VQ_EALIGN
    assert c(arr([_m()]), 1, ptrs(1, FAKE + 2), 4, ptrs(1), None) == vq.VQ_EALIGN
    assert c(arr([_m()]), 1, ptrs(1), 4, ptrs(1, FAKE + 1), None) == vq.VQ_EALIGN
    assert c(arr([_m(), _m(d=4, nbits=12)]), 2, ptrs(2), 4, ptrs(2), None) == vq.VQ_EUNSUPPORTED


def test_gemv_residual_validation_errors():
    ok_x, ok_y = [FAKE], [FAKE]
    assert _gemv([_m(signs=None)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EINVAL
    assert _gemv([_m()], ok_x, 2, ok_y, None, 0, True) == vq.VQ_EUNSUPPORTED   # one token
    assert _gemv([_m(group=64)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EUNSUPPORTED
    assert _gemv([_m(d=4, nbits=12)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EUNSUPPORTED
    # indices beyond 2 GiB: past the residual kernel's 32-bit buffer offsets
    assert _gemv([_m(K=65536, N=131072)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EUNSUPPORTED
    assert _gemv([_m(rht_sign=FAKE, had_block=3)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EINVAL
    assert _gemv([_m(rht_sign=FAKE, had_block=2048)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EINVAL
    assert _gemv([_m(rht_sign=FAKE, had_block=1024)], ok_x, 1, ok_y, None, 0, True) == vq.VQ_EWORKSPACE
    res = vq.vq_workspace_bytes([_m()], 1, residual=True)
    assert res >= 1024 * 4                       # x_rot at least


def test_gemv_oc_validation_errors():
    c = vq._c["vq_gemv_oc"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    ws = vq.vq_workspace_bytes([_m(signs=None, alpha=None)], 1, residual=True)
    assert ws > 0
    assert c(arr([_m()]), 0, ptrs(1), 1, ptrs(1), FAKE, ws, None) == vq.VQ_EINVAL
    assert c(arr([_m()]), 1, ptrs(1), 2, ptrs(1), FAKE, ws, None) == vq.VQ_EUNSUPPORTED   # one token
    assert c(arr([_m(d=4, nbits=12)]), 1, ptrs(1), 1, ptrs(1), FAKE, ws, None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m(K=65536, N=131072)]), 1, ptrs(1), 1, ptrs(1), FAKE, 1 << 30, None) == vq.VQ_EUNSUPPORTED
    assert c(arr([_m()]), 1, ptrs(1), 1, ptrs(1), None, 0, None) == vq.VQ_EWORKSPACE
    assert c(arr([_m()]), 1, ptrs(1), 1, ptrs(1), FAKE, ws - 1, None) == vq.VQ_EWORKSPACE
    assert c(arr([_m()]), 1, ptrs(1), 1, ptrs(1), FAKE + 16, ws, None) == vq.VQ_EALIGN
    assert c(arr([_m(wi=FAKE + 8)]), 1, ptrs(1), 1, ptrs(1), FAKE, ws, None) == vq.VQ_EALIGN


def test_gemv_residual_noalloc_validation_errors():
    # every check runs on the host before the scratch is looked up
    c = vq._c["vq_gemv_residual_noalloc"]
    arr = lambda ms: (vq.vq_matrix * len(ms))(*ms)
    ptrs = lambda n, v=FAKE: (ctypes.c_void_p * n)(*([v] * n))
    assert c(arr([_m()]), 0, ptrs(1), 1, ptrs(1), None) == vq.VQ_EINVAL
    assert c(arr([_m(signs=None)]), 1, ptrs(1), 1, ptrs(1), None) == vq.VQ_EINVAL
    assert c(arr([_m()]), 1, ptrs(1), 2, ptrs(1), None) == vq.VQ_EUNSUPPORTED        # one token
    assert c(arr([_m(alpha=FAKE + 16)]), 1, ptrs(1), 1, ptrs(1), None) == vq.VQ_EALIGN
    # counters and accumulators beyond VQ_NOALLOC_COUNTER_BYTES (1 MiB): 8 bytes
    # per row of a split matrix
    assert c(arr([_m(K=512, N=140000)]), 1, ptrs(1), 1, ptrs(1), None) == vq.VQ_EWORKSPACE
    # partials beyond the other 3 MiB: 56 splits x 16384 rows x 4 bytes
    assert c(arr([_m(K=14336, N=16384)]), 1, ptrs(1), 1, ptrs(1), None) == vq.VQ_EWORKSPACE


def test_other_entry_points_validate():
    c = vq._c
    assert c["vq_pack_indices"](FAKE, 10, 0, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_pack_indices"](FAKE, 10, 17, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_pack_indices"](None, 10, 8, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_pack_indices"](FAKE + 1, 10, 8, FAKE, None) == vq.VQ_EALIGN
    assert c["vq_pack_indices"](None, 0, 8, None, None) == vq.VQ_OK          # empty: nothing to do
    assert c["vq_unpack_indices"](FAKE, -1, 8, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_unpack_indices"](FAKE, 5, 8, FAKE + 2, None) == vq.VQ_EALIGN
    assert c["vq_repack_wi"](FAKE, 64, 1000, 4, 8, FAKE, None) == vq.VQ_EUNSUPPORTED
    assert c["vq_repack_wi"](FAKE, 64, 1024, 4, 8, FAKE + 4, None) == vq.VQ_EALIGN
    assert c["vq_repack_wi_rows"](None, 64, 1024, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_repack_wi_rows"](FAKE, 0, 1024, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_repack_wi_rows"](FAKE, 64, 1000, FAKE, None) == vq.VQ_EUNSUPPORTED   # K % 256
    assert c["vq_repack_wi_rows"](FAKE, 131072, 65536, FAKE, None) == vq.VQ_EUNSUPPORTED
    assert c["vq_repack_wi_rows"](FAKE + 8, 64, 1024, FAKE, None) == vq.VQ_EALIGN
    assert c["vq_repack_wi_rows"](FAKE, 64, 1024, FAKE + 4, None) == vq.VQ_EALIGN
    assert c["vq_repack_signs"](FAKE, 64, 1000, FAKE, None) == vq.VQ_EUNSUPPORTED
    assert c["vq_repack_wc"](None, 8, 16, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_repack_wc"](FAKE, 4, 10, FAKE, None) == vq.VQ_EUNSUPPORTED
    assert c["vq_repack_wc"](FAKE + 8, 8, 16, FAKE, None) == vq.VQ_EALIGN
    assert c["vq_repack_wc"](FAKE, 8, 16, FAKE + 2, None) == vq.VQ_EALIGN
    assert c["vq_repack_alpha"](FAKE, 64, 1024, 100, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_build_oc"](FAKE, 1, 10, 4, 8, FAKE, FAKE, vq.VQ_F32, None) == vq.VQ_EINVAL
    assert c["vq_build_oc"](FAKE, 1, 16, 4, 8, FAKE, FAKE, 7, None) == vq.VQ_EINVAL
    assert c["vq_build_oc"](FAKE, 1, 16, 4, 8, FAKE, FAKE + 2, vq.VQ_F32, None) == vq.VQ_EALIGN
    assert c["vq_rht"](FAKE, FAKE, 1, 3584, 1024, FAKE, None) == vq.VQ_EINVAL  # 1024 does not divide
    assert c["vq_rht"](FAKE, FAKE, 1, 1 << 15, 1 << 15, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_rht"](FAKE, None, 1, 1024, 1024, FAKE, None) == vq.VQ_EINVAL
    assert c["vq_workspace_init"](FAKE + 8, 1024, None) == vq.VQ_EALIGN
    assert c["vq_workspace_init"](None, 1024, None) == vq.VQ_EINVAL
    assert c["vq_workspace_bytes"](None, 1, 1, 0) == 0


def test_single_hip_runtime_in_process():
    """Importing the binding leaves exactly one HIP runtime mapped: the one
    torch loaded.  A second runtime would see no device and reject the
    library's launches."""
    pytest.importorskip("torch")
    import vector_quantized_decode_amd  # noqa: F401
    maps = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(maps) == 1, maps
