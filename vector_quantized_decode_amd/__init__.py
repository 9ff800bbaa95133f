"""Python binding of libvqd (vector-quantized decode GEMV for MI355X / gfx950).

Thin ctypes layer over the C ABI declared in ``include/vqd.h``: each
``vq_*`` function here has the C function's name and arguments, takes torch
device tensors (PyTorch provides device memory and streams only) and raises
:class:`VQError` on a negative status.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  If ``libvqd.so`` has
not been built the import fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m vector_quantized_decode_amd.build` (or __graft_entry__.build())")

# torch must load its HIP runtime first: libvqd.so then binds to that same
# runtime (same soname), so torch's device pointers and streams are valid in
# the library.  Loaded the other way round the process would hold two HIP
# runtimes, and the second one sees no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

VQ_OK, VQ_EINVAL, VQ_EUNSUPPORTED, VQ_EALIGN, VQ_EWORKSPACE, VQ_EHIP = 0, -1, -2, -3, -4, -5
VQ_F16, VQ_F32 = 0, 1
VQ_MAX_GROUP = 16

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class vq_matrix(ctypes.Structure):
    _fields_ = [("K", _i32), ("N", _i32), ("d", _i32), ("nbits", _i32),
                ("wi", _vp), ("wc", _vp), ("signs", _vp), ("alpha", _vp),
                ("group", _i32), ("rht_sign", _vp), ("had_block", _i32)]


def _sig(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_c = {
    "vq_status_str": _sig("vq_status_str", ctypes.c_char_p, [ctypes.c_int]),
    "vq_last_error": _sig("vq_last_error", ctypes.c_char_p, []),
    "vq_wi_device_bytes": _sig("vq_wi_device_bytes", _sz, [_i32, _i32, _i32, _i32]),
    "vq_signs_device_bytes": _sig("vq_signs_device_bytes", _sz, [_i32, _i32]),
    "vq_wc_device_bytes": _sig("vq_wc_device_bytes", _sz, [_i32, _i32]),
    "vq_repack_wc": _sig("vq_repack_wc", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "vq_alpha_device_bytes": _sig("vq_alpha_device_bytes", _sz, [_i32, _i32, _i32]),
    "vq_workspace_bytes": _sig("vq_workspace_bytes", _sz,
                               [ctypes.POINTER(vq_matrix), _i32, _i32, _i32]),
    "vq_workspace_init": _sig("vq_workspace_init", ctypes.c_int, [_vp, _sz, _vp]),
    "vq_pack_indices": _sig("vq_pack_indices", ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "vq_unpack_indices": _sig("vq_unpack_indices", ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "vq_repack_wi": _sig("vq_repack_wi", ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "vq_repack_wi_rows": _sig("vq_repack_wi_rows", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "vq_repack_signs": _sig("vq_repack_signs", ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "vq_repack_alpha": _sig("vq_repack_alpha", ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "vq_build_oc": _sig("vq_build_oc", ctypes.c_int,
                        [_vp, _i32, _i32, _i32, _i32, _vp, _vp, ctypes.c_int, _vp]),
    "vq_rht": _sig("vq_rht", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "vq_gemv": _sig("vq_gemv", ctypes.c_int,
                    [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                     ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "vq_gemv_shared": _sig("vq_gemv_shared", ctypes.c_int,
                           [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                            ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "vq_gemv_f16": _sig("vq_gemv_f16", ctypes.c_int,
                        [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                         ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "vq_gemv_oc": _sig("vq_gemv_oc", ctypes.c_int,
                       [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                        ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "vq_gemv_residual": _sig("vq_gemv_residual", ctypes.c_int,
                             [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                              ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "vq_gemv_residual_noalloc": _sig("vq_gemv_residual_noalloc", ctypes.c_int,
                                     [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                                      ctypes.POINTER(_vp), _vp]),
    "vq_gemv_swiglu": _sig("vq_gemv_swiglu", ctypes.c_int,
                           [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "vq_gemv_swiglu_f16": _sig("vq_gemv_swiglu_f16", ctypes.c_int,
                               [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "vq_gemv_tokens": _sig("vq_gemv_tokens", ctypes.c_int,
                           [ctypes.POINTER(vq_matrix), _i32, ctypes.POINTER(_vp), _i32,
                            ctypes.POINTER(_vp), _vp]),
    "vq_stream_read_sink_words": _sig("vq_stream_read_sink_words", _sz,
                                      [ctypes.POINTER(_sz), _i32]),
    "vq_stream_read": _sig("vq_stream_read", ctypes.c_int,
                           [ctypes.POINTER(_vp), ctypes.POINTER(_sz), _i32, _vp, _sz, _vp]),
}

# every symbol the header declares (checked by the ABI test)
EXPORTED = tuple(_c)


class VQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {vq_status_str(status)} ({status})"
        if status == VQ_EHIP:
            msg += f": {vq_last_error()}"
        super().__init__(msg)


def _check(status: int, where: str) -> None:
    if status != VQ_OK:
        raise VQError(status, where)


def _ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ plain calls
def vq_status_str(status: int) -> str:
    return _c["vq_status_str"](status).decode()


def vq_last_error() -> str:
    return _c["vq_last_error"]().decode()


def vq_wi_device_bytes(N: int, K: int, d: int, nbits: int) -> int:
    return _c["vq_wi_device_bytes"](N, K, d, nbits)


def vq_wc_device_bytes(d: int, nbits: int) -> int:
    return _c["vq_wc_device_bytes"](d, nbits)


def vq_repack_wc(wc, d: int, nbits: int, device_layout, stream=None) -> None:
    _check(_c["vq_repack_wc"](_ptr(wc), d, nbits, _ptr(device_layout), _stream(stream)),
           "vq_repack_wc")


def vq_signs_device_bytes(N: int, K: int) -> int:
    return _c["vq_signs_device_bytes"](N, K)


def vq_alpha_device_bytes(N: int, K: int, group: int) -> int:
    return _c["vq_alpha_device_bytes"](N, K, group)


def vq_pack_indices(idx, count: int, nbits: int, out, stream=None) -> None:
    _check(_c["vq_pack_indices"](_ptr(idx), count, nbits, _ptr(out), _stream(stream)),
           "vq_pack_indices")


def vq_unpack_indices(packed, count: int, nbits: int, out, stream=None) -> None:
    _check(_c["vq_unpack_indices"](_ptr(packed), count, nbits, _ptr(out), _stream(stream)),
           "vq_unpack_indices")


def vq_repack_wi(canonical, N: int, K: int, d: int, nbits: int, device_layout, stream=None) -> None:
    _check(_c["vq_repack_wi"](_ptr(canonical), N, K, d, nbits, _ptr(device_layout),
                              _stream(stream)), "vq_repack_wi")


def vq_repack_wi_rows(canonical, N: int, K: int, device_layout, stream=None) -> None:
    _check(_c["vq_repack_wi_rows"](_ptr(canonical), N, K, _ptr(device_layout), _stream(stream)),
           "vq_repack_wi_rows")


def vq_repack_signs(canonical, N: int, K: int, device_layout, stream=None) -> None:
    _check(_c["vq_repack_signs"](_ptr(canonical), N, K, _ptr(device_layout), _stream(stream)),
           "vq_repack_signs")


def vq_repack_alpha(canonical, N: int, K: int, group: int, device_layout, stream=None) -> None:
    _check(_c["vq_repack_alpha"](_ptr(canonical), N, K, group, _ptr(device_layout),
                                 _stream(stream)), "vq_repack_alpha")


def vq_build_oc(x, B: int, K: int, d: int, nbits: int, wc, oc, oc_dtype: int, stream=None) -> None:
    _check(_c["vq_build_oc"](_ptr(x), B, K, d, nbits, _ptr(wc), _ptr(oc), oc_dtype,
                             _stream(stream)), "vq_build_oc")


def vq_rht(x, sign, B: int, K: int, had_block: int, x_rot, stream=None) -> None:
    _check(_c["vq_rht"](_ptr(x), _ptr(sign), B, K, had_block, _ptr(x_rot), _stream(stream)),
           "vq_rht")


# ------------------------------------------------------------------ matrices
@dataclass
class DeviceMatrix:
    """Device buffers of one quantized matrix (tensors stay referenced here)."""
    K: int
    N: int
    d: int
    nbits: int
    wi: object                 # uint8 device layout
    wc: object                 # fp16 [2^n][d]
    signs: object = None       # uint8 sign device layout
    alpha: object = None       # fp16 alpha device layout
    group: int = 0
    rht_sign: object = None    # int8 [K]
    had_block: int = 0

    def c_struct(self) -> vq_matrix:
        return vq_matrix(self.K, self.N, self.d, self.nbits, _ptr(self.wi), _ptr(self.wc),
                         _ptr(self.signs), _ptr(self.alpha), self.group,
                         _ptr(self.rht_sign), self.had_block)


def _mat_array(mats: Sequence) -> ctypes.Array:
    arr = (vq_matrix * len(mats))()
    for i, m in enumerate(mats):
        arr[i] = m.c_struct() if isinstance(m, DeviceMatrix) else m
    return arr


def _ptr_array(ts: Sequence) -> ctypes.Array:
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def vq_workspace_bytes(mats: Sequence, B: int, residual: bool = False) -> int:
    arr = _mat_array(mats)
    return _c["vq_workspace_bytes"](arr, len(mats), B, 1 if residual else 0)


def vq_workspace_init(workspace, ws_bytes: int, stream=None) -> None:
    _check(_c["vq_workspace_init"](_ptr(workspace), ws_bytes, _stream(stream)),
           "vq_workspace_init")


def vq_gemv(mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace, ws_bytes: int,
            stream=None) -> None:
    arr = _mat_array(mats)
    _check(_c["vq_gemv"](arr, len(mats), _ptr_array(xs), B, _ptr_array(ys), _ptr(workspace),
                         ws_bytes, _stream(stream)), "vq_gemv")


def vq_gemv_shared(mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace=None,
                   ws_bytes: int = 0, stream=None) -> None:
    """vq_gemv with matrices that share codebook, x and shape merged into units."""
    _check(_c["vq_gemv_shared"](_mat_array(mats), len(mats), _ptr_array(xs), B, _ptr_array(ys),
                                _ptr(workspace), ws_bytes, _stream(stream)), "vq_gemv_shared")


def vq_gemv_f16(mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace, ws_bytes: int,
                stream=None) -> None:
    """vq_gemv storing fp16 y (the fp32 sums rounded to nearest even)."""
    _check(_c["vq_gemv_f16"](_mat_array(mats), len(mats), _ptr_array(xs), B, _ptr_array(ys),
                             _ptr(workspace), ws_bytes, _stream(stream)), "vq_gemv_f16")


def vq_gemv_oc(mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace, ws_bytes: int,
               stream=None) -> None:
    """vq_gemv's result through the output-codebook tile kernel (workspace of
    vq_workspace_bytes(..., residual=True))."""
    _check(_c["vq_gemv_oc"](_mat_array(mats), len(mats), _ptr_array(xs), B, _ptr_array(ys),
                            _ptr(workspace), ws_bytes, _stream(stream)), "vq_gemv_oc")


def vq_gemv_residual(mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace,
                     ws_bytes: int, stream=None) -> None:
    arr = _mat_array(mats)
    _check(_c["vq_gemv_residual"](arr, len(mats), _ptr_array(xs), B, _ptr_array(ys),
                                  _ptr(workspace), ws_bytes, _stream(stream)),
           "vq_gemv_residual")


def vq_gemv_residual_noalloc(mats: Sequence, xs: Sequence, B: int, ys: Sequence,
                             stream=None) -> None:
    """vq_gemv_residual on the library's fixed per-GPU device scratch (no workspace)."""
    _check(_c["vq_gemv_residual_noalloc"](_mat_array(mats), len(mats), _ptr_array(xs), B,
                                          _ptr_array(ys), _stream(stream)),
           "vq_gemv_residual_noalloc")


def vq_gemv_swiglu(gates: Sequence, ups: Sequence, xs: Sequence, B: int, ys: Sequence, workspace,
                   ws_bytes: int, stream=None) -> None:
    """y[i] = silu(gate[i] x[i]) * (up[i] x[i]), gate/up pairs of one shape."""
    if len(gates) != len(ups):
        raise ValueError("one up matrix per gate matrix")
    _check(_c["vq_gemv_swiglu"](_mat_array(gates), _mat_array(ups), len(gates), _ptr_array(xs), B,
                                _ptr_array(ys), _ptr(workspace), ws_bytes, _stream(stream)),
           "vq_gemv_swiglu")


def vq_gemv_swiglu_f16(gates: Sequence, ups: Sequence, xs: Sequence, B: int, ys: Sequence,
                       workspace, ws_bytes: int, stream=None) -> None:
    """vq_gemv_swiglu storing fp16 y (the fp32 gated products rounded to nearest even)."""
    if len(gates) != len(ups):
        raise ValueError("one up matrix per gate matrix")
    _check(_c["vq_gemv_swiglu_f16"](_mat_array(gates), _mat_array(ups), len(gates), _ptr_array(xs),
                                    B, _ptr_array(ys), _ptr(workspace), ws_bytes, _stream(stream)),
           "vq_gemv_swiglu_f16")


def vq_gemv_tokens(mats: Sequence, xs: Sequence, B: int, ys: Sequence, stream=None) -> None:
    """vq_gemv for 1-16 tokens at d=4, n=8; each mats[i].wi holds row tiles (vq_repack_wi_rows)."""
    _check(_c["vq_gemv_tokens"](_mat_array(mats), len(mats), _ptr_array(xs), B, _ptr_array(ys),
                                _stream(stream)), "vq_gemv_tokens")


def _size_array(ns: Sequence[int]) -> ctypes.Array:
    arr = (_sz * len(ns))()
    for i, n in enumerate(ns):
        arr[i] = int(n)
    return arr


def vq_stream_read_sink_words(nbytes: Sequence[int]) -> int:
    return _c["vq_stream_read_sink_words"](_size_array(nbytes), len(nbytes))


def vq_stream_read(buffers: Sequence, nbytes: Sequence[int], sink, sink_words: int,
                   stream=None) -> None:
    """Measurement helper: one plain streaming read of the buffers (no method
    arithmetic); sink receives one XOR word per wavefront."""
    _check(_c["vq_stream_read"](_ptr_array(buffers), _size_array(nbytes), len(buffers), _ptr(sink),
                                sink_words, _stream(stream)), "vq_stream_read")


# ------------------------------------------------------------------ prepared calls
class PreparedCall:
    """One library call with its ctypes arguments built once, for callers
    that issue the same call many times from Python (a launch loop): calling
    it passes only the stream.  It keeps the tensors and arrays it points at
    referenced."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self._f = _c[name]
        self._name = name
        self._args = args
        self._keep = keep

    def __call__(self, stream) -> None:
        st = self._f(*self._args, _stream(stream))
        if st != VQ_OK:
            raise VQError(st, self._name)


def prepare_gemv(name: str, mats: Sequence, xs: Sequence, B: int, ys: Sequence, workspace=None,
                 ws_bytes: int = 0) -> PreparedCall:
    """A PreparedCall of vq_gemv, vq_gemv_shared, vq_gemv_f16, vq_gemv_oc or
    vq_gemv_residual."""
    if name not in ("vq_gemv", "vq_gemv_f16", "vq_gemv_residual", "vq_gemv_shared", "vq_gemv_oc"):
        raise ValueError(name)
    arr, xa, ya = _mat_array(mats), _ptr_array(xs), _ptr_array(ys)
    return PreparedCall(name, (arr, len(mats), xa, B, ya, _ptr(workspace), ws_bytes),
                        (arr, xa, ya, tuple(mats), tuple(xs), tuple(ys), workspace))


def prepare_gemv_tokens(mats: Sequence, xs: Sequence, B: int, ys: Sequence) -> PreparedCall:
    arr, xa, ya = _mat_array(mats), _ptr_array(xs), _ptr_array(ys)
    return PreparedCall("vq_gemv_tokens", (arr, len(mats), xa, B, ya),
                        (arr, xa, ya, tuple(mats), tuple(xs), tuple(ys)))


def prepare_gemv_swiglu(gates: Sequence, ups: Sequence, xs: Sequence, B: int, ys: Sequence,
                        f16: bool = False) -> PreparedCall:
    if len(gates) != len(ups):
        raise ValueError("one up matrix per gate matrix")
    ga, ua, xa, ya = _mat_array(gates), _mat_array(ups), _ptr_array(xs), _ptr_array(ys)
    name = "vq_gemv_swiglu_f16" if f16 else "vq_gemv_swiglu"
    return PreparedCall(name, (ga, ua, len(gates), xa, B, ya, None, 0),
                        (ga, ua, xa, ya, tuple(gates), tuple(ups), tuple(xs), tuple(ys)))


def prepare_stream_read(buffers: Sequence, nbytes: Sequence[int], sink,
                        sink_words: int) -> PreparedCall:
    ba, na = _ptr_array(buffers), _size_array(nbytes)
    return PreparedCall("vq_stream_read", (ba, na, len(buffers), _ptr(sink), sink_words),
                        (ba, na, tuple(buffers), sink))


# ------------------------------------------------------------------ helpers
def alloc_workspace(mats: Sequence, B: int, residual: bool = False, device="cuda"):
    """Allocate (torch) and initialize a workspace for these matrices."""
    import torch
    n = vq_workspace_bytes(mats, B, residual)
    if n == 0:
        n = 256
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    vq_workspace_init(ws, n)
    return ws


def upload_matrix(idx, wc, K: int, N: int, d: int, nbits: int, *, sign_bits=None, alpha=None,
                  group: int = 128, rht_sign=None, had_block: int = 0, tokens: bool = False,
                  device="cuda", stream=None) -> DeviceMatrix:
    """Copy host inputs to the device and build the device layouts with the
    library's pack and repack kernels.

    idx: integer array [N][K/d]; wc: fp16 [2^n][d] (laid out by vq_repack_wc); sign_bits: {0,1} [N][K];
    alpha: fp16 [N][K/group]; rht_sign: int8 [K].  tokens: lay WI out in row
    tiles (vq_repack_wi_rows, what vq_gemv_tokens reads) instead of vq_repack_wi's layout.
    """
    import numpy as np
    import torch
    J = K // d
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.uint32).view(np.int32)).to(device)
    canon = torch.empty((N * J * nbits + 7) // 8, dtype=torch.uint8, device=device)
    vq_pack_indices(idx_t, N * J, nbits, canon, stream)
    if tokens:
        wi = torch.empty(vq_wi_device_bytes(N, K, d, nbits), dtype=torch.uint8, device=device)
        vq_repack_wi_rows(canon, N, K, wi, stream)
    else:
        wi = torch.empty(vq_wi_device_bytes(N, K, d, nbits), dtype=torch.uint8, device=device)
        vq_repack_wi(canon, N, K, d, nbits, wi, stream)
    wc_t = torch.from_numpy(np.ascontiguousarray(wc, dtype=np.float16)).to(device)
    wc_dev = torch.empty(vq_wc_device_bytes(d, nbits) // 2, dtype=torch.float16, device=device)
    vq_repack_wc(wc_t, d, nbits, wc_dev, stream)
    m = DeviceMatrix(K, N, d, nbits, wi, wc_dev)
    if sign_bits is not None:
        sb = torch.from_numpy(np.ascontiguousarray(sign_bits, dtype=np.uint8).astype(np.int32)).to(device)
        canon_s = torch.empty(N * K // 8, dtype=torch.uint8, device=device)
        vq_pack_indices(sb, N * K, 1, canon_s, stream)
        m.signs = torch.empty(vq_signs_device_bytes(N, K), dtype=torch.uint8, device=device)
        vq_repack_signs(canon_s, N, K, m.signs, stream)
        al = torch.from_numpy(np.ascontiguousarray(alpha, dtype=np.float16)).to(device)
        m.alpha = torch.empty(vq_alpha_device_bytes(N, K, group) // 2, dtype=torch.float16,
                              device=device)
        vq_repack_alpha(al, N, K, group, m.alpha, stream)
        m.group = group
        if rht_sign is not None:
            m.rht_sign = torch.from_numpy(np.ascontiguousarray(rht_sign, dtype=np.int8)).to(device)
            m.had_block = had_block
    return m
