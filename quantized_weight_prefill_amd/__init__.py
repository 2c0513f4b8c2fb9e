"""MI355X (gfx950) fused-dequant prefill linear layer: Python binding.

    Y[M,N] = X[M,K] . dequant(W)[K,N]

This module only marshals arguments for the C ABI of ``include/qgemm.h``
(``libqgemm.so``, built by ``python -m quantized_weight_prefill_amd.build``):
PyTorch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the call fails, an exception is raised.

Functions keep the C names without the ``qgemm_`` prefix:

* packers (host, numpy): :func:`q4k_pack`, :func:`q6k_pack`,
  :func:`w4a16_pack` and their inverses ``*_unpack``;
* GEMMs (device, torch): :func:`q4k`, :func:`q6k`, :func:`w4a16`,
  :func:`gemm_rung`;
* fragment-major activations: :func:`xf_bytes`, :func:`x_to_xf`,
  :func:`gemm_xf`, :func:`select_rung_xf`;
* the staged dequant :func:`dequant` and the M-ladder queries
  :func:`select_rung`, :func:`rung_info`, :func:`rung_name`, :func:`num_rungs`;
* the split rungs' workspace size :func:`workspace_bytes` (the C library
  never allocates: when a call needs a workspace and none is passed, the
  binding takes one from torch's allocator for that call).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgemm.so")

F16 = 0
BF16 = 1
FMT_Q4K = 0
FMT_Q6K = 1
FMT_W4A16 = 2
FORMATS = {"q4k": FMT_Q4K, "q6k": FMT_Q6K, "w4a16": FMT_W4A16}
X_ROW = 0
X_FRAG = 1

#: status codes of include/qgemm.h
STATUS = {0: "QGEMM_OK", -1: "QGEMM_ERR_NULL", -2: "QGEMM_ERR_SHAPE", -3: "QGEMM_ERR_DTYPE",
          -4: "QGEMM_ERR_ALIGN", -5: "QGEMM_ERR_FORMAT", -6: "QGEMM_ERR_SIZE", -7: "QGEMM_ERR_HIP",
          -8: "QGEMM_ERR_INPUT"}

_lib = None


class QGemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.qgemm_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

#: exported symbol -> (restype, argtypes); the tests check this against the header
SIGNATURES = {
    "qgemm_status_str": (ctypes.c_char_p, [_INT]),
    "qgemm_q4k_packed_bytes": (_SZ, [_I64, _I64]),
    "qgemm_q4k_pack": (_INT, [_VP, _I64, _I64, _VP, _SZ]),
    "qgemm_q4k_unpack": (_INT, [_VP, _I64, _I64, _VP, _SZ]),
    "qgemm_q6k_packed_bytes": (_SZ, [_I64, _I64]),
    "qgemm_q6k_pack": (_INT, [_VP, _I64, _I64, _VP, _SZ]),
    "qgemm_q6k_unpack": (_INT, [_VP, _I64, _I64, _VP, _SZ]),
    "qgemm_w4a16_packed_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "qgemm_w4a16_pack": (_INT, [_VP, _VP, _VP, _I64, _I64, _I64, _VP, _SZ]),
    "qgemm_w4a16_unpack": (_INT, [_VP, _I64, _I64, _I64, _INT, _VP, _VP, _VP]),
    "qgemm_q4k": (_INT, [_VP, _VP, _VP, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_q6k": (_INT, [_VP, _VP, _VP, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_w4a16": (_INT, [_VP, _VP, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_num_rungs": (_INT, []),
    "qgemm_rung_name": (ctypes.c_char_p, [_INT]),
    "qgemm_select_rung": (_INT, [_INT, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_rung_info": (_INT, [_INT, _INT, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_gemm_rung": (_INT, [_INT, _INT, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP, _SZ, _VP]),
    "qgemm_workspace_bytes": (_SZ, [_INT, _INT, _INT, _I64, _I64, _I64, _INT]),
    "qgemm_dequant": (_INT, [_INT, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_grouped": (_INT, [_INT, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_grouped_xf": (_INT, [_INT, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_grouped_plan": (_INT, [_I64, _I64, _I64, _I64, _VP]),
    "qgemm_staged_scratch_bytes": (_SZ, [_I64, _I64]),
    "qgemm_staged": (_INT, [_INT, _VP, _VP, _VP, _SZ, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_xf_bytes": (_SZ, [_I64, _I64]),
    "qgemm_x_to_xf": (_INT, [_VP, _VP, _I64, _I64, _VP]),
    "qgemm_gemm_xf": (_INT, [_INT, _INT, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP, _SZ, _VP]),
    "qgemm_select_rung_xf": (_INT, [_INT, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_gemm_xf_noalloc": (_INT, [_INT, _INT, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP]),
    "qgemm_gguf_header": (_INT, [_VP, _SZ, _VP, _VP, _VP, _VP, _VP]),
    "qgemm_gguf_tensor_info": (_INT, [_VP, _SZ, _I64, _VP, _SZ, _VP, _VP, _VP, _VP, _VP]),
    "qgemm_gguf_find_kv": (_INT, [_VP, _SZ, ctypes.c_char_p, _VP, _VP, _VP]),
    "qgemm_gguf_packed_bytes": (_SZ, [_VP, _SZ, _I64]),
    "qgemm_gguf_pack": (_INT, [_VP, _SZ, _I64, _VP, _SZ, _VP, _VP, _VP]),
    "qgemm_i8_xq_bytes": (_SZ, [_I64, _I64]),
    "qgemm_i8_quantize": (_INT, [_VP, _VP, _VP, _I64, _I64, _INT, _VP]),
    "qgemm_i8_colscale": (_INT, [_INT, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _VP]),
    "qgemm_i8_gemm": (_INT, [_INT, _INT, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _VP, _SZ,
                             _VP]),
    "qgemm_i8_workspace_bytes": (_SZ, [_INT, _INT, _I64, _I64, _I64]),
    "qgemm_i8_num_rungs": (_INT, []),
    "qgemm_i8_rung_name": (ctypes.c_char_p, [_INT]),
    "qgemm_i8_rung_info": (_INT, [_INT, _INT, _I64, _I64, _I64, _VP]),
    "qgemm_i8_select_rung": (_INT, [_INT, _I64, _I64, _I64, _VP]),
}


def lib():
    """The loaded C library (raises if it has not been built).

    PyTorch ships its own HIP runtime under the same SONAME as the system one.
    torch is imported first so that opening libqgemm.so binds it to the HIP
    runtime already in the process: device pointers, streams and kernels then
    all belong to one runtime."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with `python -m quantized_weight_prefill_amd.build`")
        import torch  # noqa: F401  (binds libamdhip64.so.7 to torch's runtime)

        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise QGemmError(fn, status)


def _np_ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------
# host packers
# ---------------------------------------------------------------------------

def q4k_packed_bytes(N: int, K: int) -> int:
    return int(lib().qgemm_q4k_packed_bytes(N, K))


def q6k_packed_bytes(N: int, K: int) -> int:
    return int(lib().qgemm_q6k_packed_bytes(N, K))


def w4a16_packed_bytes(N: int, K: int, group: int, has_zp: bool) -> int:
    return int(lib().qgemm_w4a16_packed_bytes(N, K, group, int(bool(has_zp))))


def q4k_pack(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    """GGUF-style Q4_K blocks [N][K/256][144] -> packed panel layout (uint8)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(q4k_packed_bytes(N, K), np.uint8)
    _check("qgemm_q4k_pack", lib().qgemm_q4k_pack(_np_ptr(b), N, K, _np_ptr(out), out.nbytes))
    return out


def q4k_unpack(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((N, K // 256, 144), np.uint8)
    _check("qgemm_q4k_unpack", lib().qgemm_q4k_unpack(_np_ptr(p), N, K, _np_ptr(out), out.nbytes))
    return out


def q6k_pack(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    """GGUF-style Q6_K blocks [N][K/256][210] -> packed panel layout (uint8)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty(q6k_packed_bytes(N, K), np.uint8)
    _check("qgemm_q6k_pack", lib().qgemm_q6k_pack(_np_ptr(b), N, K, _np_ptr(out), out.nbytes))
    return out


def q6k_unpack(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((N, K // 256, 210), np.uint8)
    _check("qgemm_q6k_unpack", lib().qgemm_q6k_unpack(_np_ptr(p), N, K, _np_ptr(out), out.nbytes))
    return out


def w4a16_pack(codes: np.ndarray, scales: np.ndarray, zeros, N: int, K: int, group: int) -> np.ndarray:
    """codes [N][K] (0..15), fp16 scale bits [K/g][N], zeros [K/g][N] or None."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    z = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    out = np.empty(w4a16_packed_bytes(N, K, group, z is not None), np.uint8)
    _check("qgemm_w4a16_pack", lib().qgemm_w4a16_pack(_np_ptr(c), _np_ptr(s), None if z is None else _np_ptr(z),
                                                      N, K, group, _np_ptr(out), out.nbytes))
    return out


def w4a16_unpack(packed: np.ndarray, N: int, K: int, group: int, has_zp: bool):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((K // group, N), np.uint16)
    zeros = np.empty((K // group, N), np.uint8) if has_zp else None
    _check("qgemm_w4a16_unpack", lib().qgemm_w4a16_unpack(_np_ptr(p), N, K, group, int(bool(has_zp)), _np_ptr(codes),
                                                          _np_ptr(scales), None if zeros is None else _np_ptr(zeros)))
    return codes, scales, zeros


def pack(fmt: str, enc, N: int, K: int) -> np.ndarray:
    """Pack the output of the synthetic generator's ``encode`` for ``fmt``."""
    if fmt == "q4k":
        return q4k_pack(enc, N, K)
    if fmt == "q6k":
        return q6k_pack(enc, N, K)
    if fmt == "w4a16":
        return w4a16_pack(enc["codes"], enc["scales"], None if enc["symmetric"] else enc["zeros"], N, K,
                          enc["group"])
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# GGUF checkpoints (host)
# ---------------------------------------------------------------------------

GGML_Q4_K = 12
GGML_Q6_K = 14
_GGUF_SCALAR = {0: "<u1", 1: "<i1", 2: "<u2", 3: "<i2", 4: "<u4", 5: "<i4", 6: "<f4", 7: "<u1", 10: "<u8", 11: "<i8",
                12: "<f8"}


def gguf_map(path: str) -> np.ndarray:
    """The whole file as a read-only uint8 array (memory-mapped)."""
    return np.memmap(path, dtype=np.uint8, mode="r")


def _buf(buf: np.ndarray):
    b = np.asarray(buf, dtype=np.uint8)
    if not b.flags.c_contiguous:
        b = np.ascontiguousarray(b)
    return b, ctypes.c_void_p(b.ctypes.data), b.nbytes


def gguf_header(buf: np.ndarray) -> dict:
    b, p, n = _buf(buf)
    v = ctypes.c_uint32()
    nt, nk, al, do = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("qgemm_gguf_header", lib().qgemm_gguf_header(p, n, ctypes.byref(v), ctypes.byref(nt), ctypes.byref(nk),
                                                        ctypes.byref(al), ctypes.byref(do)))
    return dict(version=v.value, n_tensors=nt.value, n_kv=nk.value, alignment=al.value, data_offset=do.value)


def gguf_tensors(buf: np.ndarray) -> list:
    """Every tensor's name, ggml type, dims (row length first), byte offset and size."""
    b, p, n = _buf(buf)
    out = []
    for i in range(gguf_header(b)["n_tensors"]):
        name = ctypes.create_string_buffer(1024)
        t, nd = ctypes.c_int32(), ctypes.c_int32()
        dims = (ctypes.c_int64 * 4)()
        off, nb = ctypes.c_int64(), ctypes.c_int64()
        _check("qgemm_gguf_tensor_info", lib().qgemm_gguf_tensor_info(p, n, i, name, 1024, ctypes.byref(t), ctypes.byref(nd),
                                                                      dims, ctypes.byref(off), ctypes.byref(nb)))
        out.append(dict(index=i, name=name.value.decode(), type=t.value, dims=tuple(dims[:nd.value]), offset=off.value,
                        nbytes=nb.value))
    return out


def gguf_kv(buf: np.ndarray, key: str):
    """The metadata value of `key`: a number, a string, or a list (arrays of
    numbers or strings); None when the file has no such key."""
    b, p, n = _buf(buf)
    t, off, nb = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    st = lib().qgemm_gguf_find_kv(p, n, key.encode(), ctypes.byref(t), ctypes.byref(off), ctypes.byref(nb))
    if st == -5:
        return None
    _check("qgemm_gguf_find_kv", st)
    raw = bytes(b[off.value:off.value + nb.value])

    def string(r, i):
        ln = int.from_bytes(r[i:i + 8], "little")
        return r[i + 8:i + 8 + ln].decode("utf-8", "replace"), i + 8 + ln

    if t.value == 8:
        return string(raw, 0)[0]
    if t.value == 9:
        et = int.from_bytes(raw[0:4], "little")
        cnt = int.from_bytes(raw[4:12], "little")
        if et == 8:
            vals, i = [], 12
            for _ in range(cnt):
                s, i = string(raw, i)
                vals.append(s)
            return vals
        return np.frombuffer(raw[12:], dtype=_GGUF_SCALAR[et], count=cnt).tolist()
    v = np.frombuffer(raw, dtype=_GGUF_SCALAR[t.value], count=1)[0]
    return bool(v) if t.value == 7 else v.item()


def gguf_pack(buf: np.ndarray, index: int):
    """Tensor `index` (Q4_K or Q6_K, two-dimensional) packed for the GEMMs:
    (format name, N, K, packed uint8 array)."""
    b, p, n = _buf(buf)
    need = int(lib().qgemm_gguf_packed_bytes(p, n, index))
    out = np.empty(max(need, 16), np.uint8)
    f, N, K = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check("qgemm_gguf_pack", lib().qgemm_gguf_pack(p, n, index, _np_ptr(out), need, ctypes.byref(f), ctypes.byref(N),
                                                    ctypes.byref(K)))
    name = {FMT_Q4K: "q4k", FMT_Q6K: "q6k"}[f.value]
    return name, N.value, K.value, out[:need]


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out(x, N, out):
    torch = _torch()
    M = x.shape[0]
    if out is None:
        return torch.empty((M, N), dtype=x.dtype, device=x.device)
    if out.shape != (M, N) or out.dtype != x.dtype:
        raise ValueError("out has the wrong shape or dtype")
    return out


def packed_bytes(fmt, N: int, K: int, group: int = 128, has_zp: bool = False) -> int:
    """Packed bytes of one N x K weight of format ``fmt``."""
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if f == FMT_Q4K:
        return q4k_packed_bytes(N, K)
    if f == FMT_Q6K:
        return q6k_packed_bytes(N, K)
    return w4a16_packed_bytes(N, K, group, has_zp)


def _check_wp(fmt, wp, N: int, K: int, group: int, has_zp: bool, experts: int = 1):
    need = packed_bytes(fmt, N, K, group if group else 128, has_zp) * experts
    if need == 0:
        raise QGemmError("packed_bytes", -2)
    if wp.numel() * wp.element_size() < need:
        raise ValueError(f"wp holds {wp.numel() * wp.element_size()} bytes, the packed weight needs {need}")


def workspace_bytes(fmt, rung: int, M: int, N: int, K: int, dtype: int = F16, layout: int = X_ROW) -> int:
    """Bytes of the workspace a GEMM call with these arguments needs (0: none)."""
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return int(lib().qgemm_workspace_bytes(f, rung, layout, M, N, K, dtype))


def _workspace(need: int, workspace, device):
    """(pointer, bytes) of the caller's workspace, or of one taken from
    torch's allocator when the call needs one and none was given."""
    if workspace is None:
        if need == 0:
            return None, 0, None
        workspace = _torch().empty(need, dtype=_torch().uint8, device=device)
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), workspace


def gemm_rung(fmt, rung: int, x, wp, N: int, group: int = 0, has_zp: bool = False, out=None, stream=None,
              workspace=None):
    """Y = X . dequant(W) with the rung forced (rung = -1 selects as the format calls do)."""
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    _check_wp(f, wp, N, K, group, has_zp)
    y = _out(x, N, out)
    ws, wsb, _keep = _workspace(workspace_bytes(f, rung, M, N, K, _dtype_code(x), X_ROW), workspace, x.device)
    st = lib().qgemm_gemm_rung(f, rung, _dev(x, "x"), _dev(wp, "wp"), _dev(y, "out"), M, N, K, group,
                               int(bool(has_zp)), _dtype_code(x), ws, wsb, _stream(stream))
    _check("qgemm_gemm_rung", st)
    return y


def xf_bytes(M: int, K: int) -> int:
    return int(lib().qgemm_xf_bytes(M, K))


def x_to_xf(x, out=None, stream=None):
    """The fragment-major copy of a row-major [M, K] activation matrix: a flat
    tensor of x's dtype with 32*ceil(M/32)*K elements."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    n = xf_bytes(M, K) // 2
    if n == 0 and M > 0:
        raise QGemmError("qgemm_xf_bytes", -2)
    if out is None:
        out = torch.empty((n,), dtype=x.dtype, device=x.device)
    elif out.numel() < n or out.dtype != x.dtype:
        raise ValueError("out is too small or has the wrong dtype")
    _check("qgemm_x_to_xf", lib().qgemm_x_to_xf(_dev(x, "x"), _dev(out, "out"), M, K, _stream(stream)))
    return out


def gemm_xf(fmt, xf, wp, M: int, N: int, K: int, group: int = 0, has_zp: bool = False, rung: int = -1, out=None,
            stream=None, workspace=None):
    """Y = X . dequant(W) with X given as its fragment-major copy `xf`
    (from :func:`x_to_xf`); rung -1 selects from the ladder for that layout."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if xf.numel() < xf_bytes(M, K) // 2:
        raise ValueError("xf is smaller than the fragment-major copy of an M x K matrix")
    _check_wp(f, wp, N, K, group, has_zp)
    if out is None:
        out = torch.empty((M, N), dtype=xf.dtype, device=xf.device)
    elif out.shape != (M, N) or out.dtype != xf.dtype:
        raise ValueError("out has the wrong shape or dtype")
    ws, wsb, _keep = _workspace(workspace_bytes(f, rung, M, N, K, _dtype_code(xf), X_FRAG), workspace, xf.device)
    st = lib().qgemm_gemm_xf(f, rung, _dev(xf, "xf"), _dev(wp, "wp"), _dev(out, "out"), M, N, K, group,
                             int(bool(has_zp)), _dtype_code(xf), ws, wsb, _stream(stream))
    _check("qgemm_gemm_xf", st)
    return out


#: bytes of the library's fixed device array behind gemm_xf_noalloc
NOALLOC_SCRATCH_BYTES = 16 << 20


def gemm_xf_noalloc(fmt, xf, wp, M: int, N: int, K: int, group: int = 0, has_zp: bool = False, rung: int = -1,
                    out=None, stream=None):
    """gemm_xf for callers that cannot allocate: the split rungs' partial
    sums go to the library's fixed device array (NOALLOC_SCRATCH_BYTES per
    GPU) instead of a workspace; `out` must be given (nothing is allocated)."""
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if out is None:
        raise ValueError("gemm_xf_noalloc allocates nothing: pass out")
    if out.shape != (M, N) or out.dtype != xf.dtype:
        raise ValueError("out has the wrong shape or dtype")
    if xf.numel() < xf_bytes(M, K) // 2:
        raise ValueError("xf is smaller than the fragment-major copy of an M x K matrix")
    _check_wp(f, wp, N, K, group, has_zp)
    st = lib().qgemm_gemm_xf_noalloc(f, rung, _dev(xf, "xf"), _dev(wp, "wp"), _dev(out, "out"), M, N, K, group,
                                     int(bool(has_zp)), _dtype_code(xf), _stream(stream))
    _check("qgemm_gemm_xf_noalloc", st)
    return out


# ---- int8-activation variant ----------------------------------------------

def i8_xq_bytes(M: int, K: int) -> int:
    return int(lib().qgemm_i8_xq_bytes(M, K))


def i8_colscale(fmt, wp, N: int, K: int, group: int = 0, has_zp: bool = False, out=None, stream=None):
    """Per-column int8 requantization factors (r, s) of one packed weight, as
    two float32 device tensors of N elements (computed once at load)."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if out is None:
        out = (torch.empty(N, dtype=torch.float32, device=wp.device),
               torch.empty(N, dtype=torch.float32, device=wp.device))
    rw, sw = out
    if rw.numel() < N or sw.numel() < N or rw.dtype != torch.float32 or sw.dtype != torch.float32:
        raise ValueError("colscale outputs must be float32 with N elements")
    _check_wp(f, wp, N, K, group, has_zp)
    st = lib().qgemm_i8_colscale(f, _dev(wp, "wp"), _dev(rw, "rw"), _dev(sw, "sw"), N, K, group, int(bool(has_zp)),
                                 _stream(stream))
    _check("qgemm_i8_colscale", st)
    return rw, sw


def i8_quantize(x, out=None, stream=None):
    """Row quantization of a row-major [M, K] fp16/bf16 matrix: the int8
    codes in the fragment-major int8 layout (flat int8 tensor of
    32*ceil(M/32)*K bytes) and the per-row scales (float32, M)."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    n = i8_xq_bytes(M, K)
    if n == 0 and M > 0:
        raise QGemmError("qgemm_i8_xq_bytes", -2)
    if out is None:
        out = (torch.empty((n,), dtype=torch.int8, device=x.device), torch.empty((M,), dtype=torch.float32, device=x.device))
    xq, sx = out
    if xq.numel() < n or xq.dtype != torch.int8 or sx.numel() < M or sx.dtype != torch.float32:
        raise ValueError("quantize outputs too small or of the wrong dtype")
    st = lib().qgemm_i8_quantize(_dev(x, "x"), _dev(xq, "xq"), _dev(sx, "sx"), M, K, _dtype_code(x), _stream(stream))
    _check("qgemm_i8_quantize", st)
    return xq, sx


def i8_workspace_bytes(fmt, rung: int, M: int, N: int, K: int) -> int:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return int(lib().qgemm_i8_workspace_bytes(f, rung, M, N, K))


def gemm_i8(fmt, xq, sx, wp, rw, sw, M: int, N: int, K: int, dtype, group: int = 0, has_zp: bool = False,
            rung: int = -1, out=None, stream=None, workspace=None):
    """Y [M, N] (dtype) of the int8 path from i8_quantize's (xq, sx) and
    i8_colscale's (rw, sw) of the packed weight wp."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    tdt = dtype if isinstance(dtype, torch.dtype) else (torch.float16 if dtype == F16 else torch.bfloat16)
    if xq.numel() < i8_xq_bytes(M, K) or sx.numel() < M or rw.numel() < N or sw.numel() < N:
        raise ValueError("int8 inputs are smaller than an M x K / N problem needs")
    _check_wp(f, wp, N, K, group, has_zp)
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=xq.device)
    elif out.shape != (M, N) or out.dtype != tdt:
        raise ValueError("out has the wrong shape or dtype")
    ws, wsb, _keep = _workspace(i8_workspace_bytes(f, rung, M, N, K), workspace, xq.device)
    st = lib().qgemm_i8_gemm(f, rung, _dev(xq, "xq"), _dev(sx, "sx"), _dev(wp, "wp"), _dev(rw, "rw"), _dev(sw, "sw"),
                             _dev(out, "out"), M, N, K, group, int(bool(has_zp)), _dtype_code(out), ws, wsb,
                             _stream(stream))
    _check("qgemm_i8_gemm", st)
    return out


def i8_num_rungs() -> int:
    return int(lib().qgemm_i8_num_rungs())


def i8_rung_name(rung: int):
    r = lib().qgemm_i8_rung_name(rung)
    return None if r is None else r.decode()


def i8_rung_info(rung: int, fmt, M: int, N: int, K: int) -> dict:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    info = np.zeros(8, np.int32)
    _check("qgemm_i8_rung_info", lib().qgemm_i8_rung_info(rung, f, M, N, K, _np_ptr(info)))
    d = dict(zip(_INFO_KEYS, (int(v) for v in info)))
    d["name"] = i8_rung_name(d["rung"])
    return d


def i8_select_rung(fmt, M: int, N: int, K: int) -> dict:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    info = np.zeros(8, np.int32)
    _check("qgemm_i8_select_rung", lib().qgemm_i8_select_rung(f, M, N, K, _np_ptr(info)))
    d = dict(zip(_INFO_KEYS, (int(v) for v in info)))
    d["name"] = i8_rung_name(d["rung"])
    return d


def q4k(x, wp, N: int, out=None, stream=None):
    """Y[M,N] = X[M,K] . dequant_Q4_K(W)."""
    M, K = x.shape
    _check_wp(FMT_Q4K, wp, N, K, 0, False)
    y = _out(x, N, out)
    st = lib().qgemm_q4k(_dev(x, "x"), _dev(wp, "wp"), _dev(y, "out"), M, N, K, _dtype_code(x), _stream(stream))
    _check("qgemm_q4k", st)
    return y


def q6k(x, wp, N: int, out=None, stream=None):
    """Y[M,N] = X[M,K] . dequant_Q6_K(W)."""
    M, K = x.shape
    _check_wp(FMT_Q6K, wp, N, K, 0, False)
    y = _out(x, N, out)
    st = lib().qgemm_q6k(_dev(x, "x"), _dev(wp, "wp"), _dev(y, "out"), M, N, K, _dtype_code(x), _stream(stream))
    _check("qgemm_q6k", st)
    return y


def w4a16(x, wp, N: int, group: int, has_zp: bool, out=None, stream=None):
    """Y[M,N] = X[M,K] . dequant_W4A16(W) (group-wise scale, zero-point or 8)."""
    M, K = x.shape
    _check_wp(FMT_W4A16, wp, N, K, group, has_zp)
    y = _out(x, N, out)
    st = lib().qgemm_w4a16(_dev(x, "x"), _dev(wp, "wp"), _dev(y, "out"), M, N, K, group, int(bool(has_zp)),
                           _dtype_code(x), _stream(stream))
    _check("qgemm_w4a16", st)
    return y


def dequant(fmt, wp, N: int, K: int, dtype, group: int = 0, has_zp: bool = False, stream=None):
    """Staged dequant: logical W[K][N] in fp16/bf16 written by the device unpack."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    code = F16 if dtype in (F16, torch.float16) else BF16
    tdt = torch.float16 if code == F16 else torch.bfloat16
    _check_wp(f, wp, N, K, group, has_zp)
    w = torch.empty((K, N), dtype=tdt, device=wp.device)
    st = lib().qgemm_dequant(f, _dev(wp, "wp"), _dev(w, "out"), N, K, group, int(bool(has_zp)), code,
                             _stream(stream))
    _check("qgemm_dequant", st)
    return w


def grouped(fmt, x, wp, N: int, offsets, E: int, group: int = 0, has_zp: bool = False, out=None, stream=None):
    """Grouped per-expert GEMM: rows offsets[e]..offsets[e+1]-1 of x use
    expert e's packed weights (E experts concatenated in wp); offsets is an
    int32 device tensor of E+1 entries."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [T, K]")
    T, K = x.shape
    _check_wp(f, wp, N, K, group, has_zp, experts=E)
    y = _out(x, N, out)
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.numel() != E + 1:
        raise ValueError("offsets must be an int32 device tensor of E+1 entries")
    st = lib().qgemm_grouped(f, _dev(x, "x"), _dev(wp, "wp"), _dev(y, "out"), _dev(offsets, "offsets"), E, T, N, K,
                             group, int(bool(has_zp)), _dtype_code(x), _stream(stream))
    _check("qgemm_grouped", st)
    return y


def grouped_xf(fmt, xf, wp, T: int, N: int, K: int, offsets, E: int, group: int = 0, has_zp: bool = False, out=None,
               stream=None):
    """:func:`grouped` with the routed rows given as their fragment-major copy
    `xf` (from :func:`x_to_xf` of the [T, K] rows); returns Y [T, N]."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if xf.numel() < xf_bytes(T, K) // 2:
        raise ValueError("xf is smaller than the fragment-major copy of a T x K matrix")
    _check_wp(f, wp, N, K, group, has_zp, experts=E)
    if out is None:
        out = torch.empty((T, N), dtype=xf.dtype, device=xf.device)
    elif tuple(out.shape) != (T, N) or out.dtype != xf.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, N] tensor of xf's dtype")
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.numel() != E + 1:
        raise ValueError("offsets must be an int32 device tensor of E+1 entries")
    st = lib().qgemm_grouped_xf(f, _dev(xf, "xf"), _dev(wp, "wp"), _dev(out, "out"), _dev(offsets, "offsets"), E, T, N,
                                K, group, int(bool(has_zp)), _dtype_code(xf), _stream(stream))
    _check("qgemm_grouped_xf", st)
    return out


def staged_scratch_bytes(N: int, K: int) -> int:
    return int(lib().qgemm_staged_scratch_bytes(N, K))


def staged(fmt, x, wp, N: int, scratch=None, group: int = 0, has_zp: bool = False, out=None, stream=None):
    """The staged arm: unpack into `scratch` (allocated here when None), then
    the 128x128 streaming GEMM on it.  Returns (y, scratch)."""
    torch = _torch()
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    _check_wp(f, wp, N, K, group, has_zp)
    if scratch is None:
        scratch = torch.empty(staged_scratch_bytes(N, K), dtype=torch.uint8, device=x.device)
    y = _out(x, N, out)
    st = lib().qgemm_staged(f, _dev(x, "x"), _dev(wp, "wp"), _dev(scratch, "scratch"),
                            scratch.numel() * scratch.element_size(), _dev(y, "out"), M, N, K, group,
                            int(bool(has_zp)), _dtype_code(x), _stream(stream))
    _check("qgemm_staged", st)
    return y, scratch


# ---------------------------------------------------------------------------
# M-ladder queries
# ---------------------------------------------------------------------------

# The eight integers of qgemm_select_rung / qgemm_rung_info: k_split counts the
# K-split ways inside a workgroup times the K slices across workgroups (the
# split rungs mfma32-64x64-sk and i8-64x64-sk).
_INFO_KEYS = ("rung", "rows", "cols", "k_step", "waves", "k_split", "tiles_n", "tiles_m")


def num_rungs() -> int:
    return int(lib().qgemm_num_rungs())


def rung_name(rung: int):
    r = lib().qgemm_rung_name(rung)
    return None if r is None else r.decode()


def select_rung(fmt, M: int, N: int, K: int, dtype: int = F16) -> dict:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    info = np.zeros(8, np.int32)
    _check("qgemm_select_rung", lib().qgemm_select_rung(f, M, N, K, dtype, _np_ptr(info)))
    d = dict(zip(_INFO_KEYS, (int(v) for v in info)))
    d["name"] = rung_name(d["rung"])
    return d


def select_rung_xf(fmt, M: int, N: int, K: int, dtype: int = F16) -> dict:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    info = np.zeros(8, np.int32)
    _check("qgemm_select_rung_xf", lib().qgemm_select_rung_xf(f, M, N, K, dtype, _np_ptr(info)))
    d = dict(zip(_INFO_KEYS, (int(v) for v in info)))
    d["name"] = rung_name(d["rung"])
    return d


GROUPED_KERNELS = ("direct", "shared")
_GROUPED_KEYS = ("kernel", "rows", "cols", "waves", "kw", "grid_x", "grid_y")


def grouped_plan(T: int, E: int, N: int, K: int) -> dict:
    """The launch :func:`grouped` and :func:`grouped_xf` make for T routed
    rows over E experts of N x K weights (qgemm_grouped_plan); "name" is
    "direct" or "shared"."""
    info = np.zeros(8, np.int32)
    _check("qgemm_grouped_plan", lib().qgemm_grouped_plan(T, E, N, K, _np_ptr(info)))
    d = dict(zip(_GROUPED_KEYS, (int(v) for v in info)))
    d["name"] = GROUPED_KERNELS[d["kernel"]]
    return d


def rung_info(rung: int, fmt, M: int, N: int, K: int, dtype: int = F16) -> dict:
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    info = np.zeros(8, np.int32)
    _check("qgemm_rung_info", lib().qgemm_rung_info(rung, f, M, N, K, dtype, _np_ptr(info)))
    d = dict(zip(_INFO_KEYS, (int(v) for v in info)))
    d["name"] = rung_name(d["rung"])
    return d
