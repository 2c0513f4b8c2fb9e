"""CPU oracle for the quantized-weight prefill linear layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``libqref.so`` (plain C, see
``qref.c``) with numpy in and out and shares nothing with the HIP library.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` (library roundings, exact rationals, closed forms,
special cases, brute force); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqref.so")
_lib = None

F16 = 0
BF16 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b

        _b.build()
    _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """Open a build of qref.c and declare its C signatures."""
    lib = ctypes.CDLL(path)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    c_dp = ctypes.POINTER(ctypes.c_double)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    c_fp = ctypes.POINTER(ctypes.c_float)
    c_i8p = ctypes.POINTER(ctypes.c_int8)
    i64 = ctypes.c_int64
    sig = {
        "qref_rn_f16": (ctypes.c_uint16, [ctypes.c_double]),
        "qref_rn_bf16": (ctypes.c_uint16, [ctypes.c_double]),
        "qref_rn_f32": (ctypes.c_double, [ctypes.c_double]),
        "qref_f16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "qref_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "qref_q4k_fields": (None, [c_u8p, c_u16p, c_u16p, c_u8p, c_u8p, c_u8p]),
        "qref_q6k_fields": (None, [c_u8p, c_u16p, ctypes.POINTER(ctypes.c_int8), c_u8p]),
        "qref_q4k_weight": (ctypes.c_int, [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, c_u16p]),
        "qref_q6k_weight": (ctypes.c_int, [ctypes.c_uint16, ctypes.c_int, ctypes.c_int, ctypes.c_int, c_u16p]),
        "qref_w4a16_weight": (ctypes.c_int, [ctypes.c_uint16, ctypes.c_int, ctypes.c_int, ctypes.c_int, c_u16p]),
        "qref_dequant_q4k": (ctypes.c_int, [c_u8p, i64, i64, ctypes.c_int, c_u16p]),
        "qref_fragment_major": (ctypes.c_int, [c_u16p, i64, i64, c_u16p]),
        "qref_dequant_q6k": (ctypes.c_int, [c_u8p, i64, i64, ctypes.c_int, c_u16p]),
        "qref_dequant_w4a16": (ctypes.c_int, [c_u8p, c_u16p, c_u8p, i64, i64, i64, ctypes.c_int, c_u16p]),
        "qref_gemm": (ctypes.c_int, [c_u16p, c_u16p, i64, i64, i64, ctypes.c_int, c_dp, c_dp]),
        "qref_gemm_at": (ctypes.c_int, [c_u16p, c_u16p, i64, i64, i64, ctypes.c_int, c_i64p, c_i64p, i64,
                                        c_dp, c_dp]),
        "qref_num_threads": (ctypes.c_int, []),
        "qref_set_num_threads": (None, [ctypes.c_int]),
        "qref_dequant_q4k_f32": (ctypes.c_int, [c_u8p, i64, i64, c_fp]),
        "qref_dequant_q6k_f32": (ctypes.c_int, [c_u8p, i64, i64, c_fp]),
        "qref_dequant_w4a16_f32": (ctypes.c_int, [c_u8p, c_u16p, c_u8p, i64, i64, i64, c_fp]),
        "qref_colscale_i8": (ctypes.c_int, [c_fp, i64, i64, c_fp, c_fp]),
        "qref_requant_i8": (ctypes.c_int, [c_fp, c_fp, i64, i64, c_i8p]),
        "qref_quant_rows_i8": (ctypes.c_int, [c_u16p, i64, i64, ctypes.c_int, c_i8p, c_fp]),
        "qref_gemm_i8": (ctypes.c_int, [c_i8p, c_fp, c_i8p, c_fp, i64, i64, i64, ctypes.c_int, c_u16p]),
        "qref_fragment_major_i8": (ctypes.c_int, [c_i8p, i64, i64, c_i8p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar roundings and conversions -------------------------------------

def rn_f16(x: float) -> int:
    return int(_load().qref_rn_f16(float(x)))


def rn_bf16(x: float) -> int:
    return int(_load().qref_rn_bf16(float(x)))


def rn_f32(x: float) -> float:
    return float(_load().qref_rn_f32(float(x)))


def f16_to_double(h: int) -> float:
    return float(_load().qref_f16_to_double(int(h)))


def bf16_to_double(b: int) -> float:
    return float(_load().qref_bf16_to_double(int(b)))


def bits_to_double(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Vectorised fp16/bf16 bits -> float64 (via the oracle's own decoders)."""
    lib = _load()
    f = lib.qref_f16_to_double if dtype == F16 else lib.qref_bf16_to_double
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.fromiter((f(int(v)) for v in flat), dtype=np.float64, count=flat.size)
    return out.reshape(np.shape(bits))


# ---- field decode ---------------------------------------------------------

def q4k_fields(block: np.ndarray) -> dict:
    blk = _c(block, np.uint8)
    assert blk.size == 144
    d = np.zeros(1, np.uint16)
    dm = np.zeros(1, np.uint16)
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    q = np.zeros(256, np.uint8)
    _load().qref_q4k_fields(_p(blk, ctypes.c_uint8), _p(d, ctypes.c_uint16), _p(dm, ctypes.c_uint16),
                            _p(sc, ctypes.c_uint8), _p(mn, ctypes.c_uint8), _p(q, ctypes.c_uint8))
    return {"d": int(d[0]), "dmin": int(dm[0]), "sc": sc, "m": mn, "q": q}


def q6k_fields(block: np.ndarray) -> dict:
    blk = _c(block, np.uint8)
    assert blk.size == 210
    d = np.zeros(1, np.uint16)
    s = np.zeros(16, np.int8)
    q = np.zeros(256, np.uint8)
    _load().qref_q6k_fields(_p(blk, ctypes.c_uint8), _p(d, ctypes.c_uint16), _p(s, ctypes.c_int8),
                            _p(q, ctypes.c_uint8))
    return {"d": int(d[0]), "s": s, "q": q}


# ---- single weights -------------------------------------------------------

def q4k_weight(d: int, dmin: int, sc: int, m: int, q: int, dtype: int) -> int:
    out = np.zeros(1, np.uint16)
    rc = _load().qref_q4k_weight(d, dmin, sc, m, q, dtype, _p(out, ctypes.c_uint16))
    if rc:
        raise ValueError("non-finite scale")
    return int(out[0])


def q6k_weight(d: int, s: int, q: int, dtype: int) -> int:
    out = np.zeros(1, np.uint16)
    if _load().qref_q6k_weight(d, s, q, dtype, _p(out, ctypes.c_uint16)):
        raise ValueError("non-finite scale")
    return int(out[0])


def w4a16_weight(s: int, q: int, zp: int, dtype: int) -> int:
    out = np.zeros(1, np.uint16)
    if _load().qref_w4a16_weight(s, q, zp, dtype, _p(out, ctypes.c_uint16)):
        raise ValueError("non-finite scale")
    return int(out[0])


# ---- whole-matrix dequant into logical W[K][N] (bits of dtype) -------------

def dequant_q4k(blocks: np.ndarray, N: int, K: int, dtype: int) -> np.ndarray:
    b = _c(blocks, np.uint8)
    assert b.size == N * (K // 256) * 144
    W = np.empty((K, N), np.uint16)
    rc = _load().qref_dequant_q4k(_p(b, ctypes.c_uint8), N, K, dtype, _p(W, ctypes.c_uint16))
    if rc:
        raise ValueError(f"qref_dequant_q4k failed ({rc})")
    return W


def dequant_q6k(blocks: np.ndarray, N: int, K: int, dtype: int) -> np.ndarray:
    b = _c(blocks, np.uint8)
    assert b.size == N * (K // 256) * 210
    W = np.empty((K, N), np.uint16)
    rc = _load().qref_dequant_q6k(_p(b, ctypes.c_uint8), N, K, dtype, _p(W, ctypes.c_uint16))
    if rc:
        raise ValueError(f"qref_dequant_q6k failed ({rc})")
    return W


def dequant_w4a16(codes: np.ndarray, scales: np.ndarray, zeros, N: int, K: int, group: int,
                  dtype: int) -> np.ndarray:
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint16)
    assert c.size == N * K and s.size == (K // group) * N
    z = None if zeros is None else _c(zeros, np.uint8)
    W = np.empty((K, N), np.uint16)
    zp = _p(z, ctypes.c_uint8) if z is not None else ctypes.POINTER(ctypes.c_uint8)()
    rc = _load().qref_dequant_w4a16(_p(c, ctypes.c_uint8), _p(s, ctypes.c_uint16), zp, N, K, group, dtype,
                                    _p(W, ctypes.c_uint16))
    if rc:
        raise ValueError(f"qref_dequant_w4a16 failed ({rc})")
    return W


def dequant(fmt: str, enc, N: int, K: int, dtype: int) -> np.ndarray:
    """Logical W[K][N] for the bytes/fields the synthetic generator produced."""
    if fmt == "q4k":
        return dequant_q4k(enc, N, K, dtype)
    if fmt == "q6k":
        return dequant_q6k(enc, N, K, dtype)
    if fmt == "w4a16":
        zeros = None if enc["symmetric"] else enc["zeros"]
        return dequant_w4a16(enc["codes"], enc["scales"], zeros, N, K, enc["group"], dtype)
    raise ValueError(fmt)


# ---- fp64 GEMM -------------------------------------------------------------

def gemm(X: np.ndarray, W: np.ndarray, dtype: int, want_bound: bool = True):
    """fp64 Y = X . W and B = |X| . |W| for bit-pattern inputs X[M][K], W[K][N]."""
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2
    Y = np.empty((M, N), np.float64)
    B = np.empty((M, N), np.float64) if want_bound else None
    rc = _load().qref_gemm(_p(X, ctypes.c_uint16), _p(W, ctypes.c_uint16), M, N, K, dtype, _p(Y, ctypes.c_double),
                           _p(B, ctypes.c_double) if B is not None else ctypes.POINTER(ctypes.c_double)())
    if rc:
        raise MemoryError(f"qref_gemm failed ({rc})")
    return Y, B


def gemm_at(X: np.ndarray, W: np.ndarray, dtype: int, rows, cols):
    """fp64 Y and B at chosen (row, column) pairs only."""
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    M, K = X.shape
    _, N = W.shape
    r = _c(rows, np.int64)
    c = _c(cols, np.int64)
    assert r.shape == c.shape
    Y = np.empty(r.size, np.float64)
    B = np.empty(r.size, np.float64)
    rc = _load().qref_gemm_at(_p(X, ctypes.c_uint16), _p(W, ctypes.c_uint16), M, N, K, dtype, _p(r, ctypes.c_int64),
                              _p(c, ctypes.c_int64), r.size, _p(Y, ctypes.c_double), _p(B, ctypes.c_double))
    if rc:
        raise ValueError(f"qref_gemm_at failed ({rc})")
    return Y, B


# ---- activation layout of the library under test --------------------------

def fragment_major(X: np.ndarray) -> np.ndarray:
    """The fragment-major copy of the bit patterns X [M][K] (flat, uint16,
    32*ceil(M/32)*K elements): an activation layout of the library under test,
    not a step of the pages' computation; see qref.c, item 4."""
    X = _c(X, np.uint16)
    M, K = X.shape
    out = np.full(((M + 31) // 32) * 32 * K, 0xFFFF, np.uint16)  # every element is written below
    if _load().qref_fragment_major(_p(X, ctypes.c_uint16), M, K, _p(out, ctypes.c_uint16)):
        raise ValueError(f"fragment_major: K = {K} is not a positive multiple of 128")
    return out


# ---- int8-activation variant (qref.c, item 5) -----------------------------

def dequant_f32(fmt: str, enc, N: int, K: int) -> np.ndarray:
    """Logical W[K][N] as binary32: the exact weight rounded once (float32)."""
    W = np.empty((K, N), np.float32)
    lib = _load()
    if fmt == "q4k":
        b = _c(enc, np.uint8)
        assert b.size == N * (K // 256) * 144
        rc = lib.qref_dequant_q4k_f32(_p(b, ctypes.c_uint8), N, K, _p(W, ctypes.c_float))
    elif fmt == "q6k":
        b = _c(enc, np.uint8)
        assert b.size == N * (K // 256) * 210
        rc = lib.qref_dequant_q6k_f32(_p(b, ctypes.c_uint8), N, K, _p(W, ctypes.c_float))
    elif fmt == "w4a16":
        codes = _c(enc["codes"], np.uint8)
        scales = _c(enc["scales"], np.uint16)
        group = int(enc["group"])
        assert codes.size == N * K and scales.size == (K // group) * N
        z = None if enc["symmetric"] else _c(enc["zeros"], np.uint8)
        zp = _p(z, ctypes.c_uint8) if z is not None else ctypes.POINTER(ctypes.c_uint8)()
        rc = lib.qref_dequant_w4a16_f32(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint16), zp, N, K,
                                        group, _p(W, ctypes.c_float))
    else:
        raise ValueError(f"unknown format {fmt!r}")
    if rc:
        raise ValueError(f"dequant_f32({fmt}) failed ({rc})")
    return W


def colscale_i8(W32: np.ndarray):
    """Per-column (r, s) of binary32 weights W32 [K][N]: r = RN_f32(127/amax),
    s = RN_f32(amax/127), both 0 for an all-zero column."""
    W32 = _c(W32, np.float32)
    K, N = W32.shape
    r = np.empty(N, np.float32)
    s = np.empty(N, np.float32)
    if _load().qref_colscale_i8(_p(W32, ctypes.c_float), N, K, _p(r, ctypes.c_float), _p(s, ctypes.c_float)):
        raise ValueError("colscale_i8 failed")
    return r, s


def requant_i8(W32: np.ndarray, r: np.ndarray) -> np.ndarray:
    """int8 weight codes [K][N] = RNE_int(W32 * r[n]) (exact product)."""
    W32 = _c(W32, np.float32)
    r = _c(r, np.float32)
    K, N = W32.shape
    Q = np.empty((K, N), np.int8)
    if _load().qref_requant_i8(_p(W32, ctypes.c_float), _p(r, ctypes.c_float), N, K, _p(Q, ctypes.c_int8)):
        raise ValueError("requant_i8 failed")
    return Q


def quant_rows_i8(X: np.ndarray, dtype: int):
    """Row quantization of the bit patterns X [M][K]: codes [M][K] (int8) and
    the per-row scale s = RN_f32(amax/127) (float32)."""
    X = _c(X, np.uint16)
    M, K = X.shape
    Q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    if _load().qref_quant_rows_i8(_p(X, ctypes.c_uint16), M, K, dtype, _p(Q, ctypes.c_int8), _p(s, ctypes.c_float)):
        raise ValueError("quant_rows_i8: input holds inf or nan")
    return Q, s


def gemm_i8(Qx: np.ndarray, sx: np.ndarray, Qw: np.ndarray, sw: np.ndarray, dtype: int) -> np.ndarray:
    """Y [M][N] bit patterns of dtype: RN_t(RN_f32(RN_f32(acc) * RN_f32(sx*sw)))
    with acc = sum_k Qx[m][k] * Qw[k][n] exactly."""
    Qx = _c(Qx, np.int8)
    Qw = _c(Qw, np.int8)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, K = Qx.shape
    K2, N = Qw.shape
    assert K == K2
    Y = np.empty((M, N), np.uint16)
    if _load().qref_gemm_i8(_p(Qx, ctypes.c_int8), _p(sx, ctypes.c_float), _p(Qw, ctypes.c_int8),
                            _p(sw, ctypes.c_float), M, N, K, dtype, _p(Y, ctypes.c_uint16)):
        raise ValueError("gemm_i8 failed")
    return Y


def fragment_major_i8(Q: np.ndarray) -> np.ndarray:
    """The int8 activation codes [M][K] in the library's fragment-major int8
    layout (flat, 32*ceil(M/32)*K bytes); see qref.c, item 5."""
    Q = _c(Q, np.int8)
    M, K = Q.shape
    out = np.full(((M + 31) // 32) * 32 * K, 0x55, np.int8)  # every byte is written below
    if _load().qref_fragment_major_i8(_p(Q, ctypes.c_int8), M, K, _p(out, ctypes.c_int8)):
        raise ValueError(f"fragment_major_i8: K = {K} is not a positive multiple of 32")
    return out


def num_threads() -> int:
    return int(_load().qref_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing only)."""
    _load().qref_set_num_threads(int(n))


# ---- acceptance rule -------------------------------------------------------

def gemm_error(Y_bits: np.ndarray, Yref: np.ndarray, B: np.ndarray, dtype: int):
    """max |Y - Yref| / B over all outputs, and whether every B == 0 output is 0."""
    Y = bits_to_double_fast(Y_bits, dtype)
    err = np.abs(Y - Yref)
    zero = B == 0
    ok_zero = bool(np.all(Y[zero] == 0)) if zero.any() else True
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, err / np.where(zero, 1.0, B))
    return float(rel.max()) if rel.size else 0.0, ok_zero


def bits_to_double_fast(bits: np.ndarray, dtype: int) -> np.ndarray:
    """fp16/bf16 bit patterns -> float64 via numpy's own views (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
