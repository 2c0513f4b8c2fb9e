"""Binding of libqprobe.so (include/qprobe.h): the MFMA-rate and streaming-
read probes the benchmark measures the GEMMs against.  Measurement aids, not
part of the GEMM library."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqprobe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with `python -m quantized_weight_prefill_amd.build`")
        import torch  # noqa: F401  (one HIP runtime in the process, as for libqgemm.so)

        h = ctypes.CDLL(LIB_PATH)
        h.qprobe_mfma.restype = ctypes.c_int
        h.qprobe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
        h.qprobe_read.restype = ctypes.c_int
        h.qprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        _lib = h
    return _lib


def _stream(stream):
    import torch

    return ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream().cuda_stream)


def mfma(operands, out, blocks: int, iters: int, dtype: int = 0, stream=None):
    """Launch the MFMA rate probe (fp16 dtype 0, bf16 dtype 1)."""
    st = lib().qprobe_mfma(ctypes.c_void_p(operands.data_ptr()), ctypes.c_void_p(out.data_ptr()), blocks, iters,
                           dtype, _stream(stream))
    if st != 0:
        raise RuntimeError(f"qprobe_mfma: status {st}")


def read(buf, out, blocks: int, stream=None):
    """Launch the streaming-read probe over all of `buf`."""
    st = lib().qprobe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                           ctypes.c_void_p(out.data_ptr()), blocks, _stream(stream))
    if st != 0:
        raise RuntimeError(f"qprobe_read: status {st}")
