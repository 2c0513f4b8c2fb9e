"""Shared helpers for the GPU parity tests: seeded cases, host<->device
transfers of raw fp16/bf16 bits, and the acceptance rule against the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth

#: normalized error bound on max |Y - Yref| / (|X|.|W|) for fp16/bf16 activations
GEMM_TOL = 2e-3


def torch_dtype(dtype: int):
    import torch

    return torch.float16 if dtype == qg.F16 else torch.bfloat16


def to_device(bits: np.ndarray, dtype: int):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def from_device(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bytes_to_device(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


class Case:
    """One seeded GEMM problem: X bits, the encoded weights, their packed
    device copy and (lazily) the oracle's unpacked W[K][N] bits."""

    def __init__(self, fmt: str, M: int, N: int, K: int, dtype: int, seed: int, group: int = 128,
                 symmetric: bool = False, fields=None, X=None):
        self.fmt, self.M, self.N, self.K, self.dtype = fmt, M, N, K, dtype
        self.group, self.symmetric = group, symmetric
        rx, rw = synth.streams(seed, 2)
        self.X = X if X is not None else synth.activations(rx, M, K, dtype)
        self.fields = fields if fields is not None else synth.weight_fields(fmt, rw, N, K, group, symmetric)
        self.enc = synth.encode(fmt, self.fields)
        self.packed = qg.pack(fmt, self.enc, N, K)
        self._W = None
        self.has_zp = fmt == "w4a16" and not symmetric

    @property
    def W(self) -> np.ndarray:
        if self._W is None:
            self._W = oracle.dequant(self.fmt, self.enc, self.N, self.K, self.dtype)
        return self._W

    def device_weights(self):
        return bytes_to_device(self.packed)

    def run(self, rung: int = -1, x_bits=None, wp=None, out=None):
        x = to_device(self.X if x_bits is None else x_bits, self.dtype)
        wp = self.device_weights() if wp is None else wp
        return qg.gemm_rung(self.fmt, rung, x, wp, self.N, group=self.group if self.fmt == "w4a16" else 0,
                            has_zp=self.has_zp, out=out)


    def run_xf(self, rung: int = -1, out=None):
        """The same product through the fragment-major path: the library's
        own copy of X (qgemm_x_to_xf), then qgemm_gemm_xf."""
        xf = qg.x_to_xf(to_device(self.X, self.dtype))
        return qg.gemm_xf(self.fmt, xf, self.device_weights(), self.M, self.N, self.K,
                          group=self.group if self.fmt == "w4a16" else 0, has_zp=self.has_zp, rung=rung, out=out)


def ulp_half(y: np.ndarray, dtype: int) -> np.ndarray:
    """Half an ulp of |y| in the output type (the output rounding alone)."""
    a = np.abs(y)
    if dtype == qg.F16:
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return 2.0 ** (e - 10) / 2
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7) / 2


def assert_gemm_close(Y_bits: np.ndarray, Yref: np.ndarray, B: np.ndarray, dtype: int, allow_out_ulp=False,
                      what=""):
    """max |Y - Yref| / B <= GEMM_TOL; outputs with B == 0 must be exactly 0.
    allow_out_ulp adds half an output ulp to the allowance (all-positive
    special cases, where bf16 output rounding alone can exceed the bound)."""
    Y = oracle.bits_to_double_fast(Y_bits, dtype)
    assert np.all(np.isfinite(Y)), f"{what}: non-finite outputs"
    err = np.abs(Y - Yref)
    allow = GEMM_TOL * B + (ulp_half(Yref, dtype) if allow_out_ulp else 0.0)
    zero = B == 0
    assert np.all(Y[zero] == 0), f"{what}: nonzero output where |X|.|W| is 0"
    bad = err > allow
    if bad.any():
        idx = np.argwhere(bad)[:5]
        with np.errstate(divide="ignore", invalid="ignore"):
            worst = float(np.nanmax(np.where(zero, 0, err / np.where(zero, 1, B))))
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of bound; worst rel {worst:.3e}; "
                             f"first {idx.tolist()}")
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.max(np.where(zero, 0, err / np.where(zero, 1, B)))) if err.size else 0.0


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit equality of fp16/bf16 patterns with +0 and -0 taken as equal."""
    a = np.where((a & 0x7FFF) == 0, 0, a)
    b = np.where((b & 0x7FFF) == 0, 0, b)
    return bool(np.array_equal(a, b))


def fnv1a64(bits: np.ndarray) -> int:
    """FNV-1a over the raw 16-bit patterns (little-endian bytes), signed zeros
    folded to +0 -- a one-number summary of a dequantized tensor."""
    b = np.where((bits & 0x7FFF) == 0, 0, bits).astype("<u2").tobytes()
    h = 0xCBF29CE484222325
    for byte in b:
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h
