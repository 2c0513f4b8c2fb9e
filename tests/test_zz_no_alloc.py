"""qgemm_gemm_xf_noalloc (the entry point for callers that cannot allocate)
against qgemm_gemm_xf with a caller workspace, through the C ABI: the split
rung at the down projection's shape, then a smaller call on the same fixed
scratch (whose contents the first call left behind), then the ladder's own
choice; Y bit-identical to the workspace entry point's and within the
oracle's bound."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from tests.helpers import Case, assert_gemm_close, from_device, to_device

pytestmark = pytest.mark.gpu

SK = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-64x64-sk"][0]


def _noalloc(c: Case, xf, wp, y, rung: int) -> int:
    import torch

    grp = c.group if c.fmt == "w4a16" else 0
    return qg.lib().qgemm_gemm_xf_noalloc(qg.FORMATS[c.fmt], rung, ctypes.c_void_p(xf.data_ptr()),
                                          ctypes.c_void_p(wp.data_ptr()), ctypes.c_void_p(y.data_ptr()), c.M, c.N,
                                          c.K, grp, int(c.has_zp), c.dtype,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16], ids=["f16", "bf16"])
def test_noalloc_equals_workspace_entry(dtype):
    import torch

    cases = [  # (format, M, N, K, rung): the second smaller than the first, both on the fixed scratch
        ("q6k", 128, 4096, 12288, SK),
        ("q4k", 40, 1552, 8192, SK),
        ("q6k", 64, 4096, 12288, -1),   # the ladder's pick on this layout is the split rung
        ("w4a16", 70, 200, 4096, -1),   # a rung with no partial sums
    ]
    for i, (fmt, M, N, K, rung) in enumerate(cases):
        c = Case(fmt, M, N, K, dtype, seed=990 + i)
        need = qg.workspace_bytes(fmt, rung, M, N, K, dtype, qg.X_FRAG)
        print(f"noalloc {fmt} M={M} N={N} K={K} rung={rung} dtype={dtype} partial sums {need} bytes", flush=True)
        assert need <= qg.NOALLOC_SCRATCH_BYTES
        assert (need > 0) == (i < 3)
        xf = qg.x_to_xf(to_device(c.X, dtype))
        wp = c.device_weights()
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        ref = qg.gemm_xf(fmt, xf, wp, M, N, K, group=c.group if fmt == "w4a16" else 0, has_zp=c.has_zp, rung=rung,
                         workspace=ws)
        y = torch.full((M, N), float("nan"), dtype=ref.dtype, device="cuda")
        assert _noalloc(c, xf, wp, y, rung) == 0
        torch.cuda.synchronize()
        got = from_device(y)
        assert np.array_equal(got, from_device(ref)), f"case {i}: differs from qgemm_gemm_xf"
        Yref, B = oracle.gemm(c.X, c.W, dtype)
        assert_gemm_close(got, Yref, B, dtype, what=f"noalloc case {i}")
