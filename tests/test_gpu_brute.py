"""Brute force over a grid of tiny shapes, through the format entry points
(row-major X) and the fragment-major path, on the automatic ladder.

M runs over the edges of every rung's tiles (1..3, 15..17, 31..33, 63..65,
127..129, 255, 257) and the prompt length of the layer workload (658); N
over one to ten panels; K over one to three Q4_K/Q6_K super-blocks (W4A16:
one to three 128-wide groups).  For each (format, N, K, dtype) one seeded
658-row problem is built and the oracle run once: row m of Y depends on row
m of X only, so each smaller M is the leading rows of the same X and its Y is
checked against the leading rows of that one oracle product.  That is also
the ladder-consistency check: the same rows computed at M = 658 (streaming
tiles) and at M = 1 or 16 (direct kernels) must both meet the bound against
one reference.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from tests.helpers import Case, assert_gemm_close, from_device, to_device

pytestmark = pytest.mark.gpu

MS = [1, 2, 3, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 658]
NS = [16, 32, 48, 64, 96, 128, 160]
KS = {"q4k": [256, 512, 768], "q6k": [256, 512, 768], "w4a16": [128, 256, 384]}
FMTS = [("q4k", False), ("q6k", False), ("w4a16", False), ("w4a16", True)]
FMT_IDS = ["q4k", "q6k", "w4a16-asym", "w4a16-sym"]


def _format_call(c: Case, x):
    if c.fmt == "q4k":
        return qg.q4k(x, c.device_weights(), c.N)
    if c.fmt == "q6k":
        return qg.q6k(x, c.device_weights(), c.N)
    return qg.w4a16(x, c.device_weights(), c.N, c.group, c.has_zp)


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16], ids=["f16", "bf16"])
def test_tiny_shape_grid(fmt, sym, dtype):
    Mmax = max(MS)
    checked = 0
    for ik, K in enumerate(KS[fmt]):
        for jn, N in enumerate(NS):
            c = Case(fmt, Mmax, N, K, dtype, seed=3000 + 10 * ik + jn, symmetric=sym)
            Yref, B = oracle.gemm(c.X, c.W, dtype)
            wp = c.device_weights()
            for M in MS:
                what = f"{fmt} sym={sym} dtype={dtype} M={M} N={N} K={K}"
                print("brute", what, flush=True)
                x = to_device(c.X[:M], dtype)
                y_row = from_device(_format_call(c, x))
                assert_gemm_close(y_row, Yref[:M], B[:M], dtype, what=what + " row-major")
                xf = qg.x_to_xf(x)
                y_xf = from_device(qg.gemm_xf(fmt, xf, wp, M, N, K, group=c.group if fmt == "w4a16" else 0,
                                              has_zp=c.has_zp))
                assert_gemm_close(y_xf, Yref[:M], B[:M], dtype, what=what + " fragment-major")
                checked += 2
    assert checked == 2 * len(KS[fmt]) * len(NS) * len(MS)
