"""The automatic ladder at mid and large M, through the entry points a caller
uses (the format calls on row-major X, qgemm_gemm_xf on fragment-major X):
each shape is one where the round model or the large-tile costs pick a
particular rung (asserted first, so the case keeps covering that rung), and
the product is checked against the oracle on a seeded sample of outputs
(first and last rows and columns included).  The expected rungs are the
measured winners on MI355X that the host tests pin as well."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from tests.helpers import GEMM_TOL, Case, from_device, to_device

pytestmark = pytest.mark.gpu

# (format, layout, dtype, M, N, K, rung the ladder picks)
SHAPES = [
    ("q4k", "xf", qg.F16, 320, 1024, 4096, "mfma32-64x32-k4"),       # one round of 64x32 tiles over few panels
    ("w4a16", "xf", qg.BF16, 48, 6144, 4096, "mfma32-64x32-k4"),     # decode-adjacent, 384 panels
    ("q4k", "xf", qg.F16, 100, 4096, 11008, "mfma32-64x32-k4"),      # 86 chunks: two K groups of 43
    ("q6k", "xf", qg.BF16, 160, 4096, 4096, "mfma32-96x32-k4"),      # one round of 96-row tiles
    ("w4a16", "xf", qg.F16, 384, 4096, 4096, "mfma32-128x64-k2"),    # one round of 128-row tiles
    ("q4k", "row", qg.BF16, 96, 12288, 4096, "mfma32-128x64-k2"),    # row-major, 768 panels
    ("q6k", "row", qg.F16, 64, 2048, 4096, "direct-skinny-n"),       # row-major: 16 rows, four panels per wave
    ("q4k", "xf", qg.F16, 1500, 12288, 4096, "mfma32-768x96"),       # one round of 768x96 tiles (96x96 waves)
    ("q6k", "xf", qg.BF16, 1500, 12288, 4096, "mfma32-768x96"),      # Q6_K bf16 (its 96x96 waves spill a few VGPRs)
    ("q4k", "xf", qg.BF16, 3072, 4096, 4096, "mfma32-512x128"),      # 64x128 waves
    ("w4a16", "xf", qg.F16, 1024, 12288, 4096, "mfma32-512x96"),     # 64x96 waves
    ("q6k", "row", qg.F16, 700, 12288, 4096, "mfma32-352x96"),       # row-major Q6_K: the 352-row tile
    ("q6k", "row", qg.F16, 3072, 12288, 4096, "mfma16-256x128"),     # row-major Q6_K from 512 256-row tiles
]


def _ids():
    return [f"{f}-{l}-{'f16' if d == qg.F16 else 'bf16'}-M{M}-N{N}-K{K}" for f, l, d, M, N, K, _ in SHAPES]


@pytest.mark.parametrize("fmt,layout,dtype,M,N,K,rung", SHAPES, ids=_ids())
def test_auto_ladder_sampled(fmt, layout, dtype, M, N, K, rung):
    sel = (qg.select_rung_xf if layout == "xf" else qg.select_rung)(fmt, M, N, K, dtype)
    assert sel["name"] == rung, (fmt, layout, M, N, K, sel)
    print(f"auto {fmt} {layout} dtype={dtype} M={M} N={N} K={K} rung={rung}", flush=True)
    c = Case(fmt, M, N, K, dtype, seed=7100 + M + N // 16)
    if layout == "xf":
        y = c.run_xf()
    else:
        x = to_device(c.X, dtype)
        wp = c.device_weights()
        y = {"q4k": lambda: qg.q4k(x, wp, N), "q6k": lambda: qg.q6k(x, wp, N),
             "w4a16": lambda: qg.w4a16(x, wp, N, c.group, c.has_zp)}[fmt]()
    Y = from_device(y)
    rng = np.random.default_rng(9100 + M)
    count = 1500
    rows = np.concatenate([rng.integers(0, M, count), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, count), [0, N - 1, 0, N - 1]])
    Yref, B = oracle.gemm_at(c.X, c.W, dtype, rows, cols)
    got = oracle.bits_to_double_fast(Y[rows, cols], dtype)
    assert np.all(np.isfinite(oracle.bits_to_double_fast(Y, dtype)))
    rel = np.abs(got - Yref) / B
    print(f"  max rel err {rel.max():.3e}", flush=True)
    assert rel.max() <= GEMM_TOL
