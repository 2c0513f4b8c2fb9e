"""Full-size parity for every named workload, in the launch configuration the
benchmark times (the automatic rung).  The oracle dequantizes all of W and
computes a seeded sample of outputs one by one; the sample always includes
the first and last row and column so the M and N tails are covered."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests.helpers import GEMM_TOL, bytes_to_device, from_device, to_device

pytestmark = pytest.mark.gpu

CASES = [(name, j) for name, w in synth.WORKLOADS.items() for j in range(len(w["gemms"]))]


@pytest.mark.parametrize("name,j", CASES, ids=[f"{n}-{synth.WORKLOADS[n]['gemms'][j][0]}" for n, j in CASES])
def test_workload_sampled(name, j):
    label, fmt, M, K, N, dt, group, sym = synth.WORKLOADS[name]["gemms"][j]
    print(f"fullsize {name}/{label} fmt={fmt} M={M} K={K} N={N} dtype={dt}", flush=True)
    X, fields, enc = synth.workload_inputs(name, j)
    packed = qg.pack(fmt, enc, N, K)
    x = to_device(X, dt)
    wp = bytes_to_device(packed)
    if fmt == "q4k":
        y = qg.q4k(x, wp, N)
    elif fmt == "q6k":
        y = qg.q6k(x, wp, N)
    else:
        y = qg.w4a16(x, wp, N, group, not sym)
    Y = from_device(y)
    W = oracle.dequant(fmt, enc, N, K, dt)
    rng = np.random.default_rng(4242 + j)
    count = 3000
    rows = np.concatenate([rng.integers(0, M, count), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, count), [0, N - 1, 0, N - 1]])
    Yref, B = oracle.gemm_at(X, W, dt, rows, cols)
    got = oracle.bits_to_double_fast(Y[rows, cols], dt)
    assert np.all(np.isfinite(oracle.bits_to_double_fast(Y, dt)))
    rel = np.abs(got - Yref) / B
    print(f"  max rel err {rel.max():.3e}", flush=True)
    assert rel.max() <= GEMM_TOL
