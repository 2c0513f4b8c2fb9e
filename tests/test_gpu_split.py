"""GPU parity of the rung that splits K across workgroups (64x64 tiles, fp32
partial sums per K slice, then one ordered reduction): against the oracle at
K long enough for two, four and eight slices, with ragged M and N, on both
activation layouts and through the automatic ladder at the down projection's
shape, and bit-identical from call to call and between layouts.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from tests.helpers import Case, assert_gemm_close, from_device, to_device

pytestmark = pytest.mark.gpu

SK = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-64x64-sk"][0]


@pytest.mark.parametrize("fmt,M,N,K,dtype,slices", [
    ("q4k", 37, 200, 4096, qg.F16, 2),      # 13 panels (the last ragged), 37 rows of a 64-row tile
    ("w4a16", 64, 256, 4096, qg.BF16, 2),
    ("q6k", 96, 130, 12288, qg.F16, 4),     # two row tiles, 9 panels
    ("q6k", 5, 64, 16384, qg.BF16, 8),
])
def test_split_rung_forced(fmt, M, N, K, dtype, slices):
    c = Case(fmt, M, N, K, dtype, seed=700 + M, group=128)
    info = qg.rung_info(SK, fmt, M, N, K, dtype)
    print(f"split forced {fmt} M={M} N={N} K={K} dtype={dtype} info={info}", flush=True)
    assert info["k_split"] == 4 * slices, info
    Yref, B = oracle.gemm(c.X, c.W, dtype)
    y = from_device(c.run(SK))
    assert_gemm_close(y, Yref, B, dtype, what=f"split {fmt} M={M} N={N} K={K}")
    yx = from_device(c.run_xf(SK))
    assert np.array_equal(y, yx), "row-major and fragment-major activations differ"
    assert np.array_equal(y, from_device(c.run(SK))), "not reproducible from call to call"


@pytest.mark.parametrize("M", [40, 64, 96, 128])
def test_split_rung_auto_down_projection(M):
    """Q6_K 12288 -> 4096 on fragment-major activations through the ladder:
    at 33..64 rows the split rung (four slices of 24 chunks, each split over
    four K groups), at 65..128 rows the 64x32 tiles with K split four ways
    inside the workgroup."""
    N, K = 4096, 12288
    sel = qg.select_rung_xf("q6k", M, N, K, qg.F16)
    if M <= 64:
        assert sel["name"] == "mfma32-64x64-sk" and sel["k_split"] == 16, sel
    else:
        assert sel["name"] == "mfma32-64x32-k4" and sel["k_split"] == 4, sel
    c = Case("q6k", M, N, K, qg.F16, seed=720 + M)
    print(f"split auto q6k M={M} N={N} K={K}", flush=True)
    y = from_device(c.run_xf(-1))
    Yref, B = oracle.gemm(c.X, c.W, qg.F16)
    assert_gemm_close(y, Yref, B, qg.F16, what=f"split auto M={M}")
    assert np.array_equal(y, from_device(c.run_xf(-1)))


SK768 = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-768x64-sk"][0]


@pytest.mark.parametrize("fmt,M,N,K,dtype,slices", [
    ("q6k", 600, 200, 4096, qg.F16, 8),       # 13 panels (the last ragged) in 4 column tiles, 4 chunks a slice
    ("q4k", 530, 128, 2048, qg.BF16, 8),      # 2 chunks a slice
    ("w4a16", 100, 320, 1536, qg.F16, 4),     # 100 rows of a 768-row tile, 3 chunks a slice
    ("q4k", 800, 64, 2048, qg.F16, 8),        # two row tiles, the second 32 rows
])
def test_split768_rung_forced(fmt, M, N, K, dtype, slices):
    """The 768x64 tiles (8 waves of 96x64) with K split across workgroups:
    ragged rows and columns, slices of two to four chunks, both layouts."""
    c = Case(fmt, M, N, K, dtype, seed=760 + M, group=128)
    info = qg.rung_info(SK768, fmt, M, N, K, dtype)
    print(f"split768 forced {fmt} M={M} N={N} K={K} dtype={dtype} info={info}", flush=True)
    assert (info["k_split"], info["rows"], info["cols"]) == (slices, 768, 64), info
    Yref, B = oracle.gemm(c.X, c.W, dtype)
    y = from_device(c.run_xf(SK768))
    assert_gemm_close(y, Yref, B, dtype, what=f"split768 {fmt} M={M} N={N} K={K}")
    assert np.array_equal(y, from_device(c.run(SK768))), "row-major and fragment-major activations differ"
    assert np.array_equal(y, from_device(c.run_xf(SK768))), "not reproducible from call to call"


def _ws(nbytes: int, guard: int = 0):
    import torch

    return torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")


def test_split_workspace_caller_owned_sizes():
    """The caller's workspace, sized by qgemm_workspace_bytes, for calls that
    need more, then less, than the previous one: every result meets the
    bound, and nothing past the stated size is written (a guard band of 4 KB
    after it keeps its pattern).  A workspace one slice short is refused."""
    import torch

    for i, (M, N, K) in enumerate([(8, 64, 4096), (64, 512, 8192), (16, 80, 4096)]):
        c = Case("q4k", M, N, K, qg.F16, seed=740 + i)
        need = qg.workspace_bytes("q4k", SK, M, N, K)
        print(f"split workspace M={M} N={N} K={K} bytes={need}", flush=True)
        assert need > 0
        ws = _ws(need, 4096)
        x = to_device(c.X, c.dtype)
        wp = c.device_weights()
        y = qg.gemm_rung("q4k", SK, x, wp, N, workspace=ws)
        torch.cuda.synchronize()
        Yref, B = oracle.gemm(c.X, c.W, qg.F16)
        assert_gemm_close(from_device(y), Yref, B, qg.F16, what=f"split workspace M={M} N={N} K={K}")
        assert bool((ws[need:] == 0xA5).all()), "the library wrote past the workspace size it reported"
        with pytest.raises(qg.QGemmError) as e:
            qg.gemm_rung("q4k", SK, x, wp, N, workspace=ws[:need - 16])
        assert e.value.status == -6


def test_split_rung_concurrent_streams():
    """Two streams (default priority) running split-rung GEMMs at once, each
    several times back to back, each with its own workspace: every result
    equals the same problem run alone."""
    import torch

    cases = [Case("q6k", 64, 256, 12288, qg.F16, seed=760), Case("q4k", 40, 320, 8192, qg.F16, seed=761)]
    alone = [from_device(c.run(SK)) for c in cases]
    torch.cuda.synchronize()
    xs = [to_device(c.X, c.dtype) for c in cases]
    wps = [c.device_weights() for c in cases]
    wss = [_ws(qg.workspace_bytes(c.fmt, SK, c.M, c.N, c.K)) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * 4 for _ in cases]
    torch.cuda.synchronize()
    for rep in range(4):
        for i, c in enumerate(cases):
            with torch.cuda.stream(streams[i]):
                outs[i][rep] = qg.gemm_rung(c.fmt, SK, xs[i], wps[i], c.N, stream=streams[i].cuda_stream,
                                            workspace=wss[i])
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for rep in range(4):
            assert np.array_equal(from_device(outs[i][rep]), alone[i]), (i, rep)


def test_split_rung_graph_capture_then_larger_eager_call():
    """A split-rung call captured into a HIP graph with its own workspace;
    then, between replays, eager split calls of a larger size with another
    workspace on the same stream (a library-held workspace would have been
    regrown and freed under the graph here).  Every replay equals the eager
    result, and so does every eager call."""
    import torch

    c = Case("q6k", 64, 256, 12288, qg.F16, seed=780)
    big = Case("q6k", 128, 512, 12288, qg.F16, seed=781)
    x, wp = to_device(c.X, c.dtype), c.device_weights()
    xb, wpb = to_device(big.X, big.dtype), big.device_weights()
    ref = from_device(c.run(SK))
    ref_big = from_device(big.run(SK))
    ws = _ws(qg.workspace_bytes("q6k", SK, 64, 256, 12288))
    ws_big = _ws(qg.workspace_bytes("q6k", SK, 128, 512, 12288))
    assert ws_big.numel() > ws.numel()
    s = torch.cuda.Stream()
    y = torch.empty((64, 256), dtype=torch.float16, device="cuda")
    yb = torch.empty((128, 512), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    print("split graph capture: capture", flush=True)
    with torch.cuda.graph(g, stream=s):
        qg.gemm_rung("q6k", SK, x, wp, 256, out=y, stream=s.cuda_stream, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            qg.gemm_rung("q6k", SK, xb, wpb, 512, out=yb, stream=s.cuda_stream, workspace=ws_big)
        print(f"split graph capture: replay {rep} after a larger eager call", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_device(y), ref), rep
        assert np.array_equal(from_device(yb), ref_big), rep
