"""Full-size parity for every named workload, in the launch configurations the
benchmark times (the automatic rung, on row-major and on fragment-major
activations).  The oracle dequantizes all of W and
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


@pytest.mark.parametrize("layout", ["row", "xf"])
@pytest.mark.parametrize("name,j", CASES, ids=[f"{n}-{synth.WORKLOADS[n]['gemms'][j][0]}" for n, j in CASES])
def test_workload_sampled(name, j, layout):
    label, fmt, M, K, N, dt, group, sym = synth.WORKLOADS[name]["gemms"][j]
    print(f"fullsize {name}/{label} layout={layout} fmt={fmt} M={M} K={K} N={N} dtype={dt}", flush=True)
    X, fields, enc = synth.workload_inputs(name, j)
    packed = qg.pack(fmt, enc, N, K)
    x = to_device(X, dt)
    wp = bytes_to_device(packed)
    if layout == "xf":
        y = qg.gemm_xf(fmt, qg.x_to_xf(x), wp, M, N, K, group=group if fmt == "w4a16" else 0, has_zp=not sym)
    elif fmt == "q4k":
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


# gate and up merged (Q4_K 2048 -> 2 x 768 per expert, as the benchmark runs
# them), down (Q6_K 768 -> 2048) and gate alone, with the routed counts as
# drawn (41 rows per expert: 32-row tiles of the shared-activation kernel) and
# scaled by 2.4 (99 rows: its 80-row tiles)
MOE = "moe_e128_top8_m658"
MOE_CASES = [("gate_up", 1.0), ("down", 1.0), ("gate", 1.0), ("gate_up", 2.4), ("down", 2.4)]


@pytest.mark.parametrize("layout", ["row", "xf"])
@pytest.mark.parametrize("label,scale", MOE_CASES, ids=[f"{MOE}-{lab}-x{sc}" for lab, sc in MOE_CASES])
def test_moe_grouped_sampled(label, scale, layout):
    """The grouped per-expert GEMM at the MoE workload's full size, on row-major
    routed rows and on their fragment-major copy (as the benchmark launches
    it), on a seeded sample of outputs (first and last rows included): each
    sampled row is checked against its own expert's weights (for gate_up, the
    expert's gate and up columns side by side).  Scaled counts reuse the drawn
    rows in turn."""
    import torch

    w = synth.MOE_WORKLOADS[MOE]
    sg = [g for g in synth.moe_step_gemms(MOE, merge=True) + synth.moe_step_gemms(MOE, merge=False)
          if g["label"] == label][0]
    fmt, K, N = sg["fmt"], sg["K"], sg["N"]
    E = w["experts"]
    counts0 = synth.moe_counts(MOE)
    counts = np.round(counts0 * scale).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offs[-1])
    plan = qg.grouped_plan(T, E, N, K)
    assert (plan["name"], plan["rows"]) == ("shared", 32 if scale == 1.0 else 80), plan
    print(f"moe {MOE}/{label} fmt={fmt} T={T} K={K} N={N} E={E} layout={layout} plan={plan}", flush=True)
    X, enc = synth.moe_step_inputs(MOE, sg["members"])
    X = np.ascontiguousarray(X[np.arange(T) % X.shape[0]])
    packed = np.concatenate([qg.pack(fmt, enc[e * N:(e + 1) * N], N, K) for e in range(E)])
    x, wp, offs_d = to_device(X, qg.F16), bytes_to_device(packed), torch.from_numpy(offs).cuda()
    if layout == "row":
        y = qg.grouped(fmt, x, wp, N, offs_d, E)
    else:
        y = qg.grouped_xf(fmt, qg.x_to_xf(x), wp, T, N, K, offs_d, E)
    Y = from_device(y)
    W = oracle.dequant(fmt, enc, E * N, K, qg.F16)
    rng = np.random.default_rng(4343 + K + N)
    count = 2000
    rows = np.concatenate([rng.integers(0, T, count), [0, T - 1]])
    cols = np.concatenate([rng.integers(0, N, count), [N - 1, 0]])
    expert = np.searchsorted(offs, rows, side="right") - 1
    Yref, B = oracle.gemm_at(X, W, qg.F16, rows, expert * N + cols)
    got = oracle.bits_to_double_fast(Y[rows, cols], qg.F16)
    rel = np.abs(got - Yref) / B
    print(f"  max rel err {rel.max():.3e}", flush=True)
    assert rel.max() <= GEMM_TOL


MERGED = [(name, sg["label"]) for name in synth.WORKLOADS for sg in synth.step_gemms(name) if len(sg["members"]) > 1]


@pytest.mark.parametrize("layout", ["row", "xf"])
@pytest.mark.parametrize("name,label", MERGED, ids=[f"{n}-{lab}" for n, lab in MERGED])
def test_merged_projection_sampled(name, label, layout):
    """Projections that share an input run as one GEMM over their weights
    concatenated along N, as the benchmark launches them: a seeded sample of
    outputs (first and last rows and columns, and every member's first and
    last column) against the oracle on the concatenated weights."""
    sg = [g for g in synth.step_gemms(name) if g["label"] == label][0]
    fmt, M, K, N, dt = sg["fmt"], sg["M"], sg["K"], sg["N"], sg["dt"]
    print(f"merged {name}/{label} layout={layout} fmt={fmt} M={M} K={K} N={N}", flush=True)
    X, enc = synth.step_inputs(name, sg["members"])
    wp = bytes_to_device(qg.pack(fmt, enc, N, K))
    x = to_device(X, dt)
    grp = sg["group"] if fmt == "w4a16" else 0
    if layout == "xf":
        y = qg.gemm_xf(fmt, qg.x_to_xf(x), wp, M, N, K, group=grp, has_zp=not sg["sym"])
    else:
        y = qg.gemm_rung(fmt, -1, x, wp, N, group=grp, has_zp=not sg["sym"])
    Y = from_device(y)
    W = oracle.dequant(fmt, enc, N, K, dt)
    edges = np.cumsum([0] + [synth.WORKLOADS[name]["gemms"][j][4] for j in sg["members"]])
    member_cols = np.concatenate([edges[:-1], edges[1:] - 1])
    rng = np.random.default_rng(4545)
    count = 3000
    rows = np.concatenate([rng.integers(0, M, count), [0, M - 1], np.zeros(member_cols.size, np.int64) + M // 2])
    cols = np.concatenate([rng.integers(0, N, count), [N - 1, 0], member_cols])
    Yref, B = oracle.gemm_at(X, W, dt, rows, cols)
    rel = np.abs(oracle.bits_to_double_fast(Y[rows, cols], dt) - Yref) / B
    print(f"  max rel err {rel.max():.3e}", flush=True)
    assert rel.max() <= GEMM_TOL


def test_offsets_past_4gib_sampled():
    """X of 40000 x 65536 fp16 (5.2 GB): row offsets cross 2^32 bytes in both
    activation layouts.  The rows repeat with period 61, so a wrapped 32-bit
    offset (2^32 bytes = 32768 rows here) would land on a different row.
    Sampled rows against the oracle, for the ladder's rung (direct-skinny-n,
    N = 48) and the 128x128 streaming rung."""
    import torch

    M, K, N, P = 40000, 65536, 48, 61
    rng = np.random.default_rng(4646)
    block = synth.activations(rng, P, K, qg.F16)
    fields = synth.weight_fields("q4k", rng, N, K, 128, False)
    enc = synth.encode("q4k", fields)
    wp = bytes_to_device(qg.pack("q4k", enc, N, K))
    x = to_device(block, qg.F16).repeat(-(-M // P), 1)[:M]
    assert x.is_contiguous() and x.numel() * 2 > 2 ** 32
    xf = qg.x_to_xf(x)
    W = oracle.dequant("q4k", enc, N, K, qg.F16)
    Yref, B = oracle.gemm(block, W, qg.F16)
    rows = np.concatenate([[0, 1, P - 1, P, 32767, 32768, 32769, 65535 // 2, M - 1], rng.integers(0, M, 200)])
    rung128 = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-128x128"][0]
    for layout, rung in [("row", -1), ("row", rung128), ("xf", -1), ("xf", rung128)]:
        print(f"offsets>4GiB layout={layout} rung={rung} M={M} K={K} N={N}", flush=True)
        if layout == "row":
            y = qg.gemm_rung("q4k", rung, x, wp, N)
        else:
            y = qg.gemm_xf("q4k", xf, wp, M, N, K, rung=rung)
        Y = from_device(y[torch.from_numpy(rows).cuda()])
        rel = np.abs(oracle.bits_to_double_fast(Y, qg.F16) - Yref[rows % P]) / B[rows % P]
        print(f"  max rel err {rel.max():.3e}", flush=True)
        assert rel.max() <= GEMM_TOL
        del y
