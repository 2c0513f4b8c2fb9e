"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Dequant is compared bit for bit (signed zeros equal); GEMM outputs must meet
max |Y - Yref| / (|X|.|W|) <= 2e-3 element by element.  Sizes are small
enough for the oracle to finish in seconds yet span several tiles, several
panels and ragged M/N tails, and every rung is forced on every shape.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests.helpers import (Case, assert_gemm_close, bytes_to_device, fnv1a64, from_device, same_bits, to_device,
                           torch_dtype)

pytestmark = pytest.mark.gpu

FMTS = [("q4k", False), ("q6k", False), ("w4a16", False), ("w4a16", True)]
FMT_IDS = ["q4k", "q6k", "w4a16-asym", "w4a16-sym"]
DTYPES = [qg.F16, qg.BF16]
RUNGS = list(range(qg.num_rungs()))


def _case(fmt, sym, M, N, K, dtype, seed, group=128):
    return Case(fmt, M, N, K, dtype, seed, group=group, symmetric=sym)


# ----------------------------------------------------------------------------
# dequant: bit-exact
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_dequant_bitexact(fmt, sym, dtype):
    N, K = 72, 1024  # five panels, the last one ragged
    c = _case(fmt, sym, 1, N, K, dtype, seed=100)
    print(f"dequant {fmt} sym={sym} dtype={dtype} N={N} K={K}", flush=True)
    w = qg.dequant(fmt, c.device_weights(), N, K, dtype, group=c.group, has_zp=c.has_zp)
    got = from_device(w)
    assert same_bits(got, c.W)
    assert fnv1a64(got[:64]) == fnv1a64(c.W[:64])


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_dequant_w4a16_small_groups(group, dtype):
    c = _case("w4a16", False, 1, 48, 512, dtype, seed=101, group=group)
    w = qg.dequant("w4a16", c.device_weights(), 48, 512, dtype, group=group, has_zp=True)
    assert same_bits(from_device(w), c.W)


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_dequant_q4k_wide_exponent_gap(dtype):
    """d and dmin far apart: the exact weight needs more than 24 bits, so the
    binary32 formation step decides some roundings."""
    rng = np.random.default_rng(7)
    N, K = 64, 512
    f = synth.q4k_fields(rng, N, K)
    f["d"][:] = synth.f16_bits(rng.uniform(0.5, 8.0, f["d"].shape))
    f["dmin"][:] = synth.f16_bits(rng.uniform(2.0 ** -20, 2.0 ** -12, f["dmin"].shape))
    f["d"][0, 0], f["dmin"][0, 0] = 0x3C01, 0x0001  # a double-rounding-sensitive block
    f["sc"][0, 0, :], f["m"][0, 0, :] = 1, 1
    f["q"][0, :32] = 3
    c = Case("q4k", 1, N, K, dtype, seed=102, fields=f)
    w = from_device(qg.dequant("q4k", c.device_weights(), N, K, dtype))
    assert same_bits(w, c.W)


# ----------------------------------------------------------------------------
# identity extraction: X = I makes Y equal W bit for bit through the real GEMM
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("rung", RUNGS)
def test_identity_extraction(fmt, sym, dtype, rung):
    K, N = 256, 48
    eye = synth.f16_bits(np.eye(K)) if dtype == qg.F16 else synth.bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    c = Case(fmt, K, N, K, dtype, seed=103, symmetric=sym, X=eye)
    print(f"identity {fmt} sym={sym} dtype={dtype} rung={rung}", flush=True)
    y = from_device(c.run(rung))
    assert same_bits(y, c.W)


# ----------------------------------------------------------------------------
# GEMM parity on a grid of shapes, every rung
# ----------------------------------------------------------------------------

SHAPES = [(1, 16, 256), (5, 40, 512), (16, 96, 256), (17, 144, 512), (33, 64, 256), (64, 80, 768),
          (65, 128, 256), (130, 160, 512), (257, 48, 256), (300, 272, 512)]


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("rung", RUNGS)
def test_gemm_parity_grid(fmt, sym, dtype, rung):
    for i, (M, N, K) in enumerate(SHAPES):
        c = _case(fmt, sym, M, N, K, dtype, seed=200 + i)
        print(f"grid {fmt} sym={sym} dtype={dtype} rung={rung} M={M} N={N} K={K}", flush=True)
        y = from_device(c.run(rung))
        Yref, B = oracle.gemm(c.X, c.W, dtype)
        assert_gemm_close(y, Yref, B, dtype, what=f"{fmt} M={M} N={N} K={K} rung={rung}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_w4a16_small_groups_gemm(dtype):
    for group in (32, 64):
        c = _case("w4a16", False, 70, 96, 512, dtype, seed=210, group=group)
        for rung in RUNGS:
            y = from_device(c.run(rung))
            Yref, B = oracle.gemm(c.X, c.W, dtype)
            assert_gemm_close(y, Yref, B, dtype, what=f"w4a16 g={group} rung={rung}")


# ----------------------------------------------------------------------------
# fragment-major activations
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_x_to_xf_bitexact(dtype):
    """The device copy equals the oracle's fragment-major copy bit for bit,
    padding rows included, and writes nothing past its size."""
    import torch

    for i, (M, K) in enumerate([(1, 128), (31, 256), (33, 384), (70, 4096), (658, 512), (96, 12288)]):
        print(f"x_to_xf dtype={dtype} M={M} K={K}", flush=True)
        X = synth.activations(np.random.default_rng(500 + i), M, K, dtype)
        n = qg.xf_bytes(M, K) // 2
        out = torch.full((n + 64,), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        guard = from_device(out)[n:].copy()
        qg.x_to_xf(to_device(X, dtype), out=out)
        got = from_device(out)
        assert np.array_equal(got[:n], oracle.fragment_major(X)), f"M={M} K={K}"
        assert np.array_equal(got[n:], guard)


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("rung", RUNGS)
def test_gemm_xf_parity(fmt, sym, dtype, rung):
    """Every rung on fragment-major activations: within the bound of the
    oracle, and bit-identical to the same rung on row-major activations."""
    for i, (M, N, K) in enumerate(SHAPES):
        c = _case(fmt, sym, M, N, K, dtype, seed=200 + i)
        print(f"xf grid {fmt} sym={sym} dtype={dtype} rung={rung} M={M} N={N} K={K}", flush=True)
        y = from_device(c.run_xf(rung))
        Yref, B = oracle.gemm(c.X, c.W, dtype)
        assert_gemm_close(y, Yref, B, dtype, what=f"xf {fmt} M={M} N={N} K={K} rung={rung}")
        assert np.array_equal(y, from_device(c.run(rung))), f"xf != row-major: M={M} N={N} K={K} rung={rung}"


@pytest.mark.parametrize("rung", RUNGS)
def test_gemm_xf_odd_chunks_and_ragged(rung):
    """Fragment-major activations with an odd chunk count (the K-split rungs
    run unsplit) and with ragged M and N."""
    for i, (M, N, K) in enumerate([(70, 96, 384), (37, 37, 256), (130, 144, 640), (3, 5, 512)]):
        fmt = "w4a16" if K % 256 else "q6k"
        c = _case(fmt, False, M, N, K, qg.BF16, seed=230 + i)
        print(f"xf odd/ragged {fmt} rung={rung} M={M} N={N} K={K}", flush=True)
        y = from_device(c.run_xf(rung))
        Yref, B = oracle.gemm(c.X, c.W, qg.BF16)
        assert_gemm_close(y, Yref, B, qg.BF16, what=f"xf {fmt} M={M} N={N} K={K} rung={rung}")
        assert np.array_equal(y, from_device(c.run(rung)))


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("rung", RUNGS)
def test_odd_chunk_count(dtype, rung):
    """W4A16 with K an odd multiple of 128: the K-split rungs fall back to one
    K group, every other rung walks an odd number of 128-wide chunks."""
    for i, (M, N, K) in enumerate([(70, 96, 384), (130, 144, 640), (200, 48, 128)]):
        c = _case("w4a16", i == 1, M, N, K, dtype, seed=215 + i)
        print(f"odd-chunk dtype={dtype} rung={rung} M={M} N={N} K={K}", flush=True)
        y = from_device(c.run(rung))
        Yref, B = oracle.gemm(c.X, c.W, dtype)
        assert_gemm_close(y, Yref, B, dtype, what=f"w4a16 M={M} N={N} K={K} rung={rung}")


@pytest.mark.parametrize("rung", RUNGS)
def test_config0_parity(rung):
    """Single Q4_K GEMM, X fp16 [16, 1024], W [1024, 512], seed 1000."""
    c = Case("q4k", 16, 512, 1024, qg.F16, seed=1000)
    y = from_device(c.run(rung))
    Yref, B = oracle.gemm(c.X, c.W, qg.F16)
    assert_gemm_close(y, Yref, B, qg.F16, what="config0")


# ----------------------------------------------------------------------------
# special cases and invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rung", RUNGS)
def test_special_values(rung):
    M, N, K = 40, 64, 512
    rng = np.random.default_rng(9)
    f = synth.q4k_fields(rng, N, K)
    f["q"][:] = 0
    f["m"][:] = 0
    c = Case("q4k", M, N, K, qg.F16, seed=300, fields=f)
    y = from_device(c.run(rung))
    assert not np.any(y & 0x7FFF)  # all weights zero -> Y == 0
    # X = ones: every row is the column sum of W (all-positive special case)
    ones = synth.f16_bits(np.ones((M, K)))
    c2 = Case("q4k", M, N, K, qg.F16, seed=301, X=ones)
    y2 = from_device(c2.run(rung))
    Yref, B = oracle.gemm(c2.X, c2.W, qg.F16)
    assert_gemm_close(y2, Yref, B, qg.F16, allow_out_ulp=True, what="ones")
    assert np.all(y2 == y2[0:1])
    # W4A16 with zero-point equal to the code everywhere -> Y == 0
    fw = synth.w4a16_fields(rng, N, K, 128, False)
    fw["codes"][:] = np.repeat(fw["zeros"].T, 128, axis=1)
    c3 = Case("w4a16", M, N, K, qg.BF16, seed=302, fields=fw)
    assert not np.any(from_device(c3.run(rung)) & 0x7FFF)


@pytest.mark.parametrize("rung", RUNGS)
def test_guard_bands_and_ragged_n(rung):
    """Outputs outside Y[M][N] are never written, also for N % 4 != 0."""
    import torch

    for M, N, K in [(37, 37, 256), (70, 130, 256), (3, 5, 512)]:
        c = _case("q6k", False, M, N, K, qg.F16, seed=310)
        pad = 4096
        buf = torch.full((M * N + 2 * pad,), 12345.0, dtype=torch.float16, device="cuda")
        # 16-byte aligned interior view starting at element `pad`
        out = buf[pad:pad + M * N].view(M, N)
        c.run(rung, out=out)
        host = buf.cpu()
        assert torch.all(host[:pad] == 12345.0) and torch.all(host[pad + M * N:] == 12345.0)
        Yref, B = oracle.gemm(c.X, c.W, qg.F16)
        assert_gemm_close(from_device(out), Yref, B, qg.F16, what=f"ragged M={M} N={N}")


def test_m_zero_is_noop():
    import torch

    c = _case("q4k", False, 1, 32, 256, qg.F16, seed=320)
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    y = torch.full((0, 32), 1.0, dtype=torch.float16, device="cuda")
    qg.q4k(x, c.device_weights(), 32, out=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("rung", RUNGS)
def test_determinism_and_row_permutation(rung):
    """Run-to-run bit-identical; permuting rows of X permutes rows of Y bit for
    bit (the accumulation order of an output never depends on its row)."""
    M, N, K = 96, 80, 512
    c = _case("q4k", False, M, N, K, qg.BF16, seed=330)
    y1 = from_device(c.run(rung))
    y2 = from_device(c.run(rung))
    assert np.array_equal(y1, y2)
    perm = np.random.default_rng(3).permutation(M)
    yp = from_device(c.run(rung, x_bits=c.X[perm]))
    assert np.array_equal(yp, y1[perm])


def test_rungs_agree_with_each_other():
    """Rows at M = 658 equal, within the bound, the same rows computed as an
    M = 16 problem (a different rung and K split)."""
    M, N, K = 658, 96, 1024
    c = _case("q4k", False, M, N, K, qg.F16, seed=340)
    y = oracle.bits_to_double_fast(from_device(c.run(-1)), qg.F16)
    rows = np.arange(100, 116)
    ys = oracle.bits_to_double_fast(from_device(c.run(-1, x_bits=c.X[rows])), qg.F16)
    _, B = oracle.gemm(c.X[rows], c.W, qg.F16)
    assert np.all(np.abs(y[rows] - ys) <= 2 * 2e-3 * B)



# ----------------------------------------------------------------------------
# staged arm: unpack to scratch, then the same streaming GEMM on the scratch
# ----------------------------------------------------------------------------

def _scratch_to_w(scratch_bits: np.ndarray, N: int, K: int) -> np.ndarray:
    """Logical W[K][N] from the staged scratch, read the way include/qgemm.h
    describes it: per (panel, chunk) [word i][run 16g+col][8 halves], halves
    k = 128c + 32g + 8i + 0..7 in order."""
    npan, nch = -(-N // 16), K // 128
    s = scratch_bits[:npan * 16 * K].reshape(npan, nch, 4, 4, 16, 8)  # p, c, i, g, col, h
    w = s.transpose(1, 3, 2, 5, 0, 4).reshape(K, npan * 16)           # (c, g, i, h) x (p, col)
    return w[:, :N]


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_staged_arm(fmt, sym, dtype):
    """The scratch holds the oracle's unpacked weights bit for bit, and the
    staged Y equals the fused 128x128 rung's Y bit for bit (same MFMA inputs
    in the same order), on shapes with ragged M and N."""
    rung = [r for r in RUNGS if qg.rung_name(r) == "mfma32-128x128"][0]
    for M, N, K in [(130, 160, 512), (37, 40, 256), (257, 272, 768)]:
        c = _case(fmt, sym, M, N, K, dtype, seed=360)
        print(f"staged {fmt} sym={sym} dtype={dtype} M={M} N={N} K={K}", flush=True)
        x = to_device(c.X, dtype)
        y, scratch = qg.staged(fmt, x, c.device_weights(), N, group=c.group if fmt == "w4a16" else 0,
                               has_zp=c.has_zp)
        assert scratch.numel() == qg.staged_scratch_bytes(N, K)
        sb = scratch.cpu().numpy().view(np.uint16)
        assert same_bits(_scratch_to_w(sb, N, K), c.W)
        y_fused = from_device(c.run(rung))
        assert np.array_equal(from_device(y), y_fused)


def test_staged_arm_m_zero_fills_scratch():
    import torch

    c = _case("q6k", False, 1, 48, 512, qg.F16, seed=361)
    x = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    y = torch.empty((0, 48), dtype=torch.float16, device="cuda")
    _, scratch = qg.staged("q6k", x, c.device_weights(), 48, out=y)
    assert same_bits(_scratch_to_w(scratch.cpu().numpy().view(np.uint16), 48, 512), c.W)


# ----------------------------------------------------------------------------
# grouped per-expert GEMM
# ----------------------------------------------------------------------------

def _grouped_case(fmt, sym, counts, N, K, dtype, seed, group=128):
    """Per-expert inputs: X rows grouped by expert, each expert's own weights."""
    import torch

    cases = [Case(fmt, max(m, 1), N, K, dtype, seed + e, group=group, symmetric=sym) for e, m in enumerate(counts)]
    X = np.concatenate([c.X[:m] for c, m in zip(cases, counts)], axis=0)
    W_all = np.concatenate([c.packed for c in cases])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return cases, X, torch.from_numpy(W_all).cuda(), torch.from_numpy(offs).cuda(), offs


def _grouped_call(layout, fmt, X, W, N, offs_d, E, dtype, out=None, sym=True, group=128):
    """One grouped launch on row-major X (qgemm_grouped) or on its
    fragment-major copy (qgemm_grouped_xf)."""
    x = to_device(X, dtype)
    kw = dict(group=group if fmt == "w4a16" else 0, has_zp=not sym, out=out)
    if layout == "row":
        return qg.grouped(fmt, x, W, N, offs_d, E, **kw)
    T, K = X.shape
    return qg.grouped_xf(fmt, qg.x_to_xf(x), W, T, N, K, offs_d, E, **kw)


def _clamped_ranges(offs, T):
    """The row range each expert gets from arbitrary offsets, by the header's
    rule: every offset clamped into [0, T] and to at least the previous
    expert's end (written out serially)."""
    out, hi = [], 0
    for e in range(len(offs) - 1):
        lo = min(max(int(offs[e]), hi), T)
        hi = min(max(int(offs[e + 1]), lo), T)
        out.append((lo, hi))
    return out


@pytest.mark.parametrize("layout", ["row", "xf"])
@pytest.mark.parametrize("K,kernel", [(2048, "direct"), (256, "shared")], ids=["direct", "shared"])
def test_grouped_malformed_offsets(K, kernel, layout):
    """Offsets that are negative, decreasing or past T: both grouped kernels
    (at these 75 rows per expert, K = 2048 takes the direct kernel with K
    split over its waves, K = 256 the shared-activation kernel's 80-row
    tiles) compute exactly the clamped ranges, and write nothing outside Y,
    on both activation layouts."""
    import torch

    T, N, fmt = 300, 80, "q4k"
    offs = np.array([-5, 90, 40, 250, 700], np.int32)
    assert qg.grouped_plan(T, len(offs) - 1, N, K)["name"] == kernel
    cases = [Case(fmt, T, N, K, qg.F16, seed=450 + e) for e in range(len(offs) - 1)]
    X = cases[0].X
    W = torch.from_numpy(np.concatenate([c.packed for c in cases])).cuda()
    pad = 4096
    buf = torch.full((T * N + 2 * pad,), 7.0, dtype=torch.float16, device="cuda")
    out = buf[pad:pad + T * N].view(T, N)
    print(f"grouped malformed offsets K={K} layout={layout} offs={offs.tolist()}", flush=True)
    _grouped_call(layout, fmt, X, W, N, torch.from_numpy(offs).cuda(), len(cases), qg.F16, out=out)
    host = buf.cpu()
    assert torch.all(host[:pad] == 7.0) and torch.all(host[pad + T * N:] == 7.0)
    Y = from_device(out)
    covered = np.zeros(T, bool)
    for e, (lo, hi) in enumerate(_clamped_ranges(offs, T)):
        if hi <= lo:
            continue
        covered[lo:hi] = True
        Yref, B = oracle.gemm(X[lo:hi], cases[e].W, qg.F16)
        assert_gemm_close(Y[lo:hi], Yref, B, qg.F16, what=f"malformed offsets expert {e} rows {lo}..{hi}")
    assert covered.all()  # [0, T) is covered by the clamped ranges here


def _grouped_check(fmt, sym, dtype, counts, N, K, seed, what, group=128):
    """One grouped case on both activation layouts: each expert's rows against
    the oracle on that expert's weights, nothing written outside Y, and the
    same bits from both layouts."""
    import torch

    cases, X, W, offs_d, offs = _grouped_case(fmt, sym, counts, N, K, dtype, seed=seed, group=group)
    T = int(offs[-1])
    outs = {}
    for layout in ("row", "xf"):
        print(f"{what} {fmt} sym={sym} dtype={dtype} layout={layout} counts={counts} K={K}", flush=True)
        pad = 4096
        tdt = torch.float16 if dtype == qg.F16 else torch.bfloat16
        buf = torch.full((T * N + 2 * pad,), 7.0, dtype=tdt, device="cuda")
        out = buf[pad:pad + T * N].view(T, N)
        _grouped_call(layout, fmt, X, W, N, offs_d, len(counts), dtype, out=out, sym=sym, group=group)
        host = buf.cpu()
        assert torch.all(host[:pad] == 7.0) and torch.all(host[pad + T * N:] == 7.0)
        outs[layout] = Y = from_device(out)
        for e, (c, m) in enumerate(zip(cases, counts)):
            if m == 0:
                continue
            Yref, B = oracle.gemm(c.X[:m], c.W, dtype)
            assert_gemm_close(Y[offs[e]:offs[e + 1]], Yref, B, dtype, what=f"{what} {layout} expert {e} rows {m}")
    assert np.array_equal(outs["row"], outs["xf"])


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_grouped_shared_parity(fmt, sym, dtype):
    """The shared-activation grouped kernel (K of two chunks, where the plan
    never splits K) with both tile heights: 80-row tiles at 69 rows per
    expert on average, 32-row tiles at 27 and 44.  Experts span several tiles
    and start inside a 32-row block; empty and one-row experts; N = 144 leaves
    the second column group with one live panel of eight."""
    N, K = 144, 256
    for counts, rows in (([0, 70, 130, 1, 140], 80), ([0, 1, 17, 40, 100, 3], 32), ([44, 60, 28], 32)):
        plan = qg.grouped_plan(sum(counts), len(counts), N, K)
        assert (plan["name"], plan["rows"]) == ("shared", rows), plan
        _grouped_check(fmt, sym, dtype, counts, N, K, seed=410, what="grouped shared")


@pytest.mark.parametrize("fmt,sym", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_grouped_parity(fmt, sym, dtype):
    """The direct grouped kernel: each expert's rows match the oracle on that
    expert's weights, with empty experts, one-row experts and ragged counts;
    mean rows per expert of 10, 27, 44 and 69 select one and two 16-row
    blocks per wave, and these small grids split K over the waves (two ways
    at K = 512, eight at 2048)."""
    N = 96
    for counts, K in (([0, 1, 17, 40, 100, 3], 512), ([5, 0, 12, 3, 30, 10], 512), ([44, 60, 28], 512),
                      ([0, 70, 130, 1, 140], 2048)):
        plan = qg.grouped_plan(sum(counts), len(counts), N, K)
        assert plan["name"] == "direct" and plan["kw"] > 1, plan
        _grouped_check(fmt, sym, dtype, counts, N, K, seed=400, what="grouped direct")


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("sym", [False, True], ids=["asym", "sym"])
def test_grouped_w4a16_group_sizes(group, sym):
    """W4A16 experts quantized in groups of 32 and 64 (each expert's packed
    size, and so its offset in the weights, depends on the group size): the
    shared-activation kernel (K = 256) and the direct kernel (K = 2048, K
    split over its waves), both layouts, against the oracle."""
    N = 144
    counts = [0, 70, 130, 1, 140]
    for K, kernel in ((256, "shared"), (2048, "direct")):
        assert qg.grouped_plan(sum(counts), len(counts), N, K)["name"] == kernel
        _grouped_check("w4a16", sym, qg.F16, counts, N, K, seed=470 + group, what=f"grouped w4a16 g{group} {kernel}",
                       group=group)
