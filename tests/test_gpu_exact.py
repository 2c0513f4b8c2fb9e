"""GPU parity of the unpack's exact-rounding sub-path, through every kernel.

A Q4_K weight is d*sc*q - dmin*m rounded once into fp16/bf16.  When the
exponents of d and dmin are more than three binades apart, that exact value
can need more than binary32's 24 bits, and forming it in binary32 first and
rounding again can land on the other side of a midpoint.  The kernels flag
such runs and recompute them with a two-sum and rounding to odd.  The fields
here put d and dmin 4 to 18 binades apart (with a few blocks at exactly 3
and 4), plus the two constructed blocks whose weights sit on an fp16 or bf16
midpoint after a binary32 step.  Every test first checks, on the CPU, that
the double-rounded values differ from the oracle's on some weights, so the
test fails if a kernel skips the exact path.  Each path is then checked by
identity extraction (X = I, so Y = W bit for bit) and by a GEMM on random X
against the fp64 oracle within 2e-3 of |X|.|W|.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests.helpers import Case, assert_gemm_close, bytes_to_device, from_device, same_bits, to_device

pytestmark = pytest.mark.gpu

DTYPES = [qg.F16, qg.BF16]
RUNGS = list(range(qg.num_rungs()))


def wide_gap_fields(seed: int, N: int, K: int) -> dict:
    """Q4_K fields with d in [2^-4, 2^-2) and dmin 4..18 binades below d (a
    few blocks 3 binades below), the two midpoint blocks placed in columns
    0 and 1 of the first super-block (all 32 weights of sub-block 0)."""
    rng = np.random.default_rng(seed)
    f = synth.q4k_fields(rng, N, K)
    nb = K // 256
    d = rng.uniform(2.0 ** -4, 2.0 ** -2, (N, nb))
    gap = rng.integers(4, 19, (N, nb)).astype(np.float64)
    gap[::7, 0] = 3                       # the fast path's edge: still exact in binary32
    gap[1::7, 0] = 4                      # the first gap the exact path takes
    dmin = d * 2.0 ** -gap * rng.uniform(1.0, 2.0, (N, nb))
    f["d"][:] = synth.f16_bits(d)
    f["dmin"][:] = synth.f16_bits(dmin)
    # the constructed midpoint blocks (the oracle's single-rounding pins)
    f["d"][0, 0], f["dmin"][0, 0] = 0x3C01, 0x0001
    f["sc"][0, 0, 0], f["m"][0, 0, 0] = 1, 1
    f["q"][0, :32] = 3                    # 3*(1 + 2^-10) - 2^-24: an fp16 midpoint after binary32
    if N > 1:
        f["d"][1, 0], f["dmin"][1, 0] = 0x400C, 0x0001
        f["sc"][1, 0, 0], f["m"][1, 0, 0] = 1, 1
        f["q"][1, :32] = 1                # 1036*2^-9 - 2^-24: a bf16 midpoint after binary32
    return f


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def double_rounded(f: dict, dtype: int) -> np.ndarray:
    """W[K][N] bits as a binary32 intermediate would give them: the exact
    value (exact in binary64 for these gaps), rounded to binary32, then to
    fp16/bf16 -- the value the kernels must NOT produce where it differs."""
    import torch

    N, K = f["q"].shape
    j = (np.arange(K) % 256) // 32
    b = np.arange(K) // 256
    d, dm = _f16(f["d"])[:, b], _f16(f["dmin"])[:, b]            # [N][K]
    sc = f["sc"][:, b, j].astype(np.float64)
    m = f["m"][:, b, j].astype(np.float64)
    exact = d * sc * f["q"].astype(np.float64) - dm * m
    w32 = exact.astype(np.float32)
    if dtype == qg.F16:
        bits = w32.astype(np.float16).view(np.uint16)
    else:
        bits = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return np.ascontiguousarray(bits.T)


def _eye(K: int, dtype: int) -> np.ndarray:
    return synth.f16_bits(np.eye(K)) if dtype == qg.F16 else synth.bf16_bits_from_f32(np.eye(K, dtype=np.float32))


def _wide_case(M, N, K, dtype, seed, X=None):
    return Case("q4k", M, N, K, dtype, seed, fields=wide_gap_fields(seed, N, K), X=X)


def _assert_sensitive(c: Case):
    """The binary32 route differs from the oracle on some weights of c."""
    two = double_rounded(c.fields, c.dtype)
    diff = int((~np.equal(np.where((two & 0x7FFF) == 0, 0, two), np.where((c.W & 0x7FFF) == 0, 0, c.W))).sum())
    assert diff >= 32, f"only {diff} weights tell the exact path from a binary32 intermediate"
    return diff


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("layout", ["row", "xf"])
def test_exact_path_identity_every_rung(dtype, layout):
    K, N = 512, 48
    c = _wide_case(K, N, K, dtype, seed=900 + dtype, X=_eye(K, dtype))
    nd = _assert_sensitive(c)
    for rung in RUNGS:
        print(f"exact identity dtype={dtype} layout={layout} rung={qg.rung_name(rung)} ({nd} sensitive)", flush=True)
        y = from_device(c.run(rung) if layout == "row" else c.run_xf(rung))
        assert same_bits(y, c.W), f"rung {qg.rung_name(rung)}: {int((y != c.W).sum())} weights differ"


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("layout", ["row", "xf"])
def test_exact_path_gemm_every_rung(dtype, layout):
    for i, (M, N, K) in enumerate([(70, 80, 512), (300, 144, 768)]):
        c = _wide_case(M, N, K, dtype, seed=910 + 2 * i + dtype)
        _assert_sensitive(c)
        Yref, B = oracle.gemm(c.X, c.W, dtype)
        for rung in RUNGS:
            print(f"exact gemm dtype={dtype} layout={layout} M={M} N={N} K={K} rung={qg.rung_name(rung)}", flush=True)
            y = from_device(c.run(rung) if layout == "row" else c.run_xf(rung))
            assert_gemm_close(y, Yref, B, dtype, what=f"wide-gap rung={qg.rung_name(rung)} M={M}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_exact_path_dequant_and_staged(dtype):
    """The logical dequant, the staged arm's scratch and its Y (identity
    extraction, and a random-X GEMM against the oracle)."""
    K, N = 512, 40
    c = _wide_case(K, N, K, dtype, seed=920 + dtype, X=_eye(K, dtype))
    _assert_sensitive(c)
    wp = c.device_weights()
    print(f"exact dequant/staged dtype={dtype}", flush=True)
    assert same_bits(from_device(qg.dequant("q4k", wp, N, K, dtype)), c.W)
    y, _ = qg.staged("q4k", to_device(c.X, dtype), wp, N)
    assert same_bits(from_device(y), c.W)
    r = _wide_case(96, N, K, dtype, seed=921 + dtype)
    Yref, B = oracle.gemm(r.X, r.W, dtype)
    ys, _ = qg.staged("q4k", to_device(r.X, dtype), r.device_weights(), N)
    assert_gemm_close(from_device(ys), Yref, B, dtype, what="staged wide-gap")


@pytest.mark.parametrize("layout", ["row", "xf"])
@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
@pytest.mark.parametrize("K,kernel", [(256, "shared"), (2048, "direct")])
def test_exact_path_grouped(dtype, K, kernel, layout):
    """Two experts, each fed an identity block, so each expert's rows of Y
    are its weights bit for bit (row-major X and its fragment-major copy;
    K = 256 takes the shared-activation kernel, K = 2048 the direct kernel
    with K split over its waves)."""
    import torch

    N, E = 48, 2
    assert qg.grouped_plan(E * K, E, N, K)["name"] == kernel
    cases = [_wide_case(K, N, K, dtype, seed=930 + e + 4 * dtype) for e in range(E)]
    for c in cases:
        _assert_sensitive(c)
    X = np.concatenate([_eye(K, dtype)] * E, axis=0)
    wp = bytes_to_device(np.concatenate([c.packed for c in cases]))
    offs = torch.tensor([0, K, 2 * K], dtype=torch.int32, device="cuda")
    print(f"exact grouped dtype={dtype} K={K} layout={layout}", flush=True)
    x = to_device(X, dtype)
    if layout == "row":
        y = from_device(qg.grouped("q4k", x, wp, N, offs, E))
    else:
        y = from_device(qg.grouped_xf("q4k", qg.x_to_xf(x), wp, E * K, N, K, offs, E))
    for e, c in enumerate(cases):
        assert same_bits(y[e * K:(e + 1) * K], c.W), f"expert {e}"


@pytest.mark.parametrize("dtype", DTYPES, ids=["f16", "bf16"])
def test_exact_path_int8(dtype):
    """The int8 path's weights are the binary32 rounding of the exact value:
    the per-column factors and every rung's Y match the oracle bit for bit on
    the wide-gap fields."""
    M, N, K = 96, 80, 1024
    c = _wide_case(M, N, K, dtype, seed=940 + dtype)
    wp = c.device_weights()
    W32 = oracle.dequant_f32("q4k", c.enc, N, K)
    r, s = oracle.colscale_i8(W32)
    rw, sw = qg.i8_colscale("q4k", wp, N, K)
    assert np.array_equal(rw.cpu().numpy(), r) and np.array_equal(sw.cpu().numpy(), s)
    Qx, sxo = oracle.quant_rows_i8(c.X, dtype)
    want = oracle.gemm_i8(Qx, sxo, oracle.requant_i8(W32, r), s, dtype)
    xq, sx = qg.i8_quantize(to_device(c.X, dtype))
    for rung in range(qg.i8_num_rungs()):
        print(f"exact int8 dtype={dtype} rung={qg.i8_rung_name(rung)}", flush=True)
        y = from_device(qg.gemm_i8("q4k", xq, sx, wp, rw, sw, M, N, K, dtype, rung=rung))
        assert np.array_equal(y, want), qg.i8_rung_name(rung)


@pytest.mark.parametrize("fmt,sym,dtype,wide", [
    ("q4k", False, qg.F16, True), ("q4k", False, qg.BF16, True), ("q4k", False, qg.F16, False),
    ("q6k", False, qg.F16, False), ("w4a16", False, qg.F16, False), ("w4a16", True, qg.BF16, False)])
@pytest.mark.parametrize("layout", ["row", "xf"])
def test_identity_large_m_ladder(fmt, sym, dtype, wide, layout):
    """Identity extraction through the automatic ladder at M = K = 4096 (the
    long-prefill rung): Y = W bit for bit."""
    M = K = 4096
    N = 2048
    sel = (qg.select_rung if layout == "row" else qg.select_rung_xf)(fmt, M, N, K, dtype)
    assert sel["rows"] >= 256, sel  # a long-prefill tile, not a small-M or skinny rung
    if wide:
        c = _wide_case(M, N, K, dtype, seed=950 + dtype, X=_eye(K, dtype))
        _assert_sensitive(c)
    else:
        c = Case(fmt, M, N, K, dtype, seed=951, symmetric=sym, X=_eye(K, dtype))
    print(f"identity large-M {fmt} sym={sym} dtype={dtype} wide={wide} layout={layout} rung={sel['name']}",
          flush=True)
    y = from_device(c.run(-1) if layout == "row" else c.run_xf(-1))
    assert same_bits(y, c.W), f"{int((y != c.W).sum())} weights differ on {sel['name']}"
