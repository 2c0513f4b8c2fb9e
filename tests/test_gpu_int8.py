"""Parity of the int8-activation path with the oracle (qref.c, item 5).

Every step of this path is defined to the bit (binary32 weights, per-column
and per-row int8 scales, RNE codes, exact integer sums, a binary32
epilogue), so every comparison here is exact: the row quantizer's codes in
their fragment-major layout and its scales, the per-column factors, and Y
for every rung, format and dtype, on ragged shapes and at the full sizes the
benchmark times (sampled outputs)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests.helpers import Case, bytes_to_device, from_device, same_bits, to_device

pytestmark = pytest.mark.gpu


def _f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def _i8(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int8)


def _weights_f32(c: Case) -> np.ndarray:
    return oracle.dequant_f32(c.fmt, c.enc, c.N, c.K)


def _group(c: Case) -> int:
    return c.group if c.fmt == "w4a16" else 0


@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16])
@pytest.mark.parametrize("M,K", [(1, 256), (37, 384), (70, 4096), (33, 20480)])
def test_i8_quantize_bitexact(dtype, M, K):
    """Codes in the fragment-major int8 layout (zero rows past M) and scales,
    bit for bit; K = 20480 rereads part of each row (more than fits in
    registers), and one row is all zeros."""
    print(f"i8 quantize M={M} K={K} dtype={dtype}", flush=True)
    rng = np.random.default_rng(M * 7 + K + dtype)
    X = synth.activations(rng, M, K, dtype)
    if M > 3:
        X[2] = 0
    xq, sx = qg.i8_quantize(to_device(X, dtype))
    Q, s = oracle.quant_rows_i8(X, dtype)
    assert np.array_equal(_i8(xq), oracle.fragment_major_i8(Q))
    assert np.array_equal(_f32(sx).view(np.uint32), s.view(np.uint32))


CS_CASES = [("q4k", 40, 512, 128, False), ("q6k", 33, 768, 128, False), ("w4a16", 48, 384, 128, False),
            ("w4a16", 17, 256, 64, True)]


@pytest.mark.parametrize("fmt,N,K,group,sym", CS_CASES)
def test_i8_colscale_bitexact(fmt, N, K, group, sym):
    print(f"i8 colscale {fmt} N={N} K={K} group={group} sym={sym}", flush=True)
    c = Case(fmt, 1, N, K, qg.F16, seed=77 + N, group=group, symmetric=sym)
    rw, sw = qg.i8_colscale(fmt, c.device_weights(), N, K, group=_group(c), has_zp=c.has_zp)
    r, s = oracle.colscale_i8(_weights_f32(c))
    assert np.array_equal(_f32(rw).view(np.uint32), r.view(np.uint32))
    assert np.array_equal(_f32(sw).view(np.uint32), s.view(np.uint32))


def _oracle_y(c: Case, rows=None, cols=None):
    W32 = _weights_f32(c)
    r, s = oracle.colscale_i8(W32)
    Qx, sx = oracle.quant_rows_i8(c.X, c.dtype)
    if rows is not None:
        Qx, sx = Qx[rows], sx[rows]
    if cols is not None:
        W32, r, s = W32[:, cols], r[cols], s[cols]
    return oracle.gemm_i8(Qx, sx, oracle.requant_i8(W32, r), s, c.dtype)


def _run_i8(c: Case, rung: int = -1):
    wp = c.device_weights()
    rw, sw = qg.i8_colscale(c.fmt, wp, c.N, c.K, group=_group(c), has_zp=c.has_zp)
    xq, sx = qg.i8_quantize(to_device(c.X, c.dtype))
    y = qg.gemm_i8(c.fmt, xq, sx, wp, rw, sw, c.M, c.N, c.K, c.dtype, group=_group(c), has_zp=c.has_zp, rung=rung)
    return from_device(y)


GEMM_SHAPES = [(1, 48, 512), (37, 200, 768), (130, 72, 256), (300, 264, 1024)]


@pytest.mark.parametrize("rung", list(range(qg.i8_num_rungs())))
@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16"])
@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16])
def test_i8_gemm_bitexact(rung, fmt, dtype):
    """Every rung gives the oracle's bits on shapes with ragged M and N tails,
    several tiles, and an odd chunk count (K = 768: the K-split rung runs
    unsplit)."""
    if rung >= qg.i8_num_rungs():
        pytest.skip(f"the int8 ladder has {qg.i8_num_rungs()} rungs")
    for i, (M, N, K) in enumerate(GEMM_SHAPES):
        print(f"i8 gemm rung={rung} {fmt} dtype={dtype} M={M} N={N} K={K}", flush=True)
        c = Case(fmt, M, N, K, dtype, seed=900 + 10 * i + rung, group=128)
        Y = _run_i8(c, rung)
        want = _oracle_y(c)
        assert same_bits(Y, want), f"{fmt} rung {rung} M={M} N={N} K={K}: {(Y != want).sum()} outputs differ"


I8_SK = [r for r in range(qg.i8_num_rungs()) if qg.i8_rung_name(r) == "i8-64x64-sk"][0]


@pytest.mark.parametrize("fmt,M,N,K,dtype,ways", [
    ("q4k", 37, 200, 4096, qg.F16, 16),      # four slices of four K groups; ragged M and N
    ("w4a16", 64, 256, 4096, qg.BF16, 16),
    ("q6k", 96, 130, 12288, qg.F16, 32),     # eight slices, two row tiles
    ("q4k", 5, 64, 16384, qg.BF16, 32),
])
def test_i8_split_rung_bitexact(fmt, M, N, K, dtype, ways):
    """K split across workgroups on the int8 path: the int32 partial sums of
    the slices add up exactly, so Y has the oracle's bits, and the same bits
    as the unsplit 128x128 rung."""
    info = qg.i8_rung_info(I8_SK, fmt, M, N, K)
    assert info["k_split"] == ways, info
    c = Case(fmt, M, N, K, dtype, seed=950 + M, group=128)
    print(f"i8 split {fmt} M={M} N={N} K={K} dtype={dtype} info={info}", flush=True)
    Y = _run_i8(c, I8_SK)
    want = _oracle_y(c)
    assert same_bits(Y, want), f"{(Y != want).sum()} outputs differ"
    assert same_bits(_run_i8(c, 0), Y)


@pytest.mark.parametrize("M", [40, 200])
def test_i8_split_rung_auto_down_projection(M):
    """Q6_K 12288 -> 4096 at 40 and 200 rows: the int8 ladder picks the split
    rung, and its Y has the oracle's bits."""
    N, K = 4096, 12288
    sel = qg.i8_select_rung("q6k", M, N, K)
    assert sel["name"] == "i8-64x64-sk", sel
    c = Case("q6k", M, N, K, qg.F16, seed=970 + M)
    print(f"i8 split auto q6k M={M} N={N} K={K} info={sel}", flush=True)
    Y = _run_i8(c, -1)
    want = _oracle_y(c)
    assert same_bits(Y, want), f"{(Y != want).sum()} outputs differ"


def test_i8_gemm_zero_rows_and_columns():
    """A zero activation row and an all-zero weight column give zero scales,
    zero codes and zero outputs."""
    c = Case("q4k", 40, 48, 512, qg.F16, seed=5)
    c.X[7] = 0
    c.fields["d"][3] = 0
    c.fields["dmin"][3] = 0
    c.enc = synth.encode("q4k", c.fields)
    c.packed = qg.pack("q4k", c.enc, c.N, c.K)
    Y = _run_i8(c)
    assert same_bits(Y, _oracle_y(c))
    assert not (Y[7] & 0x7FFF).any() and not (Y[:, 3] & 0x7FFF).any()


@pytest.mark.parametrize("label", ["gate_up", "down"])
def test_i8_fullsize_sampled(label):
    """The layer's dominant projections at M = 658 (the merged gate and up,
    Q4_K 4096 -> 24576; down, Q6_K 12288 -> 4096) through the automatic
    rung: a seeded sample of rows (with the first and last) against the
    oracle on a seeded sample of columns (with the first and last)."""
    name = "qwen3_8b_layer_m658"
    g = next(g for g in synth.step_gemms(name) if g["label"] == label)
    fmt, M, K, N, dt = g["fmt"], g["M"], g["K"], g["N"], g["dt"]
    print(f"i8 fullsize {label} {fmt} M={M} K={K} N={N}", flush=True)
    X, enc = synth.step_inputs(name, g["members"])
    wp = bytes_to_device(qg.pack(fmt, enc, N, K))
    rw, sw = qg.i8_colscale(fmt, wp, N, K)
    xq, sx = qg.i8_quantize(to_device(X, dt))
    Y = from_device(qg.gemm_i8(fmt, xq, sx, wp, rw, sw, M, N, K, dt))
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([rng.integers(0, M, 48), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, N, 96), [0, N - 1]]))
    W32 = oracle.dequant_f32(fmt, enc, N, K)
    r, s = oracle.colscale_i8(W32)
    assert np.array_equal(_f32(rw).view(np.uint32), r.view(np.uint32))
    Qx, sxo = oracle.quant_rows_i8(X, dt)
    assert np.array_equal(_f32(sx).view(np.uint32), sxo.view(np.uint32))
    want = oracle.gemm_i8(Qx[rows], sxo[rows], oracle.requant_i8(W32[:, cols], r[cols]), s[cols], dt)
    assert same_bits(Y[np.ix_(rows, cols)], want)


def test_i8_k_at_the_int32_limit():
    """K = 131072 (the largest K the path accepts) with every code at +-127:
    each int32 sum reaches 131072 * 127 * 127 = 2114060288, just below 2^31,
    and must still be exact."""
    M, N, K = 3, 32, 131072
    print(f"i8 K limit M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(8)
    X = np.where(rng.random((M, K)) < 0.5, 1.0, -1.0)
    X[1] = 1.0  # an all-positive row: its sums against a positive column are the maximum
    Xb = synth.f16_bits(X)
    f = synth.q6k_fields(rng, N, K)
    # every weight d * s * (q - 32) with s = 1, q = 63 or 1 and one d per column: +-31 d, so every
    # code is +-127
    f["s"][:] = 1
    f["d"][:] = f["d"][:, :1]
    f["q"][:] = np.where(rng.random(f["q"].shape) < 0.5, 63, 1).astype(f["q"].dtype)
    f["q"][0] = 63  # column 0 all positive
    c = Case("q6k", M, N, K, qg.F16, seed=1, fields=f, X=Xb)
    Y = _run_i8(c)
    want = _oracle_y(c)
    assert same_bits(Y, want)
    W32 = _weights_f32(c)
    r, _ = oracle.colscale_i8(W32)
    Qx, _ = oracle.quant_rows_i8(Xb, qg.F16)
    acc = Qx.astype(np.int64) @ oracle.requant_i8(W32, r).astype(np.int64)
    assert acc.max() == 131072 * 127 * 127 < 2 ** 31


def test_i8_bf16_rows_at_the_scale_floor():
    """bf16 rows whose largest magnitude is just below 2^-96 quantize to zero
    codes and a zero scale; a row at 2^-96 keeps full codes."""
    M, N, K = 4, 48, 256
    rng = np.random.default_rng(9)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[1] *= np.float32(2.0 ** -100)
    X[2] = X[2] / np.abs(X[2]).max() * np.float32(2.0 ** -96)
    Xb = synth.bf16_bits_from_f32(X)
    c = Case("q4k", M, N, K, qg.BF16, seed=3, X=Xb)
    wp = c.device_weights()
    xq, sx = qg.i8_quantize(to_device(Xb, qg.BF16))
    Q, s = oracle.quant_rows_i8(Xb, qg.BF16)
    assert np.array_equal(_f32(sx).view(np.uint32), s.view(np.uint32)) and s[1] == 0 and s[2] > 0
    assert np.array_equal(_i8(xq), oracle.fragment_major_i8(Q))
    rw, sw = qg.i8_colscale("q4k", wp, N, K)
    Y = from_device(qg.gemm_i8("q4k", xq, sx, wp, rw, sw, M, N, K, qg.BF16))
    assert same_bits(Y, _oracle_y(c)) and not (Y[1] & 0x7FFF).any()
