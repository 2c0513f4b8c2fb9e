"""Pins for the CPU oracle (runs without a GPU).

Every check compares the oracle with something other than itself: library
roundings (numpy float16/float32, torch bfloat16), exact rationals
(``fractions.Fraction``) rounded by a brute-force nearest-neighbour search,
closed forms the pages print, special cases whose answer is known in closed
form, and numpy's float64 matmul.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from quantized_weight_prefill_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")


def load_golden() -> dict:
    vals = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("="))
            vals[k] = float(int(v, 16)) if v.startswith("0x") else float(v)
    return vals


# ----------------------------------------------------------------------------
# Brute-force nearest-even rounding of an exact rational (independent of the
# oracle's bit manipulation): look at the neighbouring grid points of the
# target type and choose the closest, ties to the even bit pattern.
# ----------------------------------------------------------------------------

def _grid_candidates(x: Fraction, ftype, inf_at: Fraction):
    """Grid points of ftype around x; one past the largest finite value the
    grid continues at ``inf_at`` (2^(emax+1)), which stands for infinity."""
    big = np.finfo(ftype).max
    xf = float(x)
    g = ftype(np.clip(xf, -float(big), float(big)))
    cands = {(Fraction(float(c)), c) for c in (g, np.nextafter(g, ftype(np.inf)), np.nextafter(g, ftype(-np.inf)))
             if np.isfinite(c)}
    if abs(x) >= Fraction(float(big)):
        sgn = 1 if x > 0 else -1
        cands.add((sgn * inf_at, ftype(sgn * np.inf)))
    return cands


def nearest_even(x: Fraction, kind: str) -> np.generic:
    if kind == "f16":
        ftype, ut, inf_at = np.float16, np.uint16, Fraction(2 ** 16)
    elif kind == "f32":
        ftype, ut, inf_at = np.float32, np.uint32, Fraction(2 ** 128)
    else:
        raise ValueError(kind)
    best = None
    for val, c in _grid_candidates(x, ftype, inf_at):
        key = (abs(val - x), int(np.array(c, ftype).view(ut)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def nearest_even_bf16(x: Fraction) -> int:
    """bf16 bits nearest to x, ties to even: candidates on the bf16 grid
    around the float32 nearest value (2^128 stands for infinity)."""
    f = np.float32(float(x)) if abs(x) < Fraction(2 ** 128) else np.float32(np.sign(float(x)) * 3.3e38)
    b = int(np.array(f, np.float32).view(np.uint32))
    lo = b & 0xFFFF0000
    best = None
    for c in (lo, lo + 0x10000, lo - 0x10000):
        if c < 0 or c >= 1 << 32:
            continue
        v = np.array(c, np.uint32).view(np.float32)
        if np.isnan(v):
            continue
        val = Fraction(float(v)) if np.isfinite(v) else (1 if v > 0 else -1) * Fraction(2 ** 128)
        key = (abs(val - x), (c >> 16) & 1)
        if best is None or key < best[0]:
            best = (key, c >> 16)
    return best[1]


def f16_val(h: int) -> Fraction:
    return Fraction(float(np.array(h, np.uint16).view(np.float16)))


# ----------------------------------------------------------------------------
# Roundings and conversions
# ----------------------------------------------------------------------------

def test_f16_decode_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = oracle.bits_to_double(allbits, oracle.F16)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isnan(got[np.isnan(ref)]))


def test_bf16_decode_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32)
    ref = (allbits << 16).view(np.float32).astype(np.float64)
    got = oracle.bits_to_double(allbits.astype(np.uint16), oracle.BF16)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def _rounding_probe_values(rng):
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e-30, -1e-30]
    # random magnitudes across the fp16 normal, subnormal and overflow ranges
    vals += list(rng.standard_normal(2000) * np.exp2(rng.integers(-30, 20, 2000)))
    # exact midpoints between neighbouring fp16 values (ties)
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals += list((a + b) / 2) + list(-(a + b) / 2)
    # midpoints +- one double ulp
    mids = (a + b) / 2
    vals += list(np.nextafter(mids, np.inf)) + list(np.nextafter(mids, -np.inf))
    return vals


def test_rn_f16_matches_numpy():
    rng = np.random.default_rng(11)
    for x in _rounding_probe_values(rng):
        want = int(np.array(np.float16(x)).view(np.uint16))
        assert oracle.rn_f16(x) == want, x


def test_rn_f32_matches_numpy():
    rng = np.random.default_rng(12)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    f = rng.standard_normal(1000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    xs += list((f.astype(np.float64) + nxt.astype(np.float64)) / 2)  # float32 ties
    for x in xs:
        want = float(np.float32(x))
        got = oracle.rn_f32(x)
        assert got == want or (math.isinf(got) and math.isinf(want)), x


def test_rn_bf16_matches_torch():
    rng = np.random.default_rng(13)
    f = (rng.standard_normal(4000) * np.exp2(rng.integers(-130, 120, 4000))).astype(np.float32)
    bits = f.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)  # exact bf16 midpoints
    f = np.concatenate([f, ties[np.isfinite(ties)]])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, w in zip(f, want):
        assert oracle.rn_bf16(float(x)) == int(w), x


# ----------------------------------------------------------------------------
# Closed forms the pages print
# ----------------------------------------------------------------------------

def test_page_closed_forms():
    g = load_golden()
    # Q4_K: fp16 d + fp16 dmin + 12 B of 6-bit scales/mins + 128 B of nibbles
    assert 2 + 2 + 12 + 128 == synth.Q4K_BLOCK_BYTES
    assert synth.Q4K_BLOCK_BYTES / 256 == g["q4k_bytes_per_weight"]
    assert g["q4k_bytes_per_weight"] + 2.0 + 2.0 == g["staged_bytes_per_weight"]
    assert round(g["staged_bytes_per_weight"] / g["q4k_bytes_per_weight"], 1) == g["staged_over_fused"]
    assert round(g["rx9070xt_fp16_TFLOPs"] * 1000 / g["rx9070xt_bw_GBps"]) == g["ridge_flop_per_byte"]
    assert round(2 * g["tile_tokens"] / g["staged_bytes_per_weight"]) == g["staged_intensity"]
    assert round(2 * g["tile_tokens"] / g["q4k_bytes_per_weight"], -1) == g["fused_intensity"]
    assert round(g["staged_intensity"] * g["rx9070xt_bw_GBps"] / 1000) == g["staged_cap_TFLOPs"]
    T, tile = int(g["weight_reads_T"]), int(g["weight_reads_tile"])
    assert T // -(-T // tile) == g["weight_reads_ratio"]
    # Q6_K: 128 B low nibbles + 64 B high pairs + 16 int8 scales + fp16 d
    assert 128 + 64 + 16 + 2 == synth.Q6K_BLOCK_BYTES
    assert synth.Q6K_BLOCK_BYTES / 256 == 0.8203125


def test_magic_fp16_exhaustive():
    """0x6400|n read as fp16 is 1024+n for every n < 1024, and subtracting
    1024+zp from 1024+n gives n-zp exactly for every pair of 4-bit codes."""
    g = load_golden()
    base = int(g["magic_f16_bits"])
    n = np.arange(1024, dtype=np.uint16)
    v = (base | n).astype(np.uint16).view(np.float16)
    assert np.array_equal(v.astype(np.float64), g["magic_f16_base"] + n)
    for nn in range(16):
        for zp in range(16):
            a = np.array(base | nn, np.uint16).view(np.float16)
            b = np.array(base | zp, np.uint16).view(np.float16)
            assert float(a - b) == nn - zp
    # the and-or form on a whole 32-bit lane yields the nibble pair
    mask, orv = int(g["and_or_mask"]), int(g["and_or_or"])
    rng = np.random.default_rng(3)
    for x in rng.integers(0, 2 ** 32, 200, dtype=np.uint64):
        r = (int(x) & mask) | orv
        h = np.array([r & 0xFFFF, r >> 16], np.uint16).view(np.float16)
        assert float(h[0]) == 1024 + (int(x) & 15) and float(h[1]) == 1024 + ((int(x) >> 16) & 15)


def test_derived_magics_exhaustive():
    """bf16 0x4300|n = 128+n (n < 128); fp32 0x4B000000|n = 2^23+n;
    fp16 subnormal pattern n = n * 2^-24 (n < 1024)."""
    n = np.arange(128, dtype=np.uint32)
    bf = ((0x4300 | n) << 16).view(np.float32)
    assert np.array_equal(bf.astype(np.float64), 128 + n)
    n = np.arange(1 << 16, dtype=np.uint32)
    f = (0x4B000000 | n).view(np.float32)
    assert np.array_equal(f.astype(np.float64), 2 ** 23 + n)
    n = np.arange(1024, dtype=np.uint16)
    assert np.array_equal(n.view(np.float16).astype(np.float64), n * 2.0 ** -24)


# ----------------------------------------------------------------------------
# Field decode: the generator's encoder and the oracle's decoder are two
# independent readings of one layout; they must invert each other.
# ----------------------------------------------------------------------------

def test_q4k_field_roundtrip():
    rng = np.random.default_rng(21)
    f = synth.q4k_fields(rng, 8, 1024)
    f["sc"][0, 0] = np.arange(56, 64)  # exercise the top two bits of every slot
    f["m"][0, 0] = np.arange(63, 55, -1)
    enc = synth.q4k_encode(f)
    for n in range(8):
        for b in range(4):
            got = oracle.q4k_fields(enc[n, b])
            assert got["d"] == f["d"][n, b] and got["dmin"] == f["dmin"][n, b]
            assert np.array_equal(got["sc"], f["sc"][n, b])
            assert np.array_equal(got["m"], f["m"][n, b])
            assert np.array_equal(got["q"], f["q"][n, 256 * b:256 * (b + 1)])


def test_q6k_field_roundtrip():
    rng = np.random.default_rng(22)
    f = synth.q6k_fields(rng, 8, 768)
    f["s"][0, 0] = np.arange(-128, 128, 16)
    enc = synth.q6k_encode(f)
    for n in range(8):
        for b in range(3):
            got = oracle.q6k_fields(enc[n, b])
            assert got["d"] == f["d"][n, b]
            assert np.array_equal(got["s"], f["s"][n, b])
            assert np.array_equal(got["q"], f["q"][n, 256 * b:256 * (b + 1)])


# ----------------------------------------------------------------------------
# Unpacked values against exact rationals
# ----------------------------------------------------------------------------

def _expect(exact: Fraction, dtype: int) -> int:
    """RN_t(exact) by brute-force nearest search."""
    if dtype == oracle.F16:
        return int(np.array(nearest_even(exact, "f16"), np.float16).view(np.uint16))
    return nearest_even_bf16(exact)


def _expect_two_step(exact: Fraction, dtype: int) -> int:
    """RN_t(RN_32(exact)): what a binary32 intermediate would give."""
    return _expect(Fraction(float(nearest_even(exact, "f32"))), dtype)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_q4k_values_exact_rationals(dtype):
    rng = np.random.default_rng(31 + dtype)
    f = synth.q4k_fields(rng, 64, 256)
    n_exact32 = 0
    for n in range(64):
        d, dm = int(f["d"][n, 0]), int(f["dmin"][n, 0])
        for k in range(0, 256, 7):
            j = k // 32
            sc, m, q = int(f["sc"][n, 0, j]), int(f["m"][n, 0, j]), int(f["q"][n, k])
            exact = f16_val(d) * sc * q - f16_val(dm) * m
            got = oracle.q4k_weight(d, dm, sc, m, q, dtype)
            assert got == _expect(exact, dtype), (d, dm, sc, m, q)
            # at these distributions the exact weight fits binary32, so a
            # binary32 intermediate would give the same bits
            n_exact32 += Fraction(float(np.float32(float(exact)))) == exact
    assert n_exact32 == 64 * len(range(0, 256, 7))


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_q4k_values_wide_exponent_gap(dtype):
    """d and dmin far apart in magnitude: the exact value needs more than 24
    bits, and the single rounding is still taken from the exact value."""
    rng = np.random.default_rng(41 + dtype)
    hit_inexact = 0
    for _ in range(3000):
        d = int(synth.f16_bits(rng.uniform(0.5, 8.0)))
        dm = int(synth.f16_bits(rng.uniform(2.0 ** -20, 2.0 ** -12)))
        sc, m, q = (int(v) for v in rng.integers([1, 1, 1], [64, 64, 16]))
        exact = f16_val(d) * sc * q - f16_val(dm) * m
        hit_inexact += Fraction(float(np.float32(float(exact)))) != exact
        assert oracle.q4k_weight(d, dm, sc, m, q, dtype) == _expect(exact, dtype)
    assert hit_inexact > 100


def test_q4k_single_rounding():
    """Inputs where a binary32 intermediate would change the result: factor*q
    sits exactly on a midpoint of the target grid and the bias is a quarter of
    a binary32 ulp.  The oracle rounds the exact value once."""
    cases = [  # (d, dmin, sc, m, q, dtype)
        (0x3C01, 0x0001, 1, 1, 3, oracle.F16),   # 3075*2^-10 - 2^-24: fp16 tie at 1537.5 ulps
        (0x400C, 0x0001, 1, 1, 1, oracle.BF16),  # 1036*2^-9 - 2^-24: bf16 tie at 129.5 ulps
    ]
    for d, dm, sc, m, q, dtype in cases:
        exact = f16_val(d) * sc * q - f16_val(dm) * m
        direct = _expect(exact, dtype)
        assert direct != _expect_two_step(exact, dtype)
        assert oracle.q4k_weight(d, dm, sc, m, q, dtype) == direct


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_q6k_values_exact_rationals(dtype):
    rng = np.random.default_rng(51 + dtype)
    ds = list(synth.f16_bits(rng.uniform(1e-3, 1e-2, 300))) + [0x0001, 0x03FF, 0x7BFF, 0x3C00]
    for d in ds:
        d = int(d)
        for s, q in zip(rng.integers(-128, 128, 8), rng.integers(0, 64, 8)):
            exact = f16_val(d) * int(s) * (int(q) - 32)
            assert oracle.q6k_weight(d, int(s), int(q), dtype) == _expect(exact, dtype)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_w4a16_values_exact_rationals(dtype):
    rng = np.random.default_rng(61 + dtype)
    for s in synth.f16_bits(rng.uniform(1e-3, 1e-2, 200)):
        for q in range(16):
            zp = int(rng.integers(0, 16))
            exact = f16_val(int(s)) * (q - zp)
            want = _expect(exact, dtype)
            assert oracle.w4a16_weight(int(s), q, zp, dtype) == want
            if dtype == oracle.F16:
                # the packed-fp16 route of the W4A16 PR: (1024+q)-(1024+zp) is
                # exact, then one fp16 multiply
                a = np.array(0x6400 | q, np.uint16).view(np.float16)
                b = np.array(0x6400 | zp, np.uint16).view(np.float16)
                sv = np.array(s, np.uint16).view(np.float16)
                assert int(np.array((a - b) * sv, np.float16).view(np.uint16)) == want


# ----------------------------------------------------------------------------
# Special cases with closed-form answers (array walk, layout [K][N])
# ----------------------------------------------------------------------------

def test_q4k_special_cases():
    N, K = 4, 512
    one, half = 0x3C00, 0x3800
    f = {"d": np.full((N, 2), one, np.uint16), "dmin": np.zeros((N, 2), np.uint16),
         "sc": np.ones((N, 2, 8), np.uint8), "m": np.zeros((N, 2, 8), np.uint8),
         "q": np.random.default_rng(5).integers(0, 16, (N, K), dtype=np.uint8)}
    W = oracle.dequant_q4k(synth.q4k_encode(f), N, K, oracle.F16).view(np.float16)
    assert np.array_equal(W.astype(np.float64), f["q"].T.astype(np.float64))  # w = q
    # sub-block j covers k in [32j, 32j+32): scale j+1 on unit codes
    f["q"][:] = 1
    f["sc"][:] = np.arange(1, 9, dtype=np.uint8)
    W = oracle.dequant_q4k(synth.q4k_encode(f), N, K, oracle.F16).view(np.float16)
    assert np.array_equal(W[:, 0].astype(np.float64), (np.arange(K) % 256) // 32 + 1)
    # q = 0: w = -dmin*m
    f["q"][:] = 0
    f["dmin"][:] = half
    f["m"][:] = np.arange(8, dtype=np.uint8) * 3
    W = oracle.dequant_q4k(synth.q4k_encode(f), N, K, oracle.BF16)
    wv = oracle.bits_to_double_fast(W, oracle.BF16)
    assert np.array_equal(wv[:, 2], -0.5 * 3 * ((np.arange(K) % 256) // 32))
    # all codes and mins zero: exactly zero
    f["m"][:] = 0
    W = oracle.dequant_q4k(synth.q4k_encode(f), N, K, oracle.F16)
    assert not np.any(W & 0x7FFF)


def test_q6k_special_cases():
    N, K = 3, 256
    rng = np.random.default_rng(6)
    f = {"d": np.full((N, 1), 0x3C00, np.uint16), "s": np.ones((N, 1, 16), np.int8),
         "q": rng.integers(0, 64, (N, K), dtype=np.uint8)}
    W = oracle.dequant_q6k(synth.q6k_encode(f), N, K, oracle.F16).view(np.float16)
    assert np.array_equal(W.astype(np.float64), f["q"].T.astype(np.float64) - 32)  # w = q - 32
    f["q"][:] = 33
    f["s"][:] = (np.arange(16) - 8).astype(np.int8)
    W = oracle.dequant_q6k(synth.q6k_encode(f), N, K, oracle.F16).view(np.float16)
    assert np.array_equal(W[:, 1].astype(np.float64), np.arange(K) // 16 - 8)  # scale i covers [16i, 16i+16)


def test_w4a16_special_cases():
    N, K, g = 5, 256, 128
    rng = np.random.default_rng(7)
    f = synth.w4a16_fields(rng, N, K, g, symmetric=False)
    f["zeros"][:] = f["codes"][:, ::g].T  # not equal to codes everywhere; set codes instead
    codes = np.repeat(f["zeros"].T, g, axis=1)
    W = oracle.dequant_w4a16(codes, f["scales"], f["zeros"], N, K, g, oracle.F16)
    assert not np.any(W & 0x7FFF)  # q == zp gives zero
    one = np.full_like(f["scales"], 0x3C00)
    W = oracle.dequant_w4a16(f["codes"], one, None, N, K, g, oracle.BF16)
    assert np.array_equal(oracle.bits_to_double_fast(W, oracle.BF16), f["codes"].T.astype(np.float64) - 8)
    # group index: scale of group j applies to k in [g*j, g*j+g)
    sc = np.zeros_like(f["scales"])
    sc[0, :] = 0x3C00
    sc[1, :] = 0x4000
    W = oracle.dequant_w4a16(np.full((N, K), 9, np.uint8), sc, None, N, K, g, oracle.F16).view(np.float16)
    assert np.array_equal(W[:, 0].astype(np.float64), np.where(np.arange(K) < g, 1.0, 2.0))


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16"])
def test_array_walk_matches_scalar(fmt):
    """Whole-matrix dequant places weight (k, n) at W[k][n]."""
    rng = np.random.default_rng(8)
    N, K = 6, 512
    f = synth.weight_fields(fmt, rng, N, K, group=128)
    enc = synth.encode(fmt, f)
    W = oracle.dequant(fmt, enc, N, K, oracle.F16)
    for n in range(N):
        for k in rng.integers(0, K, 20):
            b, kk = k // 256, k % 256
            if fmt == "q4k":
                want = oracle.q4k_weight(int(f["d"][n, b]), int(f["dmin"][n, b]), int(f["sc"][n, b, kk // 32]),
                                         int(f["m"][n, b, kk // 32]), int(f["q"][n, k]), oracle.F16)
            elif fmt == "q6k":
                want = oracle.q6k_weight(int(f["d"][n, b]), int(f["s"][n, b, kk // 16]), int(f["q"][n, k]),
                                         oracle.F16)
            else:
                want = oracle.w4a16_weight(int(f["scales"][k // 128, n]), int(f["codes"][n, k]),
                                           int(f["zeros"][k // 128, n]), oracle.F16)
            assert W[k, n] == want


# ----------------------------------------------------------------------------
# fp64 GEMM
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("shape", [(1, 16, 256), (5, 48, 512), (17, 33, 384)])
def test_gemm_matches_numpy(dtype, shape):
    M, N, K = shape
    rng = np.random.default_rng(9)
    X = synth.activations(rng, M, K, dtype)
    W = synth.activations(rng, K, N, dtype)
    Y, B = oracle.gemm(X, W, dtype)
    xd = oracle.bits_to_double_fast(X, dtype)
    wd = oracle.bits_to_double_fast(W, dtype)
    assert np.allclose(Y, xd @ wd, rtol=1e-12, atol=1e-12)
    assert np.allclose(B, np.abs(xd) @ np.abs(wd), rtol=1e-12, atol=1e-12)
    r = rng.integers(0, M, 30)
    c = rng.integers(0, N, 30)
    Ya, Ba = oracle.gemm_at(X, W, dtype, r, c)
    assert np.array_equal(Ya, Y[r, c]) and np.array_equal(Ba, B[r, c])


def _frac_bits(bits: int, dtype: int) -> Fraction:
    if dtype == oracle.F16:
        return f16_val(bits)
    return Fraction(float(np.array(bits << 16, np.uint32).view(np.float32)))


def _exact_weight(fmt: str, f: dict, n: int, k: int) -> Fraction:
    """W[k][n] from the logical fields by the formats' formulas, as an exact rational."""
    b = k // 256
    if fmt == "q4k":
        j = (k % 256) // 32
        return (f16_val(int(f["d"][n, b])) * int(f["sc"][n, b, j]) * int(f["q"][n, k])
                - f16_val(int(f["dmin"][n, b])) * int(f["m"][n, b, j]))
    if fmt == "q6k":
        j = (k % 256) // 16
        return f16_val(int(f["d"][n, b])) * int(f["s"][n, b, j]) * (int(f["q"][n, k]) - 32)
    g = k // f["group"]
    return f16_val(int(f["scales"][g, n])) * (int(f["codes"][n, k]) - int(f["zeros"][g, n]))


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("fmt,sym", [("q4k", False), ("q6k", False), ("w4a16", False), ("w4a16", True)])
def test_gemm_smallest_shapes_exact_rationals(fmt, sym, dtype):
    """The smallest shapes of the brute-force grid end to end in exact
    arithmetic: every weight from its fields by the format's formula, rounded
    once by the brute-force nearest search, must equal the oracle's unpack bit
    for bit, and every output of the oracle's fp64 product must lie within
    fp64 summation error of the exact rational sum of X.W."""
    rng = np.random.default_rng(71 + dtype)
    N, K = 16, 256 if fmt != "w4a16" else 128
    f = synth.weight_fields(fmt, rng, N, K, 64 if fmt == "w4a16" else 128, sym)
    W = oracle.dequant(fmt, synth.encode(fmt, f), N, K, dtype)
    Wq = [[None] * N for _ in range(K)]
    for k in range(K):
        for n in range(N):
            want = _expect(_exact_weight(fmt, f, n, k), dtype)
            assert int(W[k, n]) == want, (fmt, k, n)
            Wq[k][n] = _frac_bits(want, dtype)
    for M in (1, 2, 3):
        X = synth.activations(rng, M, K, dtype)
        Y, B = oracle.gemm(X, W, dtype)
        for m in range(M):
            xs = [_frac_bits(int(X[m, k]), dtype) for k in range(K)]
            for n in range(N):
                exact = sum(xs[k] * Wq[k][n] for k in range(K))
                bound = sum(abs(xs[k] * Wq[k][n]) for k in range(K))
                assert abs(Fraction(float(Y[m, n])) - exact) <= Fraction(K + 2, 2 ** 53) * bound, (fmt, m, n)
                assert abs(Fraction(float(B[m, n])) - bound) <= Fraction(K + 2, 2 ** 53) * bound


def test_gemm_special_cases():
    rng = np.random.default_rng(10)
    K, N = 64, 24
    W = synth.activations(rng, K, N, oracle.F16)
    eye = synth.f16_bits(np.eye(K))
    Y, _ = oracle.gemm(eye, W, oracle.F16)
    assert np.array_equal(Y, oracle.bits_to_double_fast(W, oracle.F16))  # identity rows select W
    ones = synth.f16_bits(np.ones((3, K)))
    Y, _ = oracle.gemm(ones, W, oracle.F16)
    colsum = oracle.bits_to_double_fast(W, oracle.F16).sum(axis=0)
    assert np.allclose(Y, np.broadcast_to(colsum, Y.shape), rtol=1e-15, atol=1e-15)
    Y, B = oracle.gemm(ones, np.zeros((K, N), np.uint16), oracle.F16)
    assert not Y.any() and not B.any()


def test_gemm_error_rule():
    Yref = np.array([[1.0, 0.0], [2.0, -3.0]])
    B = np.array([[10.0, 0.0], [4.0, 6.0]])
    Yb = synth.f16_bits(np.array([[1.01, 0.0], [2.0, -3.0]]))
    err, zero_ok = oracle.gemm_error(Yb, Yref, B, oracle.F16)
    assert zero_ok and abs(err - abs(float(np.float16(1.01)) - 1.0) / 10.0) < 1e-12


# ---- fragment-major activations (a layout of the library under test) ------

@pytest.mark.parametrize("M,K", [(1, 128), (32, 256), (40, 384), (65, 128)])
def test_fragment_major_is_an_axis_permutation(M, K):
    """The copy equals X (zero-padded to whole 32-row blocks) with its axes
    m = 32b + r, k = 128c + 16s + 8h + j reordered to (b, c, s, h, r, j)."""
    rng = np.random.default_rng(M * 1000 + K)
    X = rng.integers(0, 1 << 16, (M, K), dtype=np.uint16)
    Mp = -(-M // 32) * 32
    Xp = np.zeros((Mp, K), np.uint16)
    Xp[:M] = X
    want = Xp.reshape(Mp // 32, 32, K // 128, 8, 2, 8).transpose(0, 2, 3, 4, 1, 5).ravel()
    assert np.array_equal(oracle.fragment_major(X), want)


def test_fragment_major_operand_blocks():
    """Each 1 KB block is the activation operand of one 32x32x16 MFMA k-step
    in lane order: lane (r, h) holds row 32b+r, k = 128c + 16s + 8h .. +7
    (zeros for rows past M)."""
    M, K = 70, 256
    rng = np.random.default_rng(77)
    X = rng.integers(1, 1 << 16, (M, K), dtype=np.uint16)
    f = oracle.fragment_major(X)
    assert f.size == 96 * K
    nch = K // 128
    for b in range(3):
        for c in range(nch):
            for s in range(8):
                blk = f[((b * nch + c) * 8 + s) * 512:][:512].reshape(64, 8)
                for lane in range(64):
                    r, h = lane % 32, lane // 32
                    m, k0 = 32 * b + r, 128 * c + 16 * s + 8 * h
                    want = X[m, k0:k0 + 8] if m < M else np.zeros(8, np.uint16)
                    assert np.array_equal(blk[lane], want), (b, c, s, lane)
    with pytest.raises(ValueError):
        oracle.fragment_major(np.zeros((4, 200), np.uint16))


# ----------------------------------------------------------------------------
# int8-activation variant (qref.c item 5): binary32 weights, per-column and
# per-row scales, int8 codes, integer GEMM with a binary32 epilogue
# ----------------------------------------------------------------------------

def _rne_int(x: Fraction) -> int:
    """Nearest integer to an exact rational, ties to even."""
    f = math.floor(x)
    d = x - f
    if d > Fraction(1, 2):
        return f + 1
    if d < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def _f32(x: Fraction) -> Fraction:
    return Fraction(float(nearest_even(x, "f32")))


def _amax_samples(rng):
    vals = [1.0, 127.0, 254.0, 0.5, 3.0, 2.0 ** -14, 2.0 ** -20, 65504.0, 1e-3, 7.25]
    vals += list(np.float32(rng.uniform(1e-3, 40.0, 200)))
    vals += list(np.float32(np.exp2(rng.uniform(-30, 30, 200))))
    return [float(np.float32(v)) for v in vals]


def test_i8_scales_exact_rationals():
    """r = RN_f32(127/amax) and s = RN_f32(amax/127), checked against the exact
    quotient rounded by brute-force nearest search; a zero column gives 0, 0."""
    rng = np.random.default_rng(501)
    for amax in _amax_samples(rng):
        W = np.array([[amax], [-amax / 2], [0.0]], np.float32)
        r, s = oracle.colscale_i8(W)
        assert Fraction(float(r[0])) == _f32(Fraction(127) / Fraction(amax)), amax
        assert Fraction(float(s[0])) == _f32(Fraction(amax) / 127), amax
        Wn = -W  # the column's extreme is negative now
        r2, s2 = oracle.colscale_i8(Wn)
        assert r2[0] == r[0] and s2[0] == s[0]
    r, s = oracle.colscale_i8(np.zeros((5, 3), np.float32))
    assert not r.any() and not s.any()


def test_i8_codes_ties_and_range():
    """Row amax 127 makes r = s = 1 exactly, so the codes are the values
    rounded to the nearest integer, ties to even (the pages' RNE reading)."""
    vals = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0, 0.0, -1.25, 64.75]
    want = [127, 2, 4, -2, -4, 0, 0, 2, 126, -127, 0, -1, 65]
    X = synth.f16_bits(np.array([vals]))
    Q, s = oracle.quant_rows_i8(X, oracle.F16)
    assert Q.tolist() == [want] and s[0] == np.float32(1.0)
    # amax 254: r = 1/2, so x = 5 -> 2.5 -> 2 and x = 7 -> 3.5 -> 4
    X = synth.f16_bits(np.array([[254.0, 5.0, 7.0, -5.0, 1.0]]))
    Q, s = oracle.quant_rows_i8(X, oracle.F16)
    assert Q.tolist() == [[127, 2, 4, -2, 0]] and s[0] == np.float32(2.0)
    # an all-zero row: codes 0, scale 0
    Q, s = oracle.quant_rows_i8(np.zeros((2, 64), np.uint16), oracle.BF16)
    assert not Q.any() and not s.any()
    # bf16 rows below and at the 2^-96 floor: scale 0 below it, full codes at it
    tiny = synth.bf16_bits_from_f32(np.array([[2.0 ** -100, -2.0 ** -101, 0.0], [2.0 ** -96, -2.0 ** -97, 0.0]]))
    Q, s = oracle.quant_rows_i8(tiny, oracle.BF16)
    assert Q.tolist() == [[0, 0, 0], [127, -64, 0]] and s[0] == 0.0
    assert Fraction(float(s[1])) == _f32(Fraction(2) ** -96 / 127)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_i8_codes_exact_rationals(dtype):
    """Every code is RNE(x * r) of the exact product, within [-127, 127], and
    the element of largest magnitude gets +-127."""
    rng = np.random.default_rng(502 + dtype)
    X = synth.activations(rng, 6, 256, dtype)
    X[3, 17] = X[3, 17] ^ 0x8000  # flip one sign: extremes of both signs
    Q, s = oracle.quant_rows_i8(X, dtype)
    xd = oracle.bits_to_double_fast(X, dtype)
    for m in range(X.shape[0]):
        amax = Fraction(float(np.abs(xd[m]).max()))
        r = _f32(Fraction(127) / amax)
        assert Fraction(float(s[m])) == _f32(amax / 127)
        for k in range(0, 256, 3):
            assert int(Q[m, k]) == _rne_int(Fraction(float(xd[m, k])) * r), (m, k)
        assert abs(int(Q[m, int(np.abs(xd[m]).argmax())])) == 127
        assert np.abs(Q[m].astype(int)).max() == 127


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16"])
def test_dequant_f32_matches_exact(fmt):
    """Binary32 weights are the exact weight rounded once to binary32; at the
    pages' distributions that rounding is exact, and the fp16 dequant of the
    same weight is the binary32 value rounded once more."""
    rng = np.random.default_rng(503)
    N, K = 24, 512
    f = synth.weight_fields(fmt, rng, N, K, 128, False)
    enc = synth.encode(fmt, f)
    W32 = oracle.dequant_f32(fmt, enc, N, K)
    W16 = oracle.dequant(fmt, enc, N, K, oracle.F16)
    assert np.array_equal(W32.astype(np.float16).view(np.uint16), W16)
    for k in range(0, K, 5):
        for n in range(0, N, 3):
            if fmt == "q4k":
                b, kk = divmod(k, 256)
                j = kk // 32
                exact = (f16_val(int(f["d"][n, b])) * int(f["sc"][n, b, j]) * int(f["q"][n, k])
                         - f16_val(int(f["dmin"][n, b])) * int(f["m"][n, b, j]))
            elif fmt == "q6k":
                b, kk = divmod(k, 256)
                exact = f16_val(int(f["d"][n, b])) * int(f["s"][n, b, kk // 16]) * (int(f["q"][n, k]) - 32)
            else:
                gi = k // 128
                exact = f16_val(int(f["scales"][gi, n])) * (int(f["codes"][n, k]) - int(f["zeros"][gi, n]))
            assert Fraction(float(W32[k, n])) == exact, (k, n)


def test_dequant_f32_rounds_once():
    """With d and dmin far apart the exact Q4_K weight needs more than 24 bits:
    the binary32 weight is then its nearest binary32 value."""
    rng = np.random.default_rng(504)
    N, K = 8, 256
    f = synth.q4k_fields(rng, N, K)
    f["d"][:] = synth.f16_bits(rng.uniform(0.5, 8.0, f["d"].shape))
    f["dmin"][:] = synth.f16_bits(rng.uniform(2.0 ** -20, 2.0 ** -12, f["dmin"].shape))
    W32 = oracle.dequant_f32("q4k", synth.q4k_encode(f), N, K)
    inexact = 0
    for n in range(N):
        for k in range(K):
            j = k // 32
            exact = (f16_val(int(f["d"][n, 0])) * int(f["sc"][n, 0, j]) * int(f["q"][n, k])
                     - f16_val(int(f["dmin"][n, 0])) * int(f["m"][n, 0, j]))
            got = Fraction(float(W32[k, n]))
            inexact += got != exact
            assert got == _f32(exact), (n, k)
    assert inexact > 0


def test_requant_i8_exact_rationals():
    """Weight codes are RNE(w * r_n) of the exact product; each column's
    largest-magnitude weight gets +-127; a constant column is all 127."""
    rng = np.random.default_rng(505)
    N, K = 12, 512
    f = synth.q4k_fields(rng, N, K)
    W32 = oracle.dequant_f32("q4k", synth.q4k_encode(f), N, K)
    W32[:, 5] = np.float32(0.3)
    r, s = oracle.colscale_i8(W32)
    Q = oracle.requant_i8(W32, r)
    assert (Q[:, 5] == 127).all()
    for n in range(N):
        assert abs(int(Q[int(np.abs(W32[:, n]).argmax()), n])) == 127
        for k in range(0, K, 7):
            assert int(Q[k, n]) == _rne_int(Fraction(float(W32[k, n])) * Fraction(float(r[n]))), (k, n)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_gemm_i8_unit_scales_is_integer_dot(dtype):
    """With unit scales the output is the integer dot product (numpy int64
    matmul) rounded to binary32 and then to the output type."""
    rng = np.random.default_rng(506 + dtype)
    M, N, K = 7, 9, 1024
    Qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Qw = rng.integers(-127, 128, (K, N)).astype(np.int8)
    Qx[:, :40] = 127  # push some sums past 2^24 / 2^11 so both roundings act
    Qw[:40, :] = 127
    one = np.ones(M, np.float32), np.ones(N, np.float32)
    Y = oracle.gemm_i8(Qx, one[0], Qw, one[1], dtype)
    acc = Qx.astype(np.int64) @ Qw.astype(np.int64)
    y32 = acc.astype(np.float32)
    if dtype == oracle.F16:
        with np.errstate(over="ignore"):  # sums past 65504 become inf in both
            want = y32.astype(np.float16).view(np.uint16)
    else:
        want = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_gemm_i8_scaled_matches_numpy_binary32(dtype):
    """Scaled epilogue against numpy's own binary32 arithmetic: RN_f32(acc),
    RN_f32(sx*sw), their RN_f32 product, then RN_t."""
    rng = np.random.default_rng(508 + dtype)
    M, N, K = 11, 13, 768
    Qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Qw = rng.integers(-127, 128, (K, N)).astype(np.int8)
    sx = np.float32(rng.uniform(1e-3, 0.1, M))
    sw = np.float32(np.exp2(rng.uniform(-14, -4, N)))
    Y = oracle.gemm_i8(Qx, sx, Qw, sw, dtype)
    acc = (Qx.astype(np.int64) @ Qw.astype(np.int64)).astype(np.float32)
    y32 = acc * (sx[:, None] * sw[None, :])
    assert y32.dtype == np.float32
    if dtype == oracle.F16:
        want = y32.astype(np.float16).view(np.uint16)
    else:
        want = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16"])
def test_gemm_i8_chain_close_to_fp64_product(fmt):
    """The whole int8 chain stays within its quantization error of the exact
    product X . W: |Y - XW| <= sum_k (|x| sw/2 + sx/2 |w| + sx sw/4) plus the
    binary32 and output roundings (a bound from the definitions alone)."""
    rng = np.random.default_rng(510)
    M, N, K = 9, 20, 512
    X = synth.activations(rng, M, K, oracle.F16)
    f = synth.weight_fields(fmt, rng, N, K, 128, False)
    enc = synth.encode(fmt, f)
    W32 = oracle.dequant_f32(fmt, enc, N, K)
    r, sw = oracle.colscale_i8(W32)
    Qw = oracle.requant_i8(W32, r)
    Qx, sx = oracle.quant_rows_i8(X, oracle.F16)
    Y = oracle.bits_to_double_fast(oracle.gemm_i8(Qx, sx, Qw, sw, oracle.F16), oracle.F16)
    xd = oracle.bits_to_double_fast(X, oracle.F16)
    wd = W32.astype(np.float64)
    exact = xd @ wd
    sxd, swd = sx.astype(np.float64), sw.astype(np.float64)
    # 1/r and s differ by at most a few binary32 ulps: allow 1e-6 relative slack
    q_err = (np.abs(xd) @ np.ones((K, N)) * swd[None, :] / 2 + sxd[:, None] / 2 * (np.ones((M, K)) @ np.abs(wd))
             + K * sxd[:, None] * swd[None, :] / 4) * (1 + 1e-6)
    bound = q_err + np.abs(exact) * 3e-7 + np.abs(Y) * 2.0 ** -11
    assert (np.abs(Y - exact) <= bound).all()
    # and the bound is not vacuous: the error is a small fraction of |X||W|
    assert (np.abs(Y - exact) <= 0.05 * (np.abs(xd) @ np.abs(wd))).all()


@pytest.mark.parametrize("M,K", [(1, 32), (32, 256), (40, 384), (65, 128)])
def test_fragment_major_i8_is_an_axis_permutation(M, K):
    """The int8 copy equals the codes (zero-padded to whole 32-row blocks) with
    their axes m = 32b + r, k = 32s + 16h + j reordered to (b, s, h, r, j):
    each 1 KB is one 32x32x32 int8 MFMA operand in lane order."""
    rng = np.random.default_rng(M * 100 + K)
    Q = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Mp = -(-M // 32) * 32
    Qp = np.zeros((Mp, K), np.int8)
    Qp[:M] = Q
    want = Qp.reshape(Mp // 32, 32, K // 32, 2, 16).transpose(0, 2, 3, 1, 4).ravel()
    assert np.array_equal(oracle.fragment_major_i8(Q), want)
    with pytest.raises(ValueError):
        oracle.fragment_major_i8(np.zeros((4, 48), np.int8))
