"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every function include/qgemm.h declares, the packers invert exactly and put
each code where the header says, argument errors come back as status codes
before any launch, and the M-ladder keeps its invariants."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")


def header_functions() -> set[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(qgemm_[a-z0-9_]+)\s*\(", text))


def test_library_exports_every_declared_function():
    lib = qg.lib()
    declared = header_functions()
    assert len(declared) >= 18
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in qgemm.h but not exported"
    assert declared == set(qg.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings():
    lib = qg.lib()
    for code in qg.STATUS:
        s = lib.qgemm_status_str(code)
        assert s and s.decode() != "unknown status"
    assert lib.qgemm_status_str(12345).decode() == "unknown status"


# ----------------------------------------------------------------------------
# packers
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 256), (16, 512), (33, 1024), (512, 1024)])
def test_q4k_roundtrip_and_size(N, K):
    rng = np.random.default_rng(N + K)
    blocks = synth.q4k_encode(synth.q4k_fields(rng, N, K))
    packed = qg.q4k_pack(blocks, N, K)
    assert packed.nbytes == -(-N // 16) * 16 * (K // 256) * 144  # 0.5625 B per weight, panel-padded
    assert np.array_equal(qg.q4k_unpack(packed, N, K), blocks)


@pytest.mark.parametrize("N,K", [(1, 256), (20, 768), (64, 1024)])
def test_q6k_roundtrip_and_size(N, K):
    rng = np.random.default_rng(N * 3 + K)
    blocks = synth.q6k_encode(synth.q6k_fields(rng, N, K))
    packed = qg.q6k_pack(blocks, N, K)
    assert packed.nbytes == -(-N // 16) * 16 * (K // 256) * 210
    assert np.array_equal(qg.q6k_unpack(packed, N, K), blocks)


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("sym", [False, True])
def test_w4a16_roundtrip_and_size(group, sym):
    N, K = 40, 512
    rng = np.random.default_rng(group + sym)
    f = synth.w4a16_fields(rng, N, K, group, sym)
    zeros = None if sym else f["zeros"]
    packed = qg.w4a16_pack(f["codes"], f["scales"], zeros, N, K, group)
    npan = -(-N // 16)
    assert packed.nbytes == npan * 16 * K // 2 + npan * 16 * (K // group) * 2 + (0 if sym else npan * 16 * (K // group) // 2)
    codes, scales, z = qg.w4a16_unpack(packed, N, K, group, not sym)
    assert np.array_equal(codes, f["codes"]) and np.array_equal(scales, f["scales"])
    if not sym:
        assert np.array_equal(z, f["zeros"])


def _pair_order_code(run16: np.ndarray, t: int) -> int:
    """Code t of a 16-byte run in pair order, read the way the header states."""
    word = int(run16[4 * (t // 8):4 * (t // 8) + 4].view("<u4")[0])
    pair, half = (t % 8) // 2, t % 2
    return (word >> (16 * half + 4 * pair)) & 15


def test_q4k_layout_matches_header():
    N, K = 20, 512
    rng = np.random.default_rng(5)
    f = synth.q4k_fields(rng, N, K)
    packed = qg.q4k_pack(synth.q4k_encode(f), N, K)
    for n in (0, 7, 16, 19):
        p, c = n // 16, n % 16
        for b in range(K // 256):
            rec = packed[(p * (K // 256) + b) * 2304:][:2304]
            hdr = rec[16 * c:16 * c + 16]
            assert int(hdr[0:2].view("<u2")[0]) == f["d"][n, b]
            assert int(hdr[2:4].view("<u2")[0]) == f["dmin"][n, b]
            for k in rng.integers(0, 256, 40):
                h, g, t = k // 128, (k % 128) // 32, k % 32
                run = rec[256 + 1024 * h + (16 * g + c) * 16:][:16]
                assert _pair_order_code(run, int(t)) == f["q"][n, 256 * b + k]


def test_q6k_layout_matches_header():
    N, K = 17, 256
    rng = np.random.default_rng(6)
    f = synth.q6k_fields(rng, N, K)
    packed = qg.q6k_pack(synth.q6k_encode(f), N, K)
    for n in (0, 5, 16):
        p, c = n // 16, n % 16
        rec = packed[p * 3360:][:3360]
        assert int(rec[2 * c:2 * c + 2].view("<u2")[0]) == f["d"][n, 0]
        assert np.array_equal(rec[32 + 16 * c:48 + 16 * c].view(np.int8), f["s"][n, 0])
        for k in range(256):
            h, g, t = k // 128, (k % 128) // 32, k % 32
            lo = _pair_order_code(rec[288 + 1024 * h + (16 * g + c) * 16:][:16], t)
            hi_words = rec[2336 + 512 * h + (16 * g + c) * 8:][:8].view("<u4")
            i, u, pr = t // 8, (t // 8) % 2, (t % 8) // 2
            bit = 16 * (t % 2) + 2 * (4 * u + pr)
            hi = (int(hi_words[t // 16]) >> bit) & 3
            assert lo | (hi << 4) == f["q"][n, k]


def test_w4a16_layout_matches_header():
    N, K, group = 18, 256, 64
    rng = np.random.default_rng(7)
    f = synth.w4a16_fields(rng, N, K, group, False)
    packed = qg.w4a16_pack(f["codes"], f["scales"], f["zeros"], N, K, group)
    npan, nch, ng = 2, K // 128, K // group
    sreg, zreg = npan * nch * 1024, npan * nch * 1024 + npan * ng * 32
    for n in (0, 3, 17):
        p, c = n // 16, n % 16
        for k in range(0, K, 5):
            ch, g, t = k // 128, (k % 128) // 32, k % 32
            run = packed[(p * nch + ch) * 1024 + (16 * g + c) * 16:][:16]
            assert _pair_order_code(run, t) == f["codes"][n, k]
        for j in range(ng):
            assert int(packed[sreg + (p * ng + j) * 32 + 2 * c:][:2].view("<u2")[0]) == f["scales"][j, n]
            assert (packed[zreg + (p * ng + j) * 8 + c // 2] >> (4 * (c % 2))) & 15 == f["zeros"][j, n]


def test_packer_errors():
    lib = qg.lib()
    buf = np.zeros(4096, np.uint8)
    p = ctypes.c_void_p(buf.ctypes.data)
    assert lib.qgemm_q4k_pack(None, 16, 256, p, buf.nbytes) == -1
    assert lib.qgemm_q4k_pack(p, 16, 300, p, buf.nbytes) == -2
    assert lib.qgemm_q4k_pack(p, 0, 256, p, buf.nbytes) == -2
    assert lib.qgemm_q4k_pack(p, 16, 256, p, 100) == -6
    assert lib.qgemm_q4k_packed_bytes(16, 100) == 0
    assert lib.qgemm_w4a16_packed_bytes(16, 256, 48, 1) == 0
    codes = np.full((16, 256), 16, np.uint8)  # 16 does not fit four bits
    scales = np.zeros((2, 16), np.uint16)
    with pytest.raises(qg.QGemmError) as e:
        qg.w4a16_pack(codes, scales, None, 16, 256, 128)
    assert e.value.status == -8


# ----------------------------------------------------------------------------
# device entry points: argument errors are detected before any launch
# ----------------------------------------------------------------------------

def test_device_entry_argument_errors():
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)        # never dereferenced: each call below fails validation
    mis = ctypes.c_void_p((1 << 20) + 8)
    s = None
    assert lib.qgemm_q4k(None, A, A, 4, 16, 256, 0, s) == -1
    assert lib.qgemm_q4k(A, A, A, 4, 16, 200, 0, s) == -2
    assert lib.qgemm_q4k(A, A, A, -1, 16, 256, 0, s) == -2
    assert lib.qgemm_q4k(A, A, A, 4, 0, 256, 0, s) == -2
    assert lib.qgemm_q4k(A, A, A, 4, 16, 256, 7, s) == -3
    assert lib.qgemm_q6k(A, mis, A, 4, 16, 256, 0, s) == -4
    assert lib.qgemm_w4a16(A, A, A, 4, 16, 256, 48, 1, 0, s) == -5
    assert lib.qgemm_w4a16(A, A, A, 4, 16, 192, 64, 1, 0, s) == -2
    assert lib.qgemm_w4a16(A, A, A, 4, 16, 256, 0, 1, 0, s) == -5
    assert lib.qgemm_gemm_rung(0, 99, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -5
    assert lib.qgemm_gemm_rung(7, 0, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -5
    # M == 0 is a no-op that touches nothing
    assert lib.qgemm_q4k(None, None, None, 0, 16, 256, 0, s) == 0
    assert lib.qgemm_dequant(0, None, A, 16, 256, 0, 0, 0, s) == -1
    assert lib.qgemm_dequant(2, A, A, 16, 256, 0, 0, 0, s) == -5
    # grouped per-expert GEMM
    assert lib.qgemm_grouped(0, A, A, A, A, 0, 8, 16, 256, 0, 0, 0, s) == -2       # E < 1
    assert lib.qgemm_grouped(0, A, A, A, None, 2, 8, 16, 256, 0, 0, 0, s) == -1    # offsets NULL
    assert lib.qgemm_grouped(0, A, A, A, ctypes.c_void_p((1 << 20) + 2), 2, 8, 16, 256, 0, 0, 0, s) == -4
    assert lib.qgemm_grouped(2, A, A, A, A, 2, 8, 16, 128, 128, 1, 0, s) == -4     # 1064-byte experts
    assert lib.qgemm_grouped(0, None, None, None, None, 3, 0, 16, 256, 0, 0, 0, s) == 0  # T = 0
    assert lib.qgemm_grouped(1, A, A, A, A, 2, 8, 16, 300, 0, 0, 0, s) == -2
    # the same checks on fragment-major routed rows
    assert lib.qgemm_grouped_xf(0, A, A, A, A, 0, 8, 16, 256, 0, 0, 0, s) == -2
    assert lib.qgemm_grouped_xf(0, A, A, A, None, 2, 8, 16, 256, 0, 0, 0, s) == -1
    assert lib.qgemm_grouped_xf(0, mis, A, A, ctypes.c_void_p((1 << 20) + 2), 2, 8, 16, 256, 0, 0, 0, s) == -4
    assert lib.qgemm_grouped_xf(0, None, None, None, None, 3, 0, 16, 256, 0, 0, 0, s) == 0
    assert lib.qgemm_grouped_xf(0, A, A, A, A, 2, 8, 16, 256, 0, 0, 5, s) == -3
    assert lib.qgemm_grouped_xf(0, A, A, A, A, 2, 1 << 20, 16, 256, 0, 0, 0, s) == -2  # grid.y beyond 65535
    # staged arm: scratch checks come before any launch
    need = lib.qgemm_staged_scratch_bytes(20, 512)
    assert need == 32 * 512 * 2 and lib.qgemm_staged_scratch_bytes(20, 200) == 0
    assert lib.qgemm_staged(0, A, A, None, need, A, 4, 20, 512, 0, 0, 0, s) == -1
    assert lib.qgemm_staged(0, A, A, A, need - 16, A, 4, 20, 512, 0, 0, 0, s) == -6
    assert lib.qgemm_staged(0, A, A, mis, need, A, 4, 20, 512, 0, 0, 0, s) == -4
    assert lib.qgemm_staged(1, A, A, A, need, A, 4, 20, 500, 0, 0, 0, s) == -2
    assert lib.qgemm_staged(2, A, A, A, need, A, 4, 20, 512, 0, 1, 0, s) == -5
    # fragment-major activations
    assert lib.qgemm_xf_bytes(1, 128) == 32 * 128 * 2 and lib.qgemm_xf_bytes(33, 256) == 64 * 256 * 2
    assert lib.qgemm_xf_bytes(0, 128) == 0 and lib.qgemm_xf_bytes(-1, 128) == 0
    assert lib.qgemm_xf_bytes(4, 200) == 0 and lib.qgemm_xf_bytes(4, 0) == 0
    assert lib.qgemm_x_to_xf(A, A, 4, 200, s) == -2
    assert lib.qgemm_x_to_xf(A, A, -1, 128, s) == -2
    assert lib.qgemm_x_to_xf(None, A, 4, 128, s) == -1
    assert lib.qgemm_x_to_xf(A, mis, 4, 128, s) == -4
    assert lib.qgemm_x_to_xf(None, None, 0, 128, s) == 0     # M = 0
    assert lib.qgemm_gemm_xf(0, -1, None, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -1
    assert lib.qgemm_gemm_xf(0, -1, mis, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -4
    assert lib.qgemm_gemm_xf(0, 99, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -5
    assert lib.qgemm_gemm_xf(2, -1, A, A, A, 4, 16, 256, 48, 1, 0, None, 0, s) == -5
    assert lib.qgemm_gemm_xf(1, -1, A, A, A, 4, 16, 300, 0, 0, 0, None, 0, s) == -2
    assert lib.qgemm_gemm_xf(0, -1, A, A, A, 4, 16, 256, 0, 0, 5, None, 0, s) == -3
    assert lib.qgemm_gemm_xf(0, -1, None, None, None, 0, 16, 256, 0, 0, 0, None, 0, s) == 0


def test_i8_entry_argument_errors():
    """The int8 path's entry points reject bad arguments before any launch."""
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    odd4 = ctypes.c_void_p((1 << 20) + 2)
    s = None
    assert lib.qgemm_i8_xq_bytes(1, 32) == 32 * 32 and lib.qgemm_i8_xq_bytes(33, 256) == 64 * 256
    assert lib.qgemm_i8_xq_bytes(4, 48) == 0 and lib.qgemm_i8_xq_bytes(-1, 64) == 0 and lib.qgemm_i8_xq_bytes(4, 0) == 0
    # quantize
    assert lib.qgemm_i8_quantize(A, A, A, 4, 48, 0, s) == -2
    assert lib.qgemm_i8_quantize(A, A, A, -1, 64, 0, s) == -2
    assert lib.qgemm_i8_quantize(A, A, A, 4, 64, 5, s) == -3
    assert lib.qgemm_i8_quantize(None, A, A, 4, 64, 0, s) == -1
    assert lib.qgemm_i8_quantize(A, A, None, 4, 64, 0, s) == -1
    assert lib.qgemm_i8_quantize(A, mis, A, 4, 64, 0, s) == -4
    assert lib.qgemm_i8_quantize(A, A, odd4, 4, 64, 0, s) == -4
    assert lib.qgemm_i8_quantize(None, None, None, 0, 64, 0, s) == 0   # M = 0
    # colscale
    assert lib.qgemm_i8_colscale(0, A, A, A, 16, 200, 0, 0, s) == -2
    assert lib.qgemm_i8_colscale(3, A, A, A, 16, 256, 0, 0, s) == -5
    assert lib.qgemm_i8_colscale(2, A, A, A, 16, 256, 0, 1, s) == -5   # W4A16 without a group size
    assert lib.qgemm_i8_colscale(0, None, A, A, 16, 256, 0, 0, s) == -1
    assert lib.qgemm_i8_colscale(0, A, odd4, A, 16, 256, 0, 0, s) == -4
    assert lib.qgemm_i8_colscale(0, mis, A, A, 16, 256, 0, 0, s) == -4
    # gemm
    g = lib.qgemm_i8_gemm
    assert g(0, -1, A, A, A, A, A, A, 4, 16, 200, 0, 0, 0, None, 0, s) == -2
    assert g(0, -1, A, A, A, A, A, A, 4, 16, 262144, 0, 0, 0, None, 0, s) == -2  # int32 sums would overflow
    assert g(0, -1, A, A, A, A, A, A, 4, 16, 256, 0, 0, 9, None, 0, s) == -3
    assert g(0, 99, A, A, A, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -5
    assert g(2, -1, A, A, A, A, A, A, 4, 16, 256, 48, 1, 0, None, 0, s) == -5
    assert g(0, -1, A, None, A, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -1
    assert g(0, -1, A, A, A, A, None, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -1
    assert g(0, -1, mis, A, A, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -4
    assert g(0, -1, A, odd4, A, A, A, A, 4, 16, 256, 0, 0, 0, None, 0, s) == -4
    assert g(0, -1, None, None, None, None, None, None, 0, 16, 256, 0, 0, 0, None, 0, s) == 0   # M = 0


def test_i8_ladder():
    """The int8 ladder: every rung plans every legal shape; the automatic
    choice is one of them; grids stay within one launch."""
    names = [qg.i8_rung_name(r) for r in range(qg.i8_num_rungs())]
    assert len(set(names)) == len(names) and qg.i8_rung_name(qg.i8_num_rungs()) is None
    for fmt in ("q4k", "q6k", "w4a16"):
        for M in (1, 31, 64, 130, 658, 2048, 4096):
            for K, N in ((4096, 24576), (12288, 4096), (4096, 1024), (256, 16)):
                sel = qg.i8_select_rung(fmt, M, N, K)
                assert 0 <= sel["rung"] < qg.i8_num_rungs()
                for r in range(qg.i8_num_rungs()):
                    info = qg.i8_rung_info(r, fmt, M, N, K)
                    assert info["tiles_m"] * info["rows"] >= M and info["tiles_n"] * info["cols"] >= N
                    assert info["tiles_m"] * info["tiles_n"] < 2 ** 31
                    assert K // info["k_step"] >= info["k_split"] >= 1, info
    # few 64x64 tiles (up to 96, 128 for Q6_K, and 256 over K >= 8192): those tiles with K also
    # split across workgroups, at any M; measured winners on MI355X (every rung forced, weights
    # rotating): Q4_K/W4A16 4096->1024 at M = 128..256 0.55-0.62 of the 192x64 time, 12288->4096
    # at M = 128 0.60, at M = 256 0.85-0.91
    for fmt, M, N, K, want in [("q4k", 256, 1024, 4096, "i8-64x64-sk"), ("w4a16", 128, 1024, 4096, "i8-64x64-sk"),
                               ("q4k", 128, 4096, 12288, "i8-64x64-sk"), ("w4a16", 256, 4096, 12288, "i8-64x64-sk"),
                               ("q6k", 128, 4096, 4096, "i8-64x64-sk"), ("q6k", 256, 4096, 4096, "i8-192x64-k2"),
                               ("q4k", 256, 4096, 4096, "i8-192x64-k2"), ("q4k", 512, 4096, 12288, "i8-192x64-k2"),
                               ("q6k", 16, 4096, 12288, "i8-64x64-sk"), ("q6k", 256, 4096, 12288, "i8-64x64-sk"),
                               ("q6k", 300, 4096, 12288, "i8-192x64-k2"), ("q4k", 64, 4096, 4096, "i8-64x64-sk"),
                               ("q4k", 96, 4096, 4096, "i8-192x64-k2"), ("q4k", 64, 6144, 4096, "i8-64x64-sk"),
                               ("q4k", 64, 12288, 4096, "i8-192x64-k2"), ("q6k", 658, 4096, 12288, "i8-192x64-k2"),
                               # one round of 768x96 tiles (96-row waves): the merged gate_up at M = 658 (Q4_K
                               # 93.7 against 95.0 us for two rounds of 352x96, Q6_K 104.2 against 117.8) and
                               # M = 1500, N = 12288 (100.1 against 116.8 for 256x96); 512x96 keeps M = 1024-4096
                               ("q4k", 658, 24576, 4096, "i8-768x96"), ("q6k", 658, 24576, 4096, "i8-768x96"),
                               ("q4k", 1500, 12288, 4096, "i8-768x96"), ("q4k", 1024, 12288, 4096, "i8-512x96"),
                               ("q4k", 2048, 12288, 4096, "i8-512x96"), ("q4k", 4096, 12288, 4096, "i8-512x96")]:
        sel = qg.i8_select_rung(fmt, M, N, K)
        assert sel["name"] == want, (fmt, M, N, K, sel)
        if want == "i8-64x64-sk":
            # at least two slices, each a whole number of chunks for each of four K groups
            assert sel["k_split"] >= 8 and (K // 128) % sel["k_split"] == 0, sel


# ----------------------------------------------------------------------------
# the M-ladder
# ----------------------------------------------------------------------------

SHAPES = [(4096, 12288), (4096, 4096), (4096, 1024), (12288, 4096), (4096, 32), (1024, 512), (256, 16)]
# streaming tiles of the round model (one workgroup per CU) and their K groups
ROUND_TILES = {"mfma32-64x64-k4": 4, "mfma32-64x32-k4": 4, "mfma32-96x32-k4": 4, "mfma32-128x64-k2": 2,
               "mfma32-192x64-k2": 2}


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16"])
@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16])
def test_ladder_sweep(fmt, dtype):
    """Sweep M over decode-adjacent to long prefill on every workload shape:
    each rung's grid covers the whole output, the K step is whole 32-wide
    runs (never straddling a Q4_K/Q6_K sub-block or a W4A16 group, whose
    sizes are multiples of 32), and the K split leaves every wave work."""
    for K, N in SHAPES:
        if fmt != "w4a16" and K % 256:
            continue
        for M in list(range(1, 130)) + [255, 256, 257, 511, 512, 658, 1024, 2048, 4096, 8192]:
            info = qg.select_rung(fmt, M, N, K, dtype)
            assert info["rung"] in range(qg.num_rungs())
            assert info["tiles_n"] * info["cols"] >= N
            assert info["tiles_m"] * info["rows"] >= M
            assert info["k_step"] % 32 == 0 and info["k_step"] <= K
            assert (K // info["k_step"]) >= info["k_split"] >= 1
            if N <= 64:
                assert info["name"] == "direct-skinny-n"
            elif M <= 16:
                assert info["name"].startswith("direct-")
            elif M <= 64:
                # the direct kernels up to 24 rows; above, also the split rung and the streaming
                # tiles of the round model
                assert info["name"].startswith("direct-") or (
                    info["name"] in set(ROUND_TILES) | {"mfma32-64x64-sk", "mfma32-128x128-k2"} and M > 24)
            if M > 16 and info["name"] in ROUND_TILES:
                # the round model's K-split tiles run with every K group they were measured with
                assert info["k_split"] == ROUND_TILES[info["name"]], (M, N, K, info)
            if info["name"] == "mfma32-64x64-sk":
                # slices across workgroups: whole chunks for every K group of every slice
                assert (K // info["k_step"]) % info["k_split"] == 0 and info["k_split"] % info["waves"] == 0
            for r in range(qg.num_rungs()):
                ri = qg.rung_info(r, fmt, M, N, K, dtype)
                assert ri["tiles_n"] * ri["cols"] >= N and ri["tiles_m"] * ri["rows"] >= M


def test_ladder_mid_m_round_model():
    """Above 64 rows the ladder first asks the round model: each candidate
    rung's workgroups run in rounds of one per CU (two for the 128-row
    tiles), each round costing what it measured on MI355X for that format
    and activation layout.  The expected names are the measured winners
    (every rung forced, weights rotating); the numbers are Q4_K at K = 4096
    unless stated."""
    xf, row = qg.select_rung_xf, qg.select_rung
    for dt in (qg.F16, qg.BF16):
        for fmt in ("q4k", "q6k", "w4a16"):
            # 64x32 tiles, K split four ways: few panels, 129..512 rows (N = 1024, M = 320: 10.5
            # against 17.1 us for direct-wide; N = 2048, M = 129..256: 10.2-11.2 against 16.3-17.9)
            for M, N in ((320, 1024), (512, 1024), (129, 2048), (256, 2048), (65, 4096), (128, 3072)):
                assert xf(fmt, M, N, 4096, dt)["name"] == "mfma32-64x32-k4", (fmt, dt, M, N)
            # 96x32 tiles: one round of them (N = 4096, M = 129..192: 13.8-14.9 against 17.2-18.8 us;
            # N = 2048, M = 320..384: 14.6-14.8 against 18.3-19.1)
            for M, N in ((129, 4096), (192, 4096), (320, 2048), (384, 2048), (65, 8192), (96, 6144)):
                assert xf(fmt, M, N, 4096, dt)["name"] == "mfma32-96x32-k4", (fmt, dt, M, N)
            # 128x64 tiles, K split two ways: N = 4096, M = 320..512 (22.7-26.0 against 28.0-32.5 us
            # for 192x64); N = 6144..8192, M = 129..256 (21.9-25.8 against 26.8-32.6); N = 12288,
            # M = 65..128 on both layouts (0.58-0.86 of the 192x64 / 64x64 times)
            for M, N in ((320, 4096), (512, 4096), (129, 6144), (256, 8192), (65, 12288), (128, 12288)):
                assert xf(fmt, M, N, 4096, dt)["name"] == "mfma32-128x64-k2", (fmt, dt, M, N)
            assert xf(fmt, 384, 4096, 12288, dt)["name"] == "mfma32-128x64-k2", (fmt, dt)
            for M in (65, 96):
                assert row(fmt, M, 12288, 4096, dt)["name"] == "mfma32-128x64-k2", (fmt, dt, M)
            # one panel and all rows per wave while its workgroups fit one round (N = 1024,
            # M = 129..256: 8.4-9.1 against 10.0-10.5 us for 64x32 tiles)
            for M, N in ((129, 1024), (256, 1024), (96, 2048)):
                assert xf(fmt, M, N, 4096, dt)["name"] == "direct-small-m", (fmt, dt, M, N)
            # 64x64 tiles, K split four ways: one round of them where the narrower tiles need two
            # (N = 4096, M = 256: 19.1 against 20.6 us for 64x32 and 21.8 for 128x64)
            assert xf(fmt, 256, 4096, 4096, dt)["name"] == "mfma32-64x64-k4", (fmt, dt)
            assert xf(fmt, 128, 8192, 4096, dt)["name"] == "mfma32-64x64-k4", (fmt, dt)
            # the large tiles keep their rules (merged QKV and beyond)
            assert xf(fmt, 658, 4096, 4096, dt)["name"] == "mfma32-192x64-k2", (fmt, dt)
            assert row(fmt, 658, 4096, 4096, dt)["name"] == "mfma32-128x128", (fmt, dt)
    # the four-panel direct kernel only for Q4_K (its 48-row variant spills for the other formats):
    # row-major fp16 Q4_K at N = 4096, M = 129..192 (19.5-19.8 against 29.2-29.4 us for 96x32 tiles)
    for M in (129, 192):
        assert row("q4k", M, 4096, 4096)["name"] == "direct-wide", M
        assert row("w4a16", M, 4096, 4096)["name"] != "direct-wide", M
        assert row("q6k", M, 4096, 4096)["name"] != "direct-wide", M
    # Q6_K over few panels, 33..64 rows: row-major takes 16 rows and four panels per wave
    # (M = 40..64: 0.50-0.68 of the time of one panel and all rows per wave), fragment-major
    # splits 64x64 tiles four ways across workgroups (M = 64: 24.2 against 28.1 us);
    # from 65 rows both take 64x32 tiles with K split four ways (M = 96: 36 against 45 us, 56
    # against 81 us on row-major X)
    for M in (33, 64):
        assert qg.select_rung("q6k", M, 4096, 12288)["name"] == "direct-skinny-n", M
        sk = qg.select_rung_xf("q6k", M, 4096, 12288)
        assert sk["name"] == "mfma32-64x64-sk" and sk["k_split"] == 16, (M, sk)
    for M in (65, 80, 128):
        for sel in (qg.select_rung, qg.select_rung_xf):
            assert sel("q6k", M, 4096, 12288)["name"] == "mfma32-64x32-k4", (M, sel.__name__)
    # the split rung never leaves the decode-adjacent range: above 64 rows the round model's
    # tiles beat it on fragment-major activations, and row-major callers get no workspace
    for fmt in ("q4k", "q6k", "w4a16"):
        for M in (65, 96, 128, 200):
            for N, K in ((4096, 12288), (4096, 4096), (2048, 4096), (1024, 4096)):
                for sel in (qg.select_rung, qg.select_rung_xf):
                    assert sel(fmt, M, N, K)["name"] != "mfma32-64x64-sk", (fmt, M, N, K, sel.__name__)
    # up to 16 rows: one panel per wave, except over >= 1536 panels (merged gate/up), where four
    # panels per wave win (M = 8, N = 24576: Q4_K 20.7 against 23.8 us); both layouts
    # (row-major X keeps four panels per wave at 9..16 rows over >= 512 panels: 12.2 against 15.7 us)
    for fmt in ("q4k", "q6k", "w4a16"):
        for sel in (qg.select_rung, qg.select_rung_xf):
            for M in (1, 8, 16):
                assert sel(fmt, M, 24576, 4096)["name"] == "direct-skinny-n", (fmt, M, sel.__name__)
        for M in (1, 8, 16):
            assert qg.select_rung_xf(fmt, M, 12288, 4096)["name"] == "direct-small-m", (fmt, M)
        assert qg.select_rung(fmt, 8, 12288, 4096)["name"] == "direct-small-m", fmt
        assert qg.select_rung(fmt, 16, 12288, 4096)["name"] == "direct-skinny-n", fmt
    # the split rung at the down projection's shape (fragment-major X): fp16 Q6_K and W4A16 33..64
    # rows, Q4_K 49..64; bf16 every format from 33 rows; above 64 rows the 64x32 tiles
    for fmt, M, want in [("q6k", 40, "mfma32-64x64-sk"), ("w4a16", 40, "mfma32-64x64-sk"),
                         ("w4a16", 64, "mfma32-64x64-sk"), ("w4a16", 128, "mfma32-64x32-k4"),
                         ("q4k", 64, "mfma32-64x64-sk"), ("q4k", 96, "mfma32-64x32-k4"), ("q4k", 32, "direct-small-m")]:
        assert qg.select_rung_xf(fmt, M, 4096, 12288)["name"] == want, (fmt, M)
    for fmt, M, want in [("q4k", 96, "mfma32-64x32-k4"), ("q4k", 48, "mfma32-64x64-sk"),
                         ("w4a16", 40, "mfma32-64x64-sk"), ("q4k", 32, "direct-small-m")]:
        assert qg.select_rung_xf(fmt, M, 4096, 12288, qg.BF16)["name"] == want, (fmt, M)
    for dt in (qg.F16, qg.BF16):
        for fmt in ("q4k", "q6k", "w4a16"):
            assert qg.select_rung_xf(fmt, 64, 4096, 4096, dt)["name"] == "direct-small-m", (fmt, dt)
    # Q6_K over many panels, 33..64 rows: 64x64 tiles unpack each weight once for all rows
    # (M = 64, N = K = 12288: 52 against 93 us for direct-skinny-n)
    for M in (33, 48, 64):
        for sel in (qg.select_rung, qg.select_rung_xf):
            assert sel("q6k", M, 12288, 12288)["name"] == "mfma32-64x64-k4", (M, sel.__name__)
            assert sel("q6k", M, 12288, 4096)["name"] == "mfma32-64x64-k4", (M, sel.__name__)


def test_ladder_decode_adjacent_tiles():
    """17..64 rows: the split rung where it pays, else the round model over
    the direct kernels and the streaming tiles.  Pinned here are decisions
    the measurements on MI355X make by at least 8% over every other rung, in
    both dtypes and all three formats (every rung forced, weights rotating,
    K = 4096)."""
    xf, row = qg.select_rung_xf, qg.select_rung
    for dt in (qg.F16, qg.BF16):
        for fmt in ("q4k", "q6k", "w4a16"):
            # few panels: one panel and all rows per wave on fragment-major X; on row-major X
            # 16 rows and four panels per wave from about 50 rows (M = 56..64: 0.57-0.68 of the
            # one-panel time), one panel per wave at 17 rows
            for N in (1024, 2048, 4096):
                for M in (17, 32, 48):
                    assert xf(fmt, M, N, 4096, dt)["name"] == "direct-small-m", (fmt, dt, N, M)
                for M in (56, 64):
                    assert row(fmt, M, N, 4096, dt)["name"] == "direct-skinny-n", (fmt, dt, N, M)
                assert row(fmt, 17, N, 4096, dt)["name"] == "direct-small-m", (fmt, dt, N)
            assert xf(fmt, 36, 3072, 4096, dt)["name"] == "direct-small-m", (fmt, dt)
            assert row(fmt, 60, 3072, 4096, dt)["name"] == "direct-skinny-n", (fmt, dt)
            # 384..512 panels on fragment-major X: 64x32 tiles in one round (N = 6144, M = 40..64:
            # 0.6-0.7 of the time of one panel per wave; N = 8192, M = 36..60)
            for M in (40, 48, 56, 64):
                assert xf(fmt, M, 6144, 4096, dt)["name"] == "mfma32-64x32-k4", (fmt, dt, M)
            for M in (36, 44, 52, 60):
                assert xf(fmt, M, 8192, 4096, dt)["name"] == "mfma32-64x32-k4", (fmt, dt, M)
            # 768 panels up to 32 rows: four panels and all rows per wave (both layouts); row-major
            # X at N = 6144, 32 rows: 16 rows and four panels per wave
            for M in (17, 24, 32):
                assert row(fmt, M, 12288, 4096, dt)["name"] == "direct-wide", (fmt, dt, M)
            assert row(fmt, 32, 6144, 4096, dt)["name"] == "direct-skinny-n", (fmt, dt)
            # 896 panels (N = 14336): four panels per wave at 20..28 rows, one round of 64x64 tiles
            # at 60 rows on fragment-major X
            for M in (20, 28):
                for sel in (xf, row):
                    assert sel(fmt, M, 14336, 4096, dt)["name"] == "direct-wide", (fmt, dt, M)
            assert xf(fmt, 60, 14336, 4096, dt)["name"] == "mfma32-64x64-k4", (fmt, dt)


def test_ladder_fragment_major():
    """The ladder for fragment-major activations above 64 rows: where the
    round model defers to the large tiles, the large tile whose whole rounds
    cost least by the full-round cost table (the 192-row K-split tiles, the
    K-split 128x128, 256x128, 352x96, 128x128, 128x160 and the 8-wave
    512x96, 512x128 and 768x96 tiles).  The pins are measured winners on
    MI355X (every large tile forced, weights rotating) by at least 10% over
    the next tile, plus the dense layer's four GEMMs at M = 658; row-major
    activations keep their rule chain."""
    XF_WINNERS = [
        # (fmt, M, N, K, rung): fp16 unless noted; the margin over the next tile
        ("q4k", 658, 4096, 4096, "mfma32-192x64-k2"),    # o (bf16: 31.8 against 36.9 us)
        ("q6k", 658, 4096, 12288, "mfma32-768x64-sk"),   # down: four slices, 92.0 against 101.4 (192x64-k2)
        ("q4k", 658, 6144, 4096, "mfma32-192x96-k2"),    # qkv: 44.6 against 59.1 us (128x160)
        ("q6k", 700, 6144, 4096, "mfma32-192x96-k2"),    # 47.5 against 64.5 (352x96)
        ("q4k", 384, 12288, 4096, "mfma32-192x96-k2"),   # 46.2 against 59.6 (128x160)
        ("w4a16", 300, 11008, 4096, "mfma32-192x96-k2"),  # 39.1 against 53.0
        ("q4k", 384, 6144, 4096, "mfma32-192x64-k2"),    # 30.1 against 34.0
        ("q4k", 658, 12288, 4096, "mfma32-352x96"),      # 75.5 against 87.3 (192x96-k2)
        ("q6k", 640, 12288, 4096, "mfma32-352x96"),      # 79.7 against 87.9 (128x128; the rule chain took 256x128, 123.7)
        ("q4k", 768, 24576, 4096, "mfma32-768x96"),      # 145.8 against 175.2 (192x96-k2)
        ("q4k", 1500, 12288, 4096, "mfma32-768x96"),     # 144.9 against 175.2
        ("q6k", 3072, 6144, 4096, "mfma32-768x96"),      # 151.9 against 186.2 (512x96)
        ("q4k", 3072, 4096, 4096, "mfma32-512x128"),     # 103.9 against 119.1 (128x128)
        ("q6k", 900, 14336, 4096, "mfma32-512x128"),     # 110.7 against 135.0
        ("w4a16", 2500, 5120, 5120, "mfma32-512x128"),   # 122.5 against 143.7 (256x128)
        ("q4k", 2048, 4096, 4096, "mfma16-256x128"),     # 68.5 against 83.5
        ("q4k", 512, 12288, 4096, "mfma16-256x128"),     # 60.5 against 72.1 (352x96)
        ("q6k", 450, 14336, 4096, "mfma16-256x128"),     # 66.9 against 83.1
        ("q4k", 1024, 4096, 12288, "mfma32-128x128-k2"),  # bf16: 113.4 against 125.4
    ]
    for fmt, M, N, K, rung in XF_WINNERS:
        assert qg.select_rung_xf(fmt, M, N, K)["name"] == rung, (fmt, M, N, K)
    # the merged gate_up at M = 658: one round of 768x96 tiles (140.8 against 147.1 us for 352x96)
    for fmt in ("q4k", "q6k", "w4a16"):
        assert qg.select_rung_xf(fmt, 658, 24576, 4096)["name"] == "mfma32-768x96", fmt
    assert qg.select_rung("q4k", 658, 24576, 4096)["name"] == "mfma32-128x160"         # row-major
    assert qg.select_rung("q4k", 658, 4096, 4096)["name"] == "mfma32-128x128"          # row-major: K < 8192
    # the 768x64 tiles split across workgroups: 513..768 rows of Q4_K or Q6_K over K >= 12288 when the
    # 64-column tiles times 2, 4 or 8 slices make one round (measured winners: Q6_K 520, 658 and 768 rows
    # over N = 4096, 600 rows over N = 8192, K = 16384; Q4_K over N = 2048 and 4096), with the slices
    # in the plan and the partial sums in the workspace query
    for fmt, M, N, K, S in [("q6k", 520, 4096, 12288, 4), ("q6k", 768, 4096, 12288, 4), ("q6k", 600, 8192, 12288, 2),
                            ("q6k", 658, 4096, 16384, 4), ("q4k", 658, 4096, 12288, 4), ("q4k", 658, 2048, 12288, 8)]:
        info = qg.select_rung_xf(fmt, M, N, K)
        assert (info["name"], info["k_split"], info["rows"], info["cols"]) == ("mfma32-768x64-sk", S, 768, 64), (fmt, M, N, K)
        assert qg.workspace_bytes(fmt, -1, M, N, K, qg.F16, qg.X_FRAG) == S * ((M * N + 3) // 4 * 4) * 4
    # not at K = 8192 (Q4_K, 700 rows: 68.0 against 64.2 us), at 400 rows (80.8 against 71.9), for W4A16,
    # over N = 6144 (no whole round), on row-major activations or past 768 rows
    for fmt, M, N, K in [("q4k", 700, 4096, 8192), ("q6k", 400, 4096, 12288), ("w4a16", 658, 4096, 12288),
                         ("q6k", 658, 6144, 12288), ("q6k", 800, 4096, 12288)]:
        assert qg.select_rung_xf(fmt, M, N, K)["name"] != "mfma32-768x64-sk", (fmt, M, N, K)
    assert qg.select_rung("q6k", 658, 4096, 12288)["name"] != "mfma32-768x64-sk"
    # one round of 128x64 tiles (the round model, before the large tiles)
    assert qg.select_rung_xf("q4k", 512, 4096, 4096)["name"] == "mfma32-128x64-k2"
    # a K-split tile with an odd chunk count (W4A16, K = 33 x 128) runs one K group: not a candidate
    assert qg.select_rung_xf("w4a16", 658, 4096, 4224)["name"] not in ("mfma32-192x64-k2", "mfma32-128x128-k2",
                                                                      "mfma32-192x96-k2")
    # row-major Q6_K (no 160-wide tile): the 352x96 tile at M = 700 over N = 11008..24576 (0.78-0.92
    # of the 128x128 time) and the 256-row tile from 512 of its tiles (M = 3072, N = 11008..12288:
    # 0.90 of it); not at 1.5 rounds (M = 1024, N = 12288) nor for the other formats
    for N in (11008, 12288, 24576):
        assert qg.select_rung("q6k", 700, N, 4096)["name"] == "mfma32-352x96", N
    for N in (11008, 12288):
        assert qg.select_rung("q6k", 3072, N, 4096)["name"] == "mfma16-256x128", N
    assert qg.select_rung("q6k", 1024, 12288, 4096)["name"] == "mfma32-128x128"
    for fmt in ("q4k", "w4a16"):
        assert qg.select_rung(fmt, 700, 12288, 4096)["name"] == "mfma32-128x160", fmt
    # (at 9..16 rows over 512..1535 panels the layouts differ on purpose: see the small-M test)
    for fmt, M, K, N in [("q4k", 8, 4096, 12288), ("w4a16", 2048, 4096, 12288), ("q4k", 4096, 4096, 32)]:
        assert qg.select_rung_xf(fmt, M, N, K)["name"] == qg.select_rung(fmt, M, N, K)["name"], (fmt, M, K, N)
    for K, N in SHAPES:
        for M in list(range(1, 70)) + [96, 200, 300, 511, 658, 1000, 1024, 4096]:
            info = qg.select_rung_xf("w4a16", M, N, K)
            assert info["tiles_n"] * info["cols"] >= N and info["tiles_m"] * info["rows"] >= M


def test_grid_limits():
    """Direct rungs put row groups of 16 on grid.y (at most 65535): forcing
    one past that is a shape error before any launch, and the ladder moves
    such shapes to a streaming rung (one-dimensional grid)."""
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    big = 65535 * 64 + 1  # past the limit of every direct rung (up to 64 rows per group)
    for rung in range(3):  # the three direct rungs
        assert lib.qgemm_gemm_rung(0, rung, A, A, A, big, 32, 256, 0, 0, 0, None, 0, None) == -2
        assert lib.qgemm_gemm_xf(0, rung, A, A, A, big, 32, 256, 0, 0, 0, None, 0, None) == -2
        with pytest.raises(qg.QGemmError) as e:
            qg.rung_info(rung, "q4k", big, 32, 256)
        assert e.value.status == -2
    assert qg.rung_info(1, "q4k", 65535 * 16, 32, 256)["tiles_m"] == 65535
    for M in (65535 * 16 + 1, big, 1 << 24):
        info = qg.select_rung("q4k", M, 32, 256)
        assert info["name"].startswith("mfma32-") and info["tiles_m"] * info["rows"] >= M
        assert not qg.select_rung_xf("q4k", M, 32, 256)["name"].startswith("direct-")


def test_ladder_rejects_bad_shapes():
    with pytest.raises(qg.QGemmError):
        qg.select_rung("q4k", 16, 512, 1000)
    with pytest.raises(qg.QGemmError):
        qg.select_rung("q4k", 16, 512, 1024, dtype=9)
    assert qg.rung_name(-1) is None and qg.rung_name(qg.num_rungs()) is None


@pytest.mark.parametrize("fmt,sym", [("q4k", False), ("q6k", False), ("w4a16", False), ("w4a16", True)])
def test_concat_encoded_columns(fmt, sym):
    """Weights concatenated along N dequantize to the members' own weights
    side by side, and pack to the same bytes as packing them jointly."""
    import oracle

    K, Ns = 512, (48, 16, 32)
    fields = [synth.weight_fields(fmt, np.random.default_rng(60 + i), n, K, 128, sym) for i, n in enumerate(Ns)]
    encs = [synth.encode(fmt, f) for f in fields]
    merged = synth.concat_encoded(fmt, encs)
    W = oracle.dequant(fmt, merged, sum(Ns), K, qg.F16)
    edges = np.cumsum((0,) + Ns)
    for i, e in enumerate(encs):
        assert np.array_equal(W[:, edges[i]:edges[i + 1]], oracle.dequant(fmt, e, Ns[i], K, qg.F16))
    packed = qg.pack(fmt, merged, sum(Ns), K)
    if fmt != "w4a16":  # k-quant panels are whole records: joint packing is the concatenation
        assert np.array_equal(packed, np.concatenate([qg.pack(fmt, e, n, K) for e, n in zip(encs, Ns)]))


def test_step_gemms_merge():
    sg = synth.step_gemms("qwen3_8b_layer_m658")
    assert [(g["label"], g["N"]) for g in sg] == [("qkv", 6144), ("o", 4096), ("gate_up", 24576), ("down", 4096)]
    assert [g["label"] for g in synth.step_gemms("qwen3_8b_layer_m658", merge=False)] == \
        ["q", "k", "v", "o", "gate", "up", "down"]
    flops = lambda gs: sum(2 * g["M"] * g["N"] * g["K"] for g in gs)
    assert flops(sg) == flops(synth.step_gemms("qwen3_8b_layer_m658", merge=False))


def test_grouped_plan():
    """The grouped plan: the direct kernel up to 16 rows per expert on average
    and where the grid needs a K split, else the shared-activation kernel with
    32-row tiles up to 48 rows per expert and 80-row tiles above (the measured
    winners on MI355X on the 128-expert routing of a 658-token prompt, its
    counts scaled); row-tile slots bound every expert's tiles."""
    E = 128
    for T, N, K, name, rows in [
        (1316, 768, 2048, "direct", 16),    # 10 rows per expert
        (3688, 768, 2048, "shared", 32),    # 29
        (5264, 768, 2048, "shared", 32),    # 41: the MoE gate and up GEMMs
        (5264, 2048, 768, "shared", 32),    # 41: the MoE down GEMM
        (6144, 768, 2048, "shared", 32),    # 48
        (6145, 768, 2048, "shared", 80),    # 49
        (36848, 2048, 768, "shared", 80),   # 288
    ]:
        p = qg.grouped_plan(T, E, N, K)
        assert (p["name"], p["rows"]) == (name, rows), (T, N, K, p)
        assert p["grid_y"] == -(-T // rows) + E
        if name == "shared":
            assert (p["cols"], p["waves"], p["kw"], p["grid_x"]) == (128, 4, 1, -(-N // 128))
        else:
            assert (p["cols"], p["grid_x"]) == (64, -(-N // 64)) and p["waves"] == p["kw"]
    # a small grid splits K in the direct kernel; at two or three chunks no
    # split is possible and the shared kernel serves it
    p = qg.grouped_plan(341, 5, 144, 2048)
    assert p["name"] == "direct" and p["kw"] == 8 and p["rows"] == 32
    for K in (256, 384):
        p = qg.grouped_plan(341, 5, 144, K)
        assert (p["name"], p["rows"], p["grid_x"], p["grid_y"]) == ("shared", 80, 2, 5 + 5)
    assert qg.grouped_plan(0, 4, 64, 256)["name"] == "direct"
    lib = qg.lib()
    info = np.zeros(8, np.int32)
    ptr = info.ctypes.data_as(ctypes.c_void_p)
    assert lib.qgemm_grouped_plan(64, 4, 64, 256, None) == -1
    for bad in [(-1, 4, 64, 256), (64, 0, 64, 256), (64, 4, 0, 256), (64, 4, 64, 100), (64, 4, 64, 0),
                (1 << 20, 4, 64, 256)]:
        assert lib.qgemm_grouped_plan(*bad, ptr) == -2, bad


def test_grouped_offset_clamping_prefix_max_form():
    """The grouped kernels find an expert's rows from prefix maxima,
    lo_e = min(T, max(0, offs[0..e])) and hi_e = min(T, max(0, offs[0..e+1])),
    instead of clamping the offsets one after another (each into [0, T] and to
    at least the previous end).  The two forms agree on arbitrary offsets,
    negative, decreasing and past T included."""
    def serial(offs, T):
        out, hi = [], 0
        for e in range(len(offs) - 1):
            lo = min(max(int(offs[e]), hi), T)
            hi = min(max(int(offs[e + 1]), lo), T)
            out.append((lo, hi))
        return out

    rng = np.random.default_rng(17)
    for _ in range(5000):
        E, T = int(rng.integers(1, 12)), int(rng.integers(0, 300))
        offs = rng.integers(-50, 400, E + 1)
        q = np.maximum.accumulate(np.concatenate([[0], offs]))[1:]
        assert [(min(int(q[e]), T), min(int(q[e + 1]), T)) for e in range(E)] == serial(offs, T), (offs, T)


def test_grid_work_item_limit():
    """A launch holds at most 2^31-1 workgroups and 2^32-1 work-items along x:
    shapes whose grid would exceed that are shape errors before any launch,
    not failed launches."""
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    # 128x128 tiles of 256 threads: 2^24 tiles is 2^32 work-items, one too many
    n_tiles = 1 << 24
    N = 128 * n_tiles
    with pytest.raises(qg.QGemmError) as e:
        qg.rung_info(4, "q4k", 128, N, 256)  # mfma32-128x128
    assert e.value.status == -2
    assert lib.qgemm_gemm_rung(0, 4, A, A, A, 128, N, 256, 0, 0, 0, None, 0, None) == -2
    info = qg.rung_info(4, "q4k", 128, N - 128, 256)  # 2^24 - 1 tiles fit
    assert info["tiles_n"] == n_tiles - 1
    # the direct rungs: 64 threads per wave, the waves splitting K (one wave
    # at K = 256); 2^26 panels of 16 columns is 2^32 work-items
    with pytest.raises(qg.QGemmError):
        qg.rung_info(0, "q4k", 16, 16 * (1 << 26), 256)
    assert qg.rung_info(0, "q4k", 16, 16 * ((1 << 26) - 1), 256)["tiles_n"] == (1 << 26) - 1
    # the fragment-major copy: one 256-thread workgroup per (32 rows, 128 k)
    assert lib.qgemm_x_to_xf(A, A, 32 * (1 << 13), 128 * (1 << 11), None) == -2
    # the dequant: one thread per (panel, chunk, run)
    assert lib.qgemm_dequant(0, A, A, 16 * (1 << 21), 256 * (1 << 10), 0, 0, 0, None) == -2


def test_workspace_contract():
    """The library allocates nothing: the split rungs take the caller's
    workspace and report its size; a call without enough of it fails before
    any launch; the other rungs need none.  The row-major ladder (the format
    entry points) never picks a rung that needs one."""
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    sk = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-64x64-sk"][0]
    M, N, K = 64, 4096, 12288
    info = qg.rung_info(sk, "q6k", M, N, K)
    S = info["k_split"] // 4  # four K groups inside each workgroup
    need = qg.workspace_bytes("q6k", sk, M, N, K)
    assert S >= 2 and need == S * M * N * 4
    assert qg.workspace_bytes("q6k", sk, M, N, K, layout=qg.X_FRAG) == need
    assert qg.workspace_bytes("q6k", sk, 0, N, K) == 0
    assert qg.workspace_bytes("q6k", 4, M, N, K) == 0                 # a rung with no split
    assert lib.qgemm_workspace_bytes(1, sk, 7, M, N, K, 0) == 0       # unknown layout
    # the fragment-major ladder picks the split rung for the down projection at M = 64
    assert qg.select_rung_xf("q6k", M, N, K)["name"] == "mfma32-64x64-sk"
    assert qg.workspace_bytes("q6k", -1, M, N, K, layout=qg.X_FRAG) == need
    for call in (lib.qgemm_gemm_rung, lib.qgemm_gemm_xf):
        assert call(1, sk, A, A, A, M, N, K, 0, 0, 0, None, 0, None) == -6
        assert call(1, sk, A, A, A, M, N, K, 0, 0, 0, A, need - 16, None) == -6
        assert call(1, sk, A, A, A, M, N, K, 0, 0, 0, mis, need, None) == -4
    assert lib.qgemm_gemm_xf(1, -1, A, A, A, M, N, K, 0, 0, 0, None, 0, None) == -6
    # odd M*N: each slice starts 16-byte aligned
    assert qg.workspace_bytes("q6k", sk, 33, 4094, K) == S * ((33 * 4094 + 3) // 4 * 4) * 4
    # the int8 path's split rung
    i8sk = [r for r in range(qg.i8_num_rungs()) if qg.i8_rung_name(r) == "i8-64x64-sk"][0]
    need8 = qg.i8_workspace_bytes("q6k", i8sk, M, N, K)
    assert need8 > 0 and need8 % (M * N * 4) == 0
    assert qg.i8_workspace_bytes("q6k", -1, 16, N, K) > 0             # the int8 ladder's pick
    assert lib.qgemm_i8_gemm(1, i8sk, A, A, A, A, A, A, M, N, K, 0, 0, 0, None, 0, None) == -6
    assert lib.qgemm_i8_gemm(1, i8sk, A, A, A, A, A, A, M, N, K, 0, 0, 0, A, need8 - 4, None) == -6
    # the row-major ladder never needs a workspace
    for fmt in ("q4k", "q6k", "w4a16"):
        for dt in (qg.F16, qg.BF16):
            for M in (1, 8, 16, 24, 33, 48, 49, 64, 80, 96, 128, 130, 200, 256, 658, 2048):
                for K, N in ((4096, 4096), (12288, 4096), (4096, 2048), (4096, 3072), (4096, 12288), (8192, 4096)):
                    assert qg.workspace_bytes(fmt, -1, M, N, K, dt, qg.X_ROW) == 0, (fmt, dt, M, N, K)


# every declaration in include/qgemm.h carries a citation of the pages (a
# page's short name from the header's preamble and the section it follows)
PAGE_NAMES = ("batched-prefill post", "W4A16 PR", "delta-net page", "dequant-scratch post", "sparkinfer PR")


def _declaration_comments(path):
    """(function name, the comment block that precedes its declaration group)."""
    text = open(path).read()
    out = []
    last_comment = ""
    pos = 0
    for m in re.finditer(r"/\*.*?\*/|^[a-z_ ]+\**\s*\b(q[a-z0-9_]+)\s*\(", text, flags=re.S | re.M):
        if m.group(0).startswith("/*"):
            last_comment = m.group(0)
        else:
            out.append((m.group(1), last_comment))
    return out


def test_header_declarations_cite_the_pages():
    decls = _declaration_comments(HEADER)
    assert len(decls) == len(header_functions())
    for name, comment in decls:
        flat = " ".join(re.sub(r"\n\s*\*(?!/)", " ", comment).split())  # comment lines joined, their '*' dropped
        if name == "qgemm_gemm_xf_noalloc":  # names the callers it is for instead
            assert "cannot allocate" in flat
            continue
        assert any(p in flat for p in PAGE_NAMES), f"{name}: its comment cites no page"
        assert re.search(r'"[^"]{3,}"', flat), f"{name}: its comment names no section of the page it cites"


def test_binding_checks_buffers_before_any_call():
    """The Python binding refuses a packed weight smaller than the format's
    packed size (times the experts for the grouped GEMM) and an output of the
    wrong shape or dtype before it calls the library, on every device entry
    point; the W4A16 zero-point flag defaults to symmetric everywhere."""
    import inspect

    import torch

    M, N, K = 8, 48, 512
    x = torch.zeros((M, K), dtype=torch.float16)
    full = qg.packed_bytes("q4k", N, K)
    short = torch.zeros(full - 16, dtype=torch.uint8)
    ok = torch.zeros(full, dtype=torch.uint8)
    offs = torch.zeros(3, dtype=torch.int32)
    xf = torch.zeros(qg.xf_bytes(M, K) // 2, dtype=torch.float16)
    for call in (lambda: qg.q4k(x, short, N), lambda: qg.gemm_rung("q4k", -1, x, short, N),
                 lambda: qg.staged("q4k", x, short, N), lambda: qg.grouped("q4k", x, ok, N, offs, 2),
                 lambda: qg.grouped_xf("q4k", xf, ok, M, N, K, offs, 2),
                 lambda: qg.dequant("q4k", short, N, K, qg.F16)):
        with pytest.raises(ValueError, match="packed weight"):
            call()
    with pytest.raises(ValueError, match="fragment-major"):
        qg.grouped_xf("q4k", xf[:-8], torch.zeros(2 * full, dtype=torch.uint8), M, N, K, offs, 2)
    w4_sym = qg.packed_bytes("w4a16", N, K, 128, False)
    assert w4_sym < qg.packed_bytes("w4a16", N, K, 128, True)
    with pytest.raises(ValueError, match="packed weight"):  # an asymmetric call on a symmetric packing
        qg.w4a16(x, torch.zeros(w4_sym, dtype=torch.uint8), N, 128, True)
    bad_out = torch.zeros((M, N + 1), dtype=torch.float16)
    bad_dt = torch.zeros((M, N), dtype=torch.bfloat16)
    two = torch.zeros(2 * full, dtype=torch.uint8)
    for out in (bad_out, bad_dt):
        for call in (lambda: qg.grouped("q4k", x, two, N, offs, 2, out=out), lambda: qg.staged("q4k", x, ok, N, out=out),
                     lambda: qg.grouped_xf("q4k", xf, two, M, N, K, offs, 2, out=out),
                     lambda: qg.gemm_rung("q4k", -1, x, ok, N, out=out), lambda: qg.q6k(x, torch.zeros(
                         qg.packed_bytes("q6k", N, K), dtype=torch.uint8), N, out=out)):
            with pytest.raises(ValueError, match="out"):
                call()
    for fn in (qg.grouped, qg.grouped_xf, qg.staged, qg.gemm_rung, qg.gemm_xf, qg.gemm_i8, qg.dequant, qg.i8_colscale):
        assert inspect.signature(fn).parameters["has_zp"].default is False, fn.__name__


def test_library_sources_allocate_nothing():
    """No device or host allocation in the library's sources: every buffer
    is the caller's, or the fixed device array of the no-alloc entry point."""
    base = os.path.join(ROOT, "quantized_weight_prefill_amd", "csrc")
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipExtMallocWithFlags|malloc|calloc|realloc|"
                        r"operator new|std::vector|std::mutex|new\s+\w)")
    for dirpath, _, files in os.walk(base):
        for f in files:
            text = open(os.path.join(dirpath, f)).read()
            code = re.sub(r"//[^\n]*|/\*.*?\*/", "", text, flags=re.S)
            hits = banned.findall(code)
            if f == "pack.cpp":
                hits = [h for h in hits if h != "std::vector"]  # host packers, host memory only
            assert not hits, f"{f}: {sorted(set(hits))}"


def test_noalloc_entry_rejects_oversized_calls_before_launch():
    lib = qg.lib()
    A = ctypes.c_void_p(1 << 20)  # never dereferenced
    sk = [r for r in range(qg.num_rungs()) if qg.rung_name(r) == "mfma32-64x64-sk"][0]
    M, N, K = 2048, 4096, 12288   # one slice of 2048 x 4096 fp32 partial sums: 32 MiB
    assert qg.workspace_bytes("q6k", sk, M, N, K, layout=qg.X_FRAG) > qg.NOALLOC_SCRATCH_BYTES
    assert lib.qgemm_gemm_xf_noalloc(1, sk, A, A, A, M, N, K, 0, 0, 0, None) == -6
    assert lib.qgemm_gemm_xf_noalloc(1, sk, A, A, ctypes.c_void_p((1 << 20) + 8), M, N, K, 0, 0, 0, None) == -4
    assert lib.qgemm_gemm_xf_noalloc(1, 99, A, A, A, 64, N, K, 0, 0, 0, None) == -5
    assert lib.qgemm_gemm_xf_noalloc(1, -1, None, A, A, 64, N, K, 0, 0, 0, None) == -1
    assert lib.qgemm_gemm_xf_noalloc(1, -1, None, None, None, 0, N, K, 0, 0, 0, None) == 0


def test_moe_step_gemms_merge():
    """The MoE step runs gate and up as one grouped GEMM: expert e of the
    merged weights is expert e's gate columns, then its up columns, and the
    merged GEMM reads the routed rows both members read."""
    name = "moe_e128_top8_m658"
    merged = synth.moe_step_gemms(name)
    assert [(g["label"], g["N"], g["members"]) for g in merged] == [("gate_up", 1536, [0, 1]), ("down", 2048, [2])]
    assert [g["label"] for g in synth.moe_step_gemms(name, merge=False)] == ["gate", "up", "down"]
    X, enc = synth.moe_step_inputs(name, [0, 1])
    Xg, _, eg = synth.moe_inputs(name, 0)
    _, _, eu = synth.moe_inputs(name, 1)
    assert np.array_equal(X, Xg)
    N = 768
    for e in (0, 63, 127):
        assert np.array_equal(enc[2 * N * e:2 * N * e + N], eg[N * e:N * (e + 1)])
        assert np.array_equal(enc[2 * N * e + N:2 * N * (e + 1)], eu[N * e:N * (e + 1)])
