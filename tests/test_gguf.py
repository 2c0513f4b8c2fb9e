"""The GGUF reader (no GPU): a Q4_K_M-style file written by the test (Q4_K
projections, Q6_K ffn_down and attn_v, f32 norms) is read back -- header,
metadata, tensor infos, alignment -- and its k-quant tensors pack to the
same bytes as packing the original blocks; other tensor types are refused;
malformed and truncated files are errors, never reads past the buffer.
Interop with real GGUF files is parity unpinned: no such file is available
here, so writer and reader both follow the published layout."""
from __future__ import annotations

import struct

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests import gguf_writer as gw

F32_T = 0


def _model(alignment=32, K=512, N=256, Nv=32):
    rng = np.random.default_rng(77)
    f_up = synth.q4k_fields(rng, N, K)
    f_q = synth.q4k_fields(rng, K, K)
    f_down = synth.q6k_fields(rng, K, N)  # down: K_in = N (multiple of 256 below), N_out = K
    f_v = synth.q6k_fields(rng, Nv, K)
    blocks = {
        "blk.0.attn_q.weight": (qg.GGML_Q4_K, (K, K), synth.q4k_encode(f_q)),
        "blk.0.attn_v.weight": (qg.GGML_Q6_K, (K, Nv), synth.q6k_encode(f_v)),
        "blk.0.ffn_up.weight": (qg.GGML_Q4_K, (K, N), synth.q4k_encode(f_up)),
        "blk.0.ffn_down.weight": (qg.GGML_Q6_K, (N, K), synth.q6k_encode(f_down)),
    }
    norm = np.linspace(0.5, 1.5, K, dtype=np.float32)
    tensors = [("blk.0.attn_norm.weight", F32_T, (K,), norm.tobytes())]
    tensors += [(name, t, dims, b.tobytes()) for name, (t, dims, b) in blocks.items()]
    kv = [("general.architecture", gw.STRING, "qwen3"), ("general.name", gw.STRING, "synthetic"),
          ("general.file_type", gw.U32, 15), ("qwen3.block_count", gw.U32, 1),
          ("qwen3.rope.freq_base", gw.F32, 1000000.0),
          ("tokenizer.ggml.tokens", gw.ARRAY, (gw.STRING, ["<a>", "b", "c"])),
          ("qwen3.layer_sizes", gw.ARRAY, (gw.U32, [1, 2, 3]))]
    return gw.as_array(gw.write(kv, tensors, alignment)), blocks, norm


@pytest.mark.parametrize("alignment", [32, 64, 256])
def test_gguf_roundtrip_q4k_m_mix(alignment):
    buf, blocks, norm = _model(alignment)
    h = qg.gguf_header(buf)
    assert h["version"] == 3 and h["n_tensors"] == 5 and h["n_kv"] == 7 + (alignment != 32)
    assert h["alignment"] == alignment and h["data_offset"] % alignment == 0
    infos = {t["name"]: t for t in qg.gguf_tensors(buf)}
    assert list(infos) == ["blk.0.attn_norm.weight"] + list(blocks)
    n = infos["blk.0.attn_norm.weight"]
    assert n["type"] == F32_T and n["dims"] == (512,) and n["nbytes"] == 2048 and n["offset"] % alignment == 0
    assert np.array_equal(buf[n["offset"]:n["offset"] + 2048].view(np.float32), norm)
    for name, (t, dims, b) in blocks.items():
        info = infos[name]
        assert info["type"] == t and info["dims"] == dims and info["nbytes"] == b.nbytes
        assert info["offset"] % alignment == 0
        assert np.array_equal(buf[info["offset"]:info["offset"] + b.nbytes], b.reshape(-1))
        fmt, N, K, packed = qg.gguf_pack(buf, info["index"])
        assert (fmt, K, N) == ("q4k" if t == qg.GGML_Q4_K else "q6k", dims[0], dims[1])
        assert np.array_equal(packed, qg.pack(fmt, b, N, K))
        # the packed weights unpack (oracle) to what the file's blocks hold
        assert np.array_equal(oracle.dequant(fmt, qg.q4k_unpack(packed, N, K) if fmt == "q4k" else
                                             qg.q6k_unpack(packed, N, K), N, K, qg.F16),
                              oracle.dequant(fmt, b, N, K, qg.F16))
    with pytest.raises(qg.QGemmError) as e:  # an f32 tensor is not a k-quant weight: no conversion
        qg.gguf_pack(buf, infos["blk.0.attn_norm.weight"]["index"])
    assert e.value.status == -5


def test_gguf_metadata():
    buf, _, _ = _model()
    assert qg.gguf_kv(buf, "general.architecture") == "qwen3"
    assert qg.gguf_kv(buf, "general.file_type") == 15
    assert qg.gguf_kv(buf, "qwen3.rope.freq_base") == 1000000.0
    assert qg.gguf_kv(buf, "tokenizer.ggml.tokens") == ["<a>", "b", "c"]
    assert qg.gguf_kv(buf, "qwen3.layer_sizes") == [1, 2, 3]
    assert qg.gguf_kv(buf, "no.such.key") is None


def test_gguf_file_on_disk(tmp_path):
    buf, blocks, _ = _model(64)
    path = tmp_path / "m.gguf"
    path.write_bytes(buf.tobytes())
    mm = qg.gguf_map(str(path))
    assert qg.gguf_header(mm)["alignment"] == 64
    fmt, N, K, packed = qg.gguf_pack(mm, 3)
    assert np.array_equal(packed, qg.pack("q4k", blocks["blk.0.ffn_up.weight"][2], N, K))


def _status(buf):
    lib = qg.lib()
    b = np.ascontiguousarray(buf, dtype=np.uint8)
    import ctypes
    p = ctypes.c_void_p(b.ctypes.data) if b.nbytes else ctypes.c_void_p(1 << 20)
    st = lib.qgemm_gguf_header(p, b.nbytes, None, None, None, None, None)
    if st != 0:
        return st
    nt = qg.gguf_header(b)["n_tensors"]
    worst = 0
    for i in range(nt):
        s = lib.qgemm_gguf_tensor_info(p, b.nbytes, i, None, 0, None, None, None, None, None)
        worst = min(worst, s)
        out = np.empty(1 << 20, np.uint8)
        s2 = lib.qgemm_gguf_pack(p, b.nbytes, i, ctypes.c_void_p(out.ctypes.data), out.nbytes, None, None, None)
        worst = min(worst, s2 if s2 not in (-5, -6) else 0)
    return worst


def test_gguf_truncated_and_malformed_files():
    buf, _, _ = _model()
    good = _status(buf)
    assert good == 0
    # every truncation point in the header and tensor-info region, and a sample of the data region
    h = qg.gguf_header(buf)
    cuts = list(range(0, h["data_offset"] + 1)) + list(range(h["data_offset"], buf.nbytes, 997))
    for cut in cuts:
        assert _status(buf[:cut]) < 0, cut
    bad = buf.copy(); bad[0] ^= 1
    assert _status(bad) == -8  # magic
    bad = buf.copy(); bad[4:8] = np.frombuffer(struct.pack("<I", 1), np.uint8)
    assert _status(bad) == -8  # version 1
    bad = buf.copy(); bad[8:16] = np.frombuffer(struct.pack("<Q", 1 << 62), np.uint8)
    assert _status(bad) == -8  # absurd tensor count
    bad = buf.copy(); bad[24:32] = np.frombuffer(struct.pack("<Q", 1 << 60), np.uint8)
    assert _status(bad) == -8  # first key's length past the end


def _one_tensor(dims, t=qg.GGML_Q4_K, data=b"", offset=None, n_dims=None):
    """A file with one tensor; its info fields can be set to bad values."""
    raw = bytearray(gw.write([], [("w", t, dims, data)]))
    # locate the tensor info: after the 24-byte header, name (8 + 1 bytes)
    pos = 24 + 8 + 1
    if n_dims is not None:
        raw[pos:pos + 4] = struct.pack("<I", n_dims)
    if offset is not None:
        p_off = pos + 4 + 8 * len(dims) + 4
        raw[p_off:p_off + 8] = struct.pack("<Q", offset)
    return gw.as_array(bytes(raw))


def test_gguf_bad_tensor_infos():
    blk = synth.q4k_encode(synth.q4k_fields(np.random.default_rng(3), 16, 256)).tobytes()
    assert _status(_one_tensor((256, 16), data=blk)) == 0
    assert _status(_one_tensor((256, 16), data=blk, offset=8)) == -8         # misaligned
    assert _status(_one_tensor((256, 16), data=blk, offset=1 << 40)) == -8   # past the end
    assert _status(_one_tensor((256, 16), data=blk[:-1])) == -8              # data cut short
    assert _status(_one_tensor((300, 16), data=blk)) == -8                   # rows not whole blocks
    assert _status(_one_tensor((256, 16), data=blk, n_dims=0)) == -8
    assert _status(_one_tensor((256, 16), data=blk, n_dims=5)) == -8
    assert _status(_one_tensor((1 << 40, 1 << 40), data=blk)) == -8          # size overflows
    fmt, N, K, packed = qg.gguf_pack(_one_tensor((256, 16), data=blk), 0)
    assert (fmt, N, K) == ("q4k", 16, 256)
