"""Weights read from a GGUF file (written by the test in the Q4_K_M mix:
Q4_K up projection, Q6_K down projection) through the reader and packers
into the fused GEMMs, against the oracle's unpack of the same file bytes."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_weight_prefill_amd as qg
from quantized_weight_prefill_amd import synth
from tests.helpers import assert_gemm_close, bytes_to_device, from_device, to_device
from tests.test_gguf import _model

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [qg.F16, qg.BF16], ids=["f16", "bf16"])
def test_gguf_weights_through_the_gemm(dtype):
    buf, blocks, _ = _model(alignment=64)
    infos = {t["name"]: t for t in qg.gguf_tensors(buf)}
    for name in ("blk.0.ffn_up.weight", "blk.0.ffn_down.weight", "blk.0.attn_v.weight"):
        fmt, N, K, packed = qg.gguf_pack(buf, infos[name]["index"])
        raw = buf[infos[name]["offset"]:infos[name]["offset"] + infos[name]["nbytes"]]
        W = oracle.dequant(fmt, raw.reshape(N, K // 256, -1), N, K, dtype)
        for M in (37, 300):
            X = synth.activations(np.random.default_rng(M), M, K, dtype)
            print(f"gguf {name} {fmt} M={M} N={N} K={K} dtype={dtype}", flush=True)
            y = from_device((qg.q4k if fmt == "q4k" else qg.q6k)(to_device(X, dtype), bytes_to_device(packed), N))
            Yref, B = oracle.gemm(X, W, dtype)
            assert_gemm_close(y, Yref, B, dtype, what=f"{name} M={M}")
