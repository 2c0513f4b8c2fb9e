"""Seeded synthetic inputs for the quantized-weight prefill linear layer.

This module only draws random numbers and lays the drawn fields out in the
GGUF-style byte formats; it holds none of the dequantisation or GEMM
arithmetic.  Both the HIP path (through the packer) and the CPU oracle read
what it produces, so it must import nothing from either of them.

Formats written here (byte layouts follow the GGUF k-quant convention):

* Q4_K, 144 bytes per 256 weights: fp16 ``d``, fp16 ``dmin``, 12 bytes that
  hold eight 6-bit sub-block scales and eight 6-bit sub-block mins, then 128
  bytes of 4-bit codes.  Byte ``32*g + l`` of the code field holds weight
  ``64*g + l`` in its low nibble and weight ``64*g + 32 + l`` in its high
  nibble.  The 12 scale bytes: bytes 0..3 hold ``sc[0..3]`` in their low six
  bits and the top two bits of ``sc[4..7]``; bytes 4..7 do the same for the
  mins; bytes 8..11 hold the low four bits of ``sc[4..7]`` (low nibble) and of
  ``m[4..7]`` (high nibble).
* Q6_K, 210 bytes per 256 weights: 128 bytes of low code nibbles ``ql``, 64
  bytes of high 2-bit pairs ``qh``, 16 signed 8-bit scales (one per 16
  weights), then fp16 ``d``.  Each 128-weight half ``h`` uses ``ql[64h:64h+64]``
  and ``qh[32h:32h+32]``; within it weight ``32*r + l`` (r = 0..3, l = 0..31)
  takes its low nibble from ``ql[64h + l + 32*(r & 1)]`` (low nibble for
  r < 2, high nibble for r >= 2) and its high two bits from bits
  ``2r..2r+1`` of ``qh[32h + l]``.
* W4A16 (GPTQ-style), kept logical: one 4-bit code per byte ``codes[N][K]``,
  fp16 ``scales[K/g][N]``, zero-points ``zeros[K/g][N]`` (0..15); the symmetric
  variant has every zero-point equal to 8.

Distributions follow the workload descriptions: activations ~ N(0, 1) drawn in
fp32 and rounded to nearest-even into fp16 or bf16; fp16 scale-like fields ~
U[1e-3, 1e-2] drawn in fp64 and rounded to fp16; integer fields uniform over
their stated range.  Seeds are ``1000 + workload index``; sub-streams come
from ``SeedSequence(seed).spawn(n)`` and are consumed in a fixed order.
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}

Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
QK = 256


def streams(seed: int, n: int) -> list[np.random.Generator]:
    """``n`` independent PCG64 generators derived from one seed."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def f16_bits(values) -> np.ndarray:
    """fp64/fp32 values -> fp16 bit patterns (numpy's round-to-nearest-even)."""
    return np.asarray(values).astype(np.float16).view(np.uint16)


def bf16_bits_from_f32(values) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (torch CPU round-to-nearest-even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(rng: np.random.Generator, M: int, K: int, dtype: int) -> np.ndarray:
    """X[M][K] ~ N(0,1) drawn in fp32, stored as fp16/bf16 bits (uint16)."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    if dtype == F16:
        return f16_bits(x)
    if dtype == BF16:
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype}")


def _u_f16(rng: np.random.Generator, shape, lo=1e-3, hi=1e-2) -> np.ndarray:
    return f16_bits(rng.uniform(lo, hi, size=shape))


# ----------------------------------------------------------------------------
# Q4_K
# ----------------------------------------------------------------------------

def q4k_fields(rng: np.random.Generator, N: int, K: int) -> dict:
    """Logical Q4_K fields for W stored per output column n, blocks along K."""
    assert K % QK == 0
    nb = K // QK
    return {
        "d": _u_f16(rng, (N, nb)),
        "dmin": _u_f16(rng, (N, nb)),
        "sc": rng.integers(0, 64, size=(N, nb, 8), dtype=np.uint8),
        "m": rng.integers(0, 64, size=(N, nb, 8), dtype=np.uint8),
        "q": rng.integers(0, 16, size=(N, K), dtype=np.uint8),
    }


def q4k_encode(f: dict) -> np.ndarray:
    """Logical fields -> GGUF-style Q4_K blocks, uint8 [N][K/256][144]."""
    d, dmin, sc, m, q = f["d"], f["dmin"], f["sc"], f["m"], f["q"]
    N, nb = d.shape
    out = np.zeros((N, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<u2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:4] = dmin.astype("<u2").view(np.uint8).reshape(N, nb, 2)
    sc = sc.astype(np.uint8)
    m = m.astype(np.uint8)
    s12 = np.zeros((N, nb, 12), dtype=np.uint8)
    s12[:, :, 0:4] = (sc[:, :, 0:4] & 63) | ((sc[:, :, 4:8] >> 4) << 6)
    s12[:, :, 4:8] = (m[:, :, 0:4] & 63) | ((m[:, :, 4:8] >> 4) << 6)
    s12[:, :, 8:12] = (sc[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)
    out[:, :, 4:16] = s12
    qb = q.reshape(N, nb, 4, 2, 32)  # [.., g, lo/hi half of 64, l]
    out[:, :, 16:] = (qb[:, :, :, 0, :] | (qb[:, :, :, 1, :] << 4)).reshape(N, nb, 128)
    return out


# ----------------------------------------------------------------------------
# Q6_K
# ----------------------------------------------------------------------------

def q6k_fields(rng: np.random.Generator, N: int, K: int) -> dict:
    assert K % QK == 0
    nb = K // QK
    return {
        "d": _u_f16(rng, (N, nb)),
        "s": rng.integers(-128, 128, size=(N, nb, 16), dtype=np.int16).astype(np.int8),
        "q": rng.integers(0, 64, size=(N, K), dtype=np.uint8),
    }


def q6k_encode(f: dict) -> np.ndarray:
    """Logical fields -> GGUF-style Q6_K blocks, uint8 [N][K/256][210]."""
    d, s, q = f["d"], f["s"], f["q"]
    N, nb = d.shape
    out = np.zeros((N, nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    qh4 = q.reshape(N, nb, 2, 4, 32)  # [.., half, r, l]
    lo = qh4 & 15
    hi = qh4 >> 4
    ql = np.zeros((N, nb, 2, 64), dtype=np.uint8)
    ql[..., 0:32] = lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4)
    ql[..., 32:64] = lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)
    qhb = hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4) | (hi[:, :, :, 3, :] << 6)
    out[:, :, 0:128] = ql.reshape(N, nb, 128)
    out[:, :, 128:192] = qhb.reshape(N, nb, 64)
    out[:, :, 192:208] = s.view(np.uint8)
    out[:, :, 208:210] = d.astype("<u2").view(np.uint8).reshape(N, nb, 2)
    return out


# ----------------------------------------------------------------------------
# W4A16 (group-wise scale + zero-point)
# ----------------------------------------------------------------------------

def w4a16_fields(rng: np.random.Generator, N: int, K: int, group: int, symmetric: bool) -> dict:
    assert K % group == 0
    ng = K // group
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = _u_f16(rng, (ng, N))
    if symmetric:
        zeros = np.full((ng, N), 8, dtype=np.uint8)
    else:
        zeros = rng.integers(0, 16, size=(ng, N), dtype=np.uint8)
    return {"codes": codes, "scales": scales, "zeros": zeros, "group": group, "symmetric": symmetric}


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

#: One Qwen3-8B dense layer's seven projections at M = 658 prompt tokens:
#: (name, K, N, format).
QWEN3_8B_LAYER = (
    ("q", 4096, 4096, "q4k"),
    ("k", 4096, 1024, "q4k"),
    ("v", 4096, 1024, "q4k"),
    ("o", 4096, 4096, "q4k"),
    ("gate", 4096, 12288, "q4k"),
    ("up", 4096, 12288, "q4k"),
    ("down", 12288, 4096, "q6k"),
)
QWEN3_8B_LAYERS = 36
QWEN3_8B_PROMPT = 658


def weight_fields(fmt: str, rng: np.random.Generator, N: int, K: int, group: int = 128,
                  symmetric: bool = False) -> dict:
    if fmt == "q4k":
        return q4k_fields(rng, N, K)
    if fmt == "q6k":
        return q6k_fields(rng, N, K)
    if fmt == "w4a16":
        return w4a16_fields(rng, N, K, group, symmetric)
    raise ValueError(fmt)


def encode(fmt: str, fields: dict):
    """GGUF-style bytes for the k-quants; the W4A16 fields stay logical."""
    if fmt == "q4k":
        return q4k_encode(fields)
    if fmt == "q6k":
        return q6k_encode(fields)
    if fmt == "w4a16":
        return fields
    raise ValueError(fmt)


#: The named workloads.  Each GEMM is (label, fmt, M, K, N, dtype, group, symmetric);
#: the seed of workload i is 1000 + i and GEMM j of it draws from sub-stream
#: pair j of SeedSequence(seed).spawn(2 * len(gemms)) (X first, then W).
#: "shared_x" maps a GEMM label to the label whose activations it reads (the
#: projections of one layer that take the same input).
WORKLOADS = {
    "q4k_small": {  # single Q4_K GEMM, fp16
        "index": 0,
        "gemms": [("q4k_16x1024x512", "q4k", 16, 1024, 512, F16, 0, False)],
    },
    "q4k_ffn_up_m512": {  # Qwen3-8B FFN up-projection shape at M = 512, fp16
        "index": 1,
        "gemms": [("up", "q4k", 512, 4096, 12288, F16, 0, False)],
    },
    "qwen3_8b_layer_m658": {  # one dense layer's seven linears at 658 prompt tokens, fp16
        "index": 2,
        "gemms": [(name, fmt, QWEN3_8B_PROMPT, K, N, F16, 0, False) for name, K, N, fmt in QWEN3_8B_LAYER],
        # q, k and v read the same normalized hidden state; gate and up the same MLP input
        "shared_x": {"k": "q", "v": "q", "up": "gate"},
        # projections that share an input, run as one GEMM over their weights
        # concatenated along N (each member's outputs are its own columns)
        "merged": [("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up"))],
    },
    "w4a16_g128_m2048": {  # group-wise W4A16, fp16 and bf16, asymmetric and symmetric
        "index": 3,
        "gemms": [(f"{DTYPE_NAMES[dt]}_{'sym' if sym else 'asym'}", "w4a16", 2048, 4096, 12288, dt, 128, sym)
                  for dt in (F16, BF16) for sym in (False, True)],
    },
    "long_prefill_m4096_bf16": {  # wide Q4_K projection plus a 32-wide skinny projection, bf16
        "index": 4,
        "gemms": [("wide", "q4k", 4096, 4096, 12288, BF16, 0, False),
                  ("skinny", "q4k", 4096, 4096, 32, BF16, 0, False)],
        "shared_x": {"skinny": "wide"},  # the narrow gate reads the same hidden state
    },
    "small_m_probes": {  # decode-adjacent M on the up (Q4_K) and down (Q6_K) shapes: weight streams
        "index": 5,
        "gemms": [(f"{lab}_m{M}", fmt, M, K, N, F16, 0, False) for M in (1, 16, 64)
                  for lab, fmt, K, N in (("up", "q4k", 4096, 12288), ("down", "q6k", 12288, 4096))],
    },
}


def x_source(name: str, j: int) -> int:
    """Index of the GEMM whose activations GEMM j of a named workload reads."""
    w = WORKLOADS[name]
    src = w.get("shared_x", {}).get(w["gemms"][j][0])
    return j if src is None else [g[0] for g in w["gemms"]].index(src)


def workload_inputs(name: str, j: int):
    """(X bits, weight fields, encoded weights) of GEMM j of a named workload."""
    w = WORKLOADS[name]
    label, fmt, M, K, N, dt, group, sym = w["gemms"][j]
    rs = streams(1000 + w["index"], 2 * len(w["gemms"]))
    X = activations(rs[2 * x_source(name, j)], M, K, dt)
    fields = weight_fields(fmt, rs[2 * j + 1], N, K, group or 128, sym)
    return X, fields, encode(fmt, fields)


def concat_encoded(fmt: str, encs):
    """Encoded weights of several N x K matrices (one format) as one matrix of
    their columns side by side, in the order given."""
    if fmt in ("q4k", "q6k"):
        return np.concatenate(encs, axis=0)  # [N][K/256][bytes]: columns are the first axis
    out = dict(encs[0])
    out["codes"] = np.concatenate([e["codes"] for e in encs], axis=0)
    out["scales"] = np.concatenate([e["scales"] for e in encs], axis=1)
    if out.get("zeros") is not None:
        out["zeros"] = np.concatenate([e["zeros"] for e in encs], axis=1)
    return out


def step_gemms(name: str, merge: bool = True) -> list[dict]:
    """The GEMMs of one step of a named workload: with merge, each merged
    group of the workload is one GEMM over its members' concatenated weights
    (placed where its first member is), every other GEMM stays as it is.
    Each entry: label, members (GEMM indices), fmt, M, K, N, dtype, group, sym."""
    w = WORKLOADS[name]
    labels = [g[0] for g in w["gemms"]]
    groups = {}
    if merge:
        for lab, members in w.get("merged", []):
            idx = [labels.index(m) for m in members]
            first = w["gemms"][idx[0]]
            for j in idx:
                g = w["gemms"][j]
                assert g[1:4] == first[1:4] and g[5:] == first[5:] and x_source(name, j) == x_source(name, idx[0])
            groups[idx[0]] = (lab, idx)
    member_of = {j for _, idx in groups.values() for j in idx}
    out = []
    for j, (label, fmt, M, K, N, dt, group, sym) in enumerate(w["gemms"]):
        if j in groups:
            lab, idx = groups[j]
            out.append(dict(label=lab, members=idx, fmt=fmt, M=M, K=K, N=sum(w["gemms"][i][4] for i in idx), dt=dt,
                            group=group, sym=sym))
        elif j not in member_of:
            out.append(dict(label=label, members=[j], fmt=fmt, M=M, K=K, N=N, dt=dt, group=group, sym=sym))
    return out


def step_inputs(name: str, members):
    """(X bits, encoded weights) of a step GEMM: the members' shared
    activations and their weights concatenated along N."""
    encs = []
    for j in members:
        X, _, enc = workload_inputs(name, j)
        encs.append(enc)
    fmt = WORKLOADS[name]["gemms"][members[0]][1]
    return X, (encs[0] if len(encs) == 1 else concat_encoded(fmt, encs))


# ---------------------------------------------------------------------------
# Grouped (per-expert) workloads: the routed rows of a mixture-of-experts FFN,
# already grouped by expert.  Routing is not part of the GEMM; its outcome is
# drawn here: each token picks top_k distinct experts with probabilities from
# a seeded Zipf-like popularity, so expert row counts are skewed and some may
# be empty.
# ---------------------------------------------------------------------------

MOE_WORKLOADS = {
    "moe_e128_top8_m658": {  # 128 experts, 8 per token, hidden 2048, expert width 768, 658 prompt tokens
        "index": 6, "tokens": 658, "experts": 128, "top_k": 8, "zipf": 0.8,
        "gemms": [("gate", "q4k", 2048, 768), ("up", "q4k", 2048, 768), ("down", "q6k", 768, 2048)],
        "input_of": [0, 0, 2],  # GEMM j reads the routed rows of GEMM input_of[j]: gate and up share theirs
        "merged": [("gate_up", ("gate", "up"))],  # one grouped GEMM over each expert's gate and up columns
    },
}


def moe_counts(name: str) -> np.ndarray:
    """Rows routed to each expert (int64 [E])."""
    w = MOE_WORKLOADS[name]
    rng = streams(1000 + w["index"], 1)[0]
    E, k = w["experts"], w["top_k"]
    pop = 1.0 / np.arange(1, E + 1) ** w["zipf"]
    pop = pop[rng.permutation(E)]
    pop /= pop.sum()
    counts = np.zeros(E, np.int64)
    for _ in range(w["tokens"]):
        counts[rng.choice(E, size=k, replace=False, p=pop)] += 1
    return counts


def moe_inputs(name: str, j: int, dtype: int = F16):
    """(X bits [T][K], weight fields of all experts as one N*E-column matrix,
    encoded blocks) of GEMM j; expert e owns columns e*N .. (e+1)*N-1.  GEMMs
    that read the same routed rows (gate and up) get the same X."""
    w = MOE_WORKLOADS[name]
    label, fmt, K, N = w["gemms"][j]
    T = int(moe_counts(name).sum())
    rs = streams(2000 + w["index"], 2 * len(w["gemms"]))
    X = activations(rs[2 * w["input_of"][j]], T, K, dtype)
    fields = weight_fields(fmt, rs[2 * j + 1], N * w["experts"], K)
    return X, fields, encode(fmt, fields)


def moe_step_gemms(name: str, merge: bool = True) -> list[dict]:
    """The grouped GEMMs of one MoE step: with merge, each merged group is one
    grouped GEMM whose expert e holds its members' expert-e columns side by
    side (placed where its first member is).  Each entry: label, members
    (GEMM indices), fmt, K, N, input (the GEMM whose routed rows it reads)."""
    w = MOE_WORKLOADS[name]
    labels = [g[0] for g in w["gemms"]]
    groups = {}
    if merge:
        for lab, members in w.get("merged", []):
            idx = [labels.index(m) for m in members]
            first = w["gemms"][idx[0]]
            for j in idx:
                g = w["gemms"][j]
                assert g[1:3] == first[1:3] and w["input_of"][j] == w["input_of"][idx[0]]
            groups[idx[0]] = (lab, idx)
    member_of = {j for _, idx in groups.values() for j in idx}
    out = []
    for j, (label, fmt, K, N) in enumerate(w["gemms"]):
        if j in groups:
            lab, idx = groups[j]
            out.append(dict(label=lab, members=idx, fmt=fmt, K=K, N=sum(w["gemms"][i][3] for i in idx),
                            input=w["input_of"][j]))
        elif j not in member_of:
            out.append(dict(label=label, members=[j], fmt=fmt, K=K, N=N, input=w["input_of"][j]))
    return out


def moe_step_inputs(name: str, members):
    """(X bits [T][K], encoded weights of all experts as one E*N-column
    matrix) of a step GEMM: expert e owns columns e*N .. (e+1)*N-1, its
    members' expert-e columns side by side in member order."""
    w = MOE_WORKLOADS[name]
    E = w["experts"]
    fmt = w["gemms"][members[0]][1]
    X, parts = None, []
    for j in members:
        Xj, _, enc = moe_inputs(name, j)
        X = Xj if X is None else X
        parts.append((enc, w["gemms"][j][3]))
    if len(parts) == 1:
        return X, parts[0][0]
    cols = []
    for e in range(E):
        cols += [enc[e * n:(e + 1) * n] if fmt in ("q4k", "q6k") else _enc_cols(enc, e * n, (e + 1) * n)
                 for enc, n in parts]
    return X, concat_encoded(fmt, cols)


def _enc_cols(enc, c0: int, c1: int):
    """Columns c0 .. c1-1 of a W4A16 encoding (codes [N][...], scales and
    zeros [groups][N])."""
    out = dict(enc)
    out["codes"] = enc["codes"][c0:c1]
    out["scales"] = enc["scales"][:, c0:c1]
    if enc.get("zeros") is not None:
        out["zeros"] = enc["zeros"][:, c0:c1]
    return out
