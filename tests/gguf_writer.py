"""A minimal GGUF (version 3) writer for the tests: header, metadata,
tensor infos, alignment padding and the data section, written from the
container's published layout independently of the library's reader."""
from __future__ import annotations

import struct

import numpy as np

U32, I32, F32, BOOL, STRING, ARRAY, U64, F64 = 4, 5, 6, 7, 8, 9, 10, 12


def _str(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STRING:
        return _str(v)
    if t == ARRAY:
        et, items = v
        body = b"".join(_value(et, x) for x in items)
        return struct.pack("<IQ", et, len(items)) + body
    fmt = {U32: "<I", I32: "<i", F32: "<f", BOOL: "<B", U64: "<Q", F64: "<d"}[t]
    return struct.pack(fmt, v)


def write(kv, tensors, alignment: int = 32, version: int = 3) -> bytes:
    """kv: [(key, type, value)]; tensors: [(name, ggml type, dims (row length
    first), raw bytes)].  general.alignment is written when alignment != 32."""
    kv = list(kv)
    if alignment != 32:
        kv.append(("general.alignment", U32, alignment))
    out = bytearray(struct.pack("<IIQQ", 0x46554747, version, len(tensors), len(kv)))
    for key, t, v in kv:
        out += _str(key) + struct.pack("<I", t) + _value(t, v)
    offs, pos = [], 0
    for name, gt, dims, data in tensors:
        pos = -(-pos // alignment) * alignment
        offs.append(pos)
        pos += len(data)
    for (name, gt, dims, data), off in zip(tensors, offs):
        out += _str(name) + struct.pack("<I", len(dims)) + b"".join(struct.pack("<Q", d) for d in dims)
        out += struct.pack("<IQ", gt, off)
    out += b"\0" * (-len(out) % alignment)
    base = len(out)
    for (name, gt, dims, data), off in zip(tensors, offs):
        out += b"\0" * (base + off - len(out))
        out += bytes(data)
    return bytes(out)


def as_array(b: bytes) -> np.ndarray:
    return np.frombuffer(b, dtype=np.uint8).copy()
