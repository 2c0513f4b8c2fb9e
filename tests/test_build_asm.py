"""The fp16 unpack's rounding, checked in the compiled kernels (no GPU).

An fp16 weight is code*factor - bias rounded once.  In source it is a
binary32 fma followed by a conversion to fp16; the compiler turns that pair
into one v_fma_mix{lo,hi}_f16, whose result is the single rounding of the
exact value (the GPU tests pin that on blocks where a binary32 intermediate
would round differently).  Were the compiler ever to keep the binary32 FMA
and a separate conversion instead, fp16 weights of Q4_K blocks with d and
dmin far apart would be rounded twice.  This test compiles every fp16
translation unit to gfx950 assembly and checks that no kernel that unpacks
weights contains a binary32 FMA."""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from quantized_weight_prefill_amd import build as B

# kernels that unpack weights: FMT is their first template argument, DT the second
UNPACKING = ("k_direct", "k_stream", "k_stream32", "k_stream32_sk", "k_grouped_shared", "k_direct_grouped",
             "k_dequant", "k_stage")


def _device_asm(src: str, defines, out: str):
    cmd = [B.hipcc(), *B.COMMON_FLAGS, *defines, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return open(out).read()


def _kernels(asm: str):
    """(kernel symbol, its body) of every kernel in a device .s file."""
    parts = re.split(r"\n(?=_Z\S+:\s+; @)", asm)
    for p in parts:
        m = re.match(r"(_Z\S+):", p)
        if m:
            yield m.group(1), p


@pytest.mark.slow
def test_fp16_unpack_is_one_rounding_in_every_kernel():
    units = [("inst_fp.hip", [f"-DQG_FMT={f}", "-DQG_DT=0", f"-DQG_XL={x}"]) for f in B.FORMATS for x in B.LAYOUTS]
    units += [("misc.hip", []), ("misc_grouped.hip", [])]
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 4)) as ex:
            asms = list(ex.map(lambda iu: _device_asm(iu[1][0], iu[1][1], os.path.join(d, f"u{iu[0]}.s")),
                               enumerate(units)))
    checked = 0
    for asm in asms:
        for name, body in _kernels(asm):
            m = re.match(r"_ZN2qg(\d+)(k_\w+?)ILi(\d+)ELi(\d+)E", name)
            if not m or m.group(2) not in UNPACKING or m.group(4) != "0" or m.group(3) == "3":
                continue  # not an fp16 kernel that unpacks (3: the staged GEMM reads unpacked weights)
            mix = len(re.findall(r"\bv_fma_mix(lo|hi)_f16\b", body))
            fma32 = re.findall(r"\bv_(fmac?_f32|fma_mix_f32|mad_f32|mac_f32|pk_fma_f32)\b", body)
            assert mix > 0, f"{name}: no v_fma_mix in an fp16 unpacking kernel"
            assert not fma32, f"{name}: binary32 FMA {sorted(set(fma32))} in an fp16 unpacking kernel"
            checked += 1
    assert checked >= 80, checked  # every fp16 rung of every format and layout, the grouped and staged kernels
