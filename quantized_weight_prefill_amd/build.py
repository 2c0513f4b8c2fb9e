"""Build the HIP library libqgemm.so in-tree for gfx950 (hipcc).

The library is the product: the fused-dequant kernels, the packers and the C
ABI of include/qgemm.h.  Run `python -m quantized_weight_prefill_amd.build`.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libqgemm.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("qgemm.hip", "pack.cpp", "probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-o", LIB + ".tmp", *SOURCES,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
