"""Build the HIP library libqgemm.so in-tree for gfx950 (hipcc), and the
measurement-aid library libqprobe.so beside it.

The library is the product: the fused-dequant kernels, the packers and the C
ABI of include/qgemm.h.  The kernels are split into translation units (one
per format x dtype x activation layout for the fp16/bf16 path, one per
format x dtype for the int8 path) that compile in parallel into
``_build/`` and link into one shared object.
Run `python -m quantized_weight_prefill_amd.build`.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqgemm.so")
PROBE_LIB = os.path.join(PKG, "libqprobe.so")
ARCH = "gfx950"
FORMATS = (0, 1, 2)  # QGEMM_FMT_Q4K, _Q6K, _W4A16
DTYPES = (0, 1)      # QGEMM_F16, QGEMM_BF16
LAYOUTS = (0, 1)     # row-major, fragment-major activations

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def units():
    """(object name, source, extra flags) of every translation unit."""
    out = [("api", "api.hip", []), ("misc", "misc.hip", []), ("misc_grouped", "misc_grouped.hip", []),
           ("misc_i8", "misc_i8.hip", []), ("pack", "pack.cpp", []),
           ("noalloc", "noalloc.hip", []), ("gguf", "gguf.cpp", [])]
    for f in FORMATS:
        for d in DTYPES:
            for x in LAYOUTS:
                out.append((f"inst_fp_{f}{d}{x}", "inst_fp.hip", [f"-DQG_FMT={f}", f"-DQG_DT={d}", f"-DQG_XL={x}"]))
            out.append((f"inst_i8_{f}{d}", "inst_i8.hip", [f"-DQG_FMT={f}", f"-DQG_DT={d}"]))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag: harmless
    text = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if text.strip():
        print(text, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = jobs or min(16, os.cpu_count() or 4)
    cmds = []
    for name, src, extra in units():
        obj = os.path.join(BUILD, name + ".o")
        cmds.append((obj, [cc, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda oc: _run(oc[1], verbose), cmds))
    # export the C ABI only (the kernels' host stubs and the internal
    # launch functions stay local to the library)
    vscript = os.path.join(BUILD, "exports.map")
    with open(vscript, "w") as f:
        f.write("{ global: qgemm_*; local: *; };\n")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", f"-Wl,--version-script={vscript}", "-o", LIB + ".tmp",
          *[o for o, _ in cmds]], verbose)
    os.replace(LIB + ".tmp", LIB)
    _run([cc, *COMMON_FLAGS, "-shared", "-o", PROBE_LIB + ".tmp", os.path.join(CSRC, "probe", "qprobe.hip")], verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    sys.exit(0)
