"""The library runs on the same HIP runtime as PyTorch (one runtime per
process), whatever the import order of the caller."""
from __future__ import annotations

import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import quantized_weight_prefill_amd as qg
lib = qg.lib()                       # opened before any explicit torch use
import torch
maps = open('/proc/self/maps').read()
hip = sorted({{l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}})
print('HIP runtimes:', hip)
assert len(hip) == 1, hip
x = torch.zeros((16, 256), dtype=torch.float16, device='cuda')
w = torch.zeros(qg.q4k_packed_bytes(16, 256), dtype=torch.uint8, device='cuda')
y = qg.q4k(x, w, 16)
torch.cuda.synchronize()
assert not y.any()
print('ok')
"""


def test_single_hip_runtime():
    import os

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=root)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "ok" in r.stdout
