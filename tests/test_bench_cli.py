"""bench.py's command-line contract on the host (no GPU): more than one GPU
is refused with a message, and the helpers that shape the JSON line behave
(kernel names picked like the library, the packed-layer digest, the CPU
model string)."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("name,T,kernel", [
    ("olmoe", 1, "gemv_dx_kernel"), ("olmoe", 512, "mfma_dx_kernel"),
    ("qwen235", 1, "gemv_dx_kernel"), ("mixtral", 2048, "mfma_dx_kernel"),
])
def test_dx_kernel_name(name, T, kernel):
    assert bench.dx_kernel_name(synth.CONFIGS[name], T) == kernel


def test_packed_digest_changes_with_one_byte():
    class PW:
        def __init__(self, codes, scales):
            self.codes, self.scales, self.scales2 = codes, scales, None

    class L:
        pass

    a, b = L(), L()
    codes = torch.arange(64, dtype=torch.uint8)
    a.projs = [PW(codes.clone(), torch.ones(4))]
    c2 = codes.clone()
    c2[17] ^= 1
    b.projs = [PW(c2, torch.ones(4))]
    da, db = bench.packed_digest(a), bench.packed_digest(b)
    assert len(da) == 64 and da != db
    assert da == bench.packed_digest(a)


def test_cpu_model_is_a_string_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
