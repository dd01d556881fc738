"""The binding loads libfa.so on PyTorch's HIP runtime, whatever the caller
touches first. PyTorch ships its own copy of the runtime; had libfa.so been
loaded before torch, the process would hold the system runtime as well, and
launches on torch's streams and memory would go through the wrong one. CPU
only: it inspects the mapped libraries of a fresh interpreter."""
import subprocess
import sys

import pytest

pytestmark = pytest.mark.cpu

PROBE = r"""
import attention_fa_prefill_amd as fa
fa.decode_split_tokens(1, 1, 1, 16, 0)   # the first call loads libfa.so
import torch
paths = sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})
print('\n'.join(paths))
"""


def test_one_hip_runtime_in_the_process():
    pytest.importorskip("torch")
    out = subprocess.run([sys.executable, "-c", PROBE], capture_output=True, text=True, check=True, timeout=300,
                         cwd=__import__("os").path.dirname(__import__("os").path.dirname(__file__))).stdout
    paths = [p for p in out.split("\n") if p]
    assert len(paths) == 1, paths
