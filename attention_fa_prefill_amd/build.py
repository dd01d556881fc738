"""Build the gfx950 HIP libraries in-tree with hipcc.

    python -m attention_fa_prefill_amd.build

libfa.so holds the attention path behind include/fa.h; libfa_ceiling.so holds
the two measurement kernels (streaming read, MFMA loop) that bench.py reports
as the practical ceilings next to the published peaks.

Every source is compiled for gfx950 only. Packed fp32 VALU instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.hip", "prefill_bf16.hip", "prefill_hd.hip", "prefill_f32.hip", "decode.hip"]
CEILING_LIB = os.path.join(HERE, "libfa_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _build_one(sources, lib, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _build_one(CEILING_SOURCES, CEILING_LIB, verbose)
    return _build_one(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
