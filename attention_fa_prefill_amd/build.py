"""Build the gfx950 HIP libraries in-tree with hipcc.

    python -m attention_fa_prefill_amd.build

libfa.so holds the attention path behind include/fa.h; libfa_ceiling.so holds
the two measurement kernels (streaming read, MFMA loop) that bench.py reports
as the practical ceilings next to the published peaks.

Every source is compiled for gfx950 only. Packed fp32 VALU instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless. prefill_hd.hip is compiled on
its own with the MFMA results in vector registers (its d = 256 kernels keep Q^T
in the accumulation registers instead; see the note above pin_q there), and
linked with the rest.
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
# extra device-compiler flags per source (compiled to an object of its own)
SOURCE_FLAGS = {"prefill_hd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def _build_one(sources, lib, verbose):
    """Each source to an object of its own (with its extra flags), in parallel,
    then one link; hipcc would read an object given beside .hip sources as
    source."""
    objs = [os.path.join(os.path.dirname(lib), "." + src + ".tmp.o") for src in sources]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    try:
        for src, obj in zip(sources, objs):
            cmd = [HIPCC, *compile_flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        for proc in procs:
            out = "\n".join(line for line in proc.communicate()[0].splitlines() if "packed-fp32-ops" not in line)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
            if verbose and out.strip():
                print(out)
        tmp = lib + ".tmp"
        _run([HIPCC, *FLAGS, *objs, "-o", tmp], verbose)
    finally:
        for proc in procs:
            if proc.poll() is None:
                proc.kill()
                proc.communicate()
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _build_one(CEILING_SOURCES, CEILING_LIB, verbose)
    return _build_one(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
