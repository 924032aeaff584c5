"""Build libblockattn.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libblockattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 VALU ops stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


EXAMPLE_OUT = os.path.join(HERE, "abi_example")


def build_example(verbose=False):
    """The C-ABI example program (host code only), linked against the in-tree library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = EXAMPLE_OUT + ".tmp"
    cmd = [hipcc, "-O2", "-std=c++17", os.path.join(CSRC, "abi_example.cpp"), "-o", tmp,
           "-L" + HERE, "-lblockattn", "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-4000:]}")
    os.replace(tmp, EXAMPLE_OUT)
    return EXAMPLE_OUT


def build_library(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, os.path.join(CSRC, "blockattn.hip"), os.path.join(CSRC, "noalloc.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-4000:]}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_example(verbose=True))
