"""Build the HIP library ``libkda_decode.so`` for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "kda_decode.hip"),
           os.path.join(PKG, "csrc", "kda_chunked.hip"),
           os.path.join(PKG, "csrc", "kda_chunk_pass.hip"),
           os.path.join(PKG, "csrc", "kda_probe.hip")]
LIB = os.path.join(PKG, "libkda_decode.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=fast",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 3 kernel-argument dwords preloaded into scalar registers
    # (the decode kernel's slot-index pointer and head count)
    "-mllvm", "-amdgpu-kernarg-preload-count=3",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES,
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkda_decode.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
