"""Build the gfx950 C-ABI library ``libxpress_argmax.so`` in-tree with hipcc.

Usage: ``python -m vocab_wide_add_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "xpress_argmax.hip"),
        os.path.join(PKG, "csrc", "readout_gemm.hip"),
        os.path.join(PKG, "csrc", "latent.hip"),
        os.path.join(PKG, "csrc", "read_probe.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libxpress_argmax.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE behaviour the readout depends on: no flush of fp32 denormals, no
    # fast-math reassociation.
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # packed fp32 VALU ops stay off (plain v_add_f32 / v_cvt_pk_bf16_f32 only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compile the library and return its path (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-o", tmp] + SRCS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
