"""Build the HIP shared library (libq8gemv.so) in-tree for gfx950.

    python -m block_quantized_gemv_amd.build

Every HIP source is compiled with hipcc for gfx950 only.  Packed-fp32 vector
instructions are switched off for the device code (the host pass warns that
it does not know the feature; that is harmless).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libq8gemv.so")
ARCH = "gfx950"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def command(out: str = LIB) -> list[str]:
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-o", out] + sources()


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
