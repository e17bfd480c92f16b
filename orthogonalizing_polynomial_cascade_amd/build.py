"""Build libanvil.so in-tree with hipcc for gfx950.

    python -m orthogonalizing_polynomial_cascade_amd.build

Flags: -O3; -ffp-contract=off so every fp32 operation of the elementwise steps rounds on its own
(as the page's separate tensor operations do); packed fp32 instructions disabled for the device
code; correctly rounded fp32 division (hipcc's default) is kept, no fast-math.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libanvil.so")
SOURCES = ["momentum.hip", "gemm.hip", "normalize.hip", "update.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-function",
        # the LDS-DMA inline assembly writes m0, a reserved register the kernels use nowhere else
        "-Wno-inline-asm",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libanvil.so (always recompiles).  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
