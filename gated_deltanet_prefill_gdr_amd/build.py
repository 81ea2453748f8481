"""Build the HIP library libgdr.so in-tree for gfx950 (MI355X) with hipcc.

Cross-compiles without a GPU. Every call rebuilds (no staleness heuristics), writing to a
temporary file first and renaming it into place, so a failed build never leaves a broken
library behind.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = ["gdr_prep.hip", "gdr_scan.hip", "gdr_decode.hip", "gdr_layer.hip", "gdr_noalloc.hip", "gdr_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError(f"hipcc not found ({exe})")
    return exe


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops are kept off for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        # inline assembly must not name reserved registers in its clobber lists
        "-Werror=inline-asm",
    ]


def build(verbose: bool = False) -> str:
    """Compile csrc/ into libgdr.so next to this file; return its path."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(), "-shared", "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
