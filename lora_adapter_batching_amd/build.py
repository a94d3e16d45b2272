"""Builds liblora_sgmv.so (gfx950) in-tree with hipcc.

Usage: python -m lora_adapter_batching_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblora_sgmv.so")
SOURCES = ["lora_api.cpp", "lora_fwd.hip", "lora_bwd.hip", "lora_noalloc.hip"]
ARCH = os.environ.get("LORA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


# Code-generation flags of every device compile (the library and the ISA checks).
CODEGEN_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    # packed fp32 instructions stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels read their plan (the kernel argument) in many places; above
    # LLVM's default of 300 such reads it keeps a private copy of the plan in
    # scratch memory instead of reading the argument itself
    "-mllvm", "-instcombine-max-copied-from-constant-users=4096",
]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    cmd = [hipcc()] + CODEGEN_FLAGS + ["-fPIC", "-shared",
                                       "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
                                       "-o", LIB + ".tmp"]
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        if s.endswith(".cpp"):
            cmd += ["-x", "hip", src]
        else:
            cmd += [src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
