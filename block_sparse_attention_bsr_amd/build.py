"""Build the HIP library (gfx950) in-tree: ``python -m block_sparse_attention_bsr_amd.build``.

Produces ``block_sparse_attention_bsr_amd/libbsr_attn.so`` from the sources in
``csrc/`` with hipcc. Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
LIBRARY = PKG / "libbsr_attn.so"
SOURCES = [PKG / "csrc" / "kernels.hip", PKG / "csrc" / "api.cpp", PKG / "csrc" / "structure.cpp",
           PKG / "csrc" / "timing.cpp"]
ARCH = "gfx950"

# Device code only: packed fp32 instructions are disabled (the host pass warns
# that it does not know the feature; that is harmless). -Wno-inline-asm
# silences one note repeated for every LDS-DMA asm statement: M0, which the
# statement writes, is a register the compiler reserves (kernels.hip explains
# why that is safe for these kernels).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build_library(verbose: bool = False, extra_flags=()) -> Path:
    out = LIBRARY.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *HIP_FLAGS, *extra_flags, "-shared",
           "-I", str(ROOT / "include"), *map(str, SOURCES), "-o", str(out)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(out, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose=True))
