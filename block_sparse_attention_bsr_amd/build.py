"""Build the libraries in-tree: ``python -m block_sparse_attention_bsr_amd.build``.

Produces ``block_sparse_attention_bsr_amd/libbsr_attn.so`` (the HIP kernels
for gfx950 and the C ABI, from ``csrc/`` with hipcc) and
``block_sparse_attention_bsr_amd/libbsr_attn_torch.so`` (the PyTorch operator
registration over that C ABI, ``csrc/torch_ops.cpp``, host code built with
g++ against the installed torch). Always recompiles.
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
TORCH_LIBRARY = PKG / "libbsr_attn_torch.so"
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
    cmd = [hipcc(), f"--offload-arch={ARCH}", *HIP_FLAGS, *extra_flags, "-shared", f"-Wl,-soname,{LIBRARY.name}",
           "-I", str(ROOT / "include"), *map(str, SOURCES), "-o", str(out)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(out, LIBRARY)
    return LIBRARY


def build_torch_ops(verbose: bool = False) -> Path:
    """The operator library; links libbsr_attn.so (found next to it at run
    time) and torch's own libraries."""
    import torch

    if not LIBRARY.exists():
        raise RuntimeError(f"{LIBRARY} is missing: build it first")
    tdir = Path(torch.__file__).resolve().parent
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    out = TORCH_LIBRARY.with_suffix(".so.tmp")
    cmd = [os.environ.get("CXX", "g++"), "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-I", str(ROOT / "include"), "-I", str(tdir / "include"),
           "-I", str(tdir / "include" / "torch" / "csrc" / "api" / "include"), "-I", "/opt/rocm/include",
           str(PKG / "csrc" / "torch_ops.cpp"), "-L", str(PKG), "-lbsr_attn", "-L", str(tdir / "lib"), "-ltorch",
           "-ltorch_cpu", "-lc10", "-lc10_hip", "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{tdir / 'lib'}", "-o", str(out)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"g++ failed with status {res.returncode}")
    os.replace(out, TORCH_LIBRARY)
    return TORCH_LIBRARY


def build_all(verbose: bool = False) -> None:
    build_library(verbose=verbose)
    build_torch_ops(verbose=verbose)


if __name__ == "__main__":
    build_all(verbose=True)
    print(LIBRARY, TORCH_LIBRARY)
