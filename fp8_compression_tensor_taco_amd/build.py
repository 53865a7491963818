"""Build libtaco.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m fp8_compression_tensor_taco_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libtaco.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, "taco.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # packed fp32 VALU ops stay off on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in VGPRs (no v_accvgpr_read copies before the VALU epilogue)
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        f"-I{INCLUDE}",
    ]


def build_library(verbose: bool = True) -> str:
    """Compile every HIP source into ``libtaco.so`` next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_asm(out_path: str) -> None:
    """Device assembly of the library (for inspection of the generated gfx950 code)."""
    cmd = [hipcc(), *compile_flags(), "--cuda-device-only", "-S", *SOURCES, "-o", out_path]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build_library())
