"""Compile the HIP sources of this package into ``libq8proj.so`` for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libq8proj.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed FP32 (v_pk_*_f32) code generation is switched off on purpose; the
# kernels are written for plain f32 VALU and MFMA.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    # MFMA results go straight to VGPRs (the GEMM epilogue reads them with VALU).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(extra: list[str] | None = None, out: str = LIB_PATH, verbose: bool = False) -> str:
    """Always recompiles; returns the path of the shared library."""
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *(extra or []), *sources(), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
