"""Ahead-of-time build of the gfx950 library (``libfp8gemm.so``, in-tree).

``python -m moe_grouped_gemm_e4m3_amd.build`` compiles every HIP source of the
package with hipcc for gfx950.  hipcc cross-compiles without a GPU.
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
LIB_NAME = "libfp8gemm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["fp8gemm.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code: the scalar fp32
# FMAs of the promotion are written one per element and stay that way.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA results in VGPRs: the promotion FMAs read them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise FileNotFoundError("hipcc not found (ROCm is required to build)")
    return p


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile the library; returns the path of the built .so."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [hipcc_path(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
