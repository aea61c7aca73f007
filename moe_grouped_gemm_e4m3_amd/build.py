"""Ahead-of-time build of the gfx950 library (``libfp8gemm.so``, in-tree).

``python -m moe_grouped_gemm_e4m3_amd.build`` compiles every HIP source of the
package with hipcc for gfx950.  hipcc cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8gemm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code: the scalar fp32
# FMAs of the promotion are written one per element and stay that way.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Sources and their own options.  The fp32-factor kernels keep MFMA results in
# VGPRs (the promotion FMAs read them directly); the power-of-two-factor
# kernel accumulates in the matrix core and is built without that option, so
# its accumulators go to the accumulation registers.
SOURCES = [
    ("fp8gemm.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("ue8m0.hip", []),
]


def hipcc_path() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise FileNotFoundError("hipcc not found (ROCm is required to build)")
    return p


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source to an object with its options, link the library;
    returns the path of the built .so."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    hipcc = hipcc_path()
    with tempfile.TemporaryDirectory(prefix="fp8gemm_build_") as objdir:
        objs = []
        for src, opts in SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            _run([hipcc, *HIPCC_FLAGS, *opts, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
