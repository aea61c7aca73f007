"""The library's host code (argument checks, plans, size arithmetic) built
with AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
C entry point by tests/host_abi_driver.cpp.  CPU only: the driver's calls
fail a host check, are empty, or stop at the first device query.

The device code is compiled as usual (it is never run here); the sanitizers
instrument the host side only."""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_e4m3_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_abi_driver.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

# each host-only option behind -Xarch_host, so no device code is instrumented
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_code_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory(prefix="fg_san_") as d:
        jobs = []
        for src in ("fp8gemm.hip", "ue8m0.hip"):
            obj = os.path.join(d, src.replace(".hip", ".o"))
            cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
                   *HOST_SAN, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        for j in jobs:
            out, _ = j.communicate(timeout=600)
            assert j.returncode == 0, out[-3000:]
        drv_obj = os.path.join(d, "driver.o")
        exe = os.path.join(d, "host_abi_driver")
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
        r = subprocess.run([CLANG, "-g", "-std=c++17", *san, "-I", INCLUDE, "-c", DRIVER, "-o", drv_obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([CLANG, *san, drv_obj, os.path.join(d, "fp8gemm.o"), os.path.join(d, "ue8m0.o"),
                            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                            "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        env["HIP_VISIBLE_DEVICES"] = ""  # the host paths only, also on a machine with a GPU
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        report = r.stdout + r.stderr
        assert r.returncode == 0, report[-4000:]
        assert "host abi ok" in r.stdout
        assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
