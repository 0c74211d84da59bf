"""The oracle and the library's host-side code built with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): tests/sanitize/oracle_driver.cpp runs the oracle on
small problems and its error paths; tests/sanitize/abi_driver.c calls every C-ABI entry point
with arguments the host validation must reject (no device work).  A sanitizer report aborts
the driver, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
           ASAN_OPTIONS="abort_on_error=0:halt_on_error=1")


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{out}"
    return out


def test_oracle_under_asan_ubsan():
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    run(["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-I" + os.path.join(ROOT, "oracle"), os.path.join(SAN, "oracle_driver.cpp"),
         os.path.join(ROOT, "oracle", "iha_oracle.cpp"), "-o", exe])
    out = run([exe], env=dict(ENV, OMP_NUM_THREADS="2"))
    assert "oracle driver: ok" in out, out


def test_host_validation_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from interleaved_head_layer_amd import build as hb
    os.makedirs(OUT, exist_ok=True)
    os.makedirs(hb.OBJDIR, exist_ok=True)
    # The kernels' objects as the library builds them; the C-ABI source again with the host
    # half instrumented (device code is never instrumented).
    others = [s for s in hb.SOURCES if s != "iha.hip"]
    objs = [os.path.join(hb.OBJDIR, s.replace(".hip", ".o")) for s in others]
    for s, o in zip(others, objs):
        if not os.path.exists(o) or os.path.getmtime(o) < os.path.getmtime(os.path.join(hb.CSRC, s)):
            hb._compile(s, False)
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + hb.CSRC]
    san_obj = os.path.join(OUT, "iha_san.o")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         *inc, "-c", os.path.join(hb.CSRC, "iha.hip"), "-o", san_obj])
    drv_obj = os.path.join(OUT, "abi_driver.o")
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-D__HIP_PLATFORM_AMD__",
         "-I" + os.path.join(ROCM, "include"), *inc, "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv_obj])
    exe = os.path.join(OUT, "abi_driver")
    run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-fno-gpu-sanitize",
         san_obj, *objs, drv_obj, "-o", exe])
    out = run([exe], env=dict(ENV, ASAN_OPTIONS=ENV["ASAN_OPTIONS"] + ":detect_leaks=0"))
    assert "abi driver: ok" in out, out
