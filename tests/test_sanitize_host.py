"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

av_api.hip (host argument checks, launch planning, status strings) and
av_lmhead.hip (the LM-head backward's checks and split planning) are compiled
with -fsanitize=address,undefined for the host only, linked with the
already-built kernel object and a driver (tests/sanitize/abi_driver.cpp) that
calls every entry point with sizes at and beyond their limits and with each
kind of bad argument.  No call reaches the device; a sanitizer report or a
wrong status fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "drafter_distillation_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="hipcc / clang++ not found")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(PKG, "_build", n) for n in ("av_kernels.o",)]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library not built (python -m drafter_distillation_amd.build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    api = str(tmp_path / "av_api_san.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "abi_driver")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    lmh = str(tmp_path / "av_lmhead_san.o")
    for src, obj in (("av_api.hip", api), ("av_lmhead.hip", lmh)):
        subprocess.run([HIPCC, *common, *san, *inc, "-c", os.path.join(PKG, "csrc", src), "-o", obj],
                       check=True, capture_output=True)
    subprocess.run([HIPCC, *common, *san, *inc, "-x", "hip", "-c",
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv],
                   check=True, capture_output=True)
    # linked by the host compiler (the sanitizer runtimes are host-only)
    subprocess.run([CLANG, "-fsanitize=address,undefined", drv, api, lmh, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "ok (0 failed)" in out
