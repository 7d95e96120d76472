"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

A copy of libfp4mi.so is built with the host code instrumented (the
sanitizer flags apply to the host compilation only; the device code is
built unoptimised because it never runs here), and tests/test_abi_cpu.py --
the status of every documented rule, a randomized sweep of invalid calls and
the exported symbols -- runs against it in a child process with the
sanitizer runtime preloaded.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["quant.hip", "fp4quant.hip", "fp8col.hip", "abi.hip"]


def _tool(*candidates):
    for c in candidates:
        if c and os.path.exists(c):
            return c
    return None


def test_host_validation_under_asan_and_ubsan(tmp_path):
    hipcc = _tool("/opt/rocm/bin/hipcc", shutil.which("hipcc"))
    clang = _tool("/opt/rocm/llvm/bin/clang++")
    if hipcc is None or clang is None:
        pytest.skip("hipcc / clang++ not available")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isfile(rt):
        pytest.skip("the ASan runtime is not available")
    lib = str(tmp_path / "libfp4mi_sanitized.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Wno-unused-command-line-argument", "-Xarch_device", "-O0",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"),
           *[os.path.join(ROOT, "block_scaled_fp4_amd", "csrc", s) for s in SOURCES], "-o", lib]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert b.returncode == 0, b.stderr[-2000:]
    env = dict(os.environ, LD_PRELOAD=rt, FP4MI_SANITIZED_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-3000:]
    assert "runtime error:" not in out and "AddressSanitizer" not in out, out[-3000:]
