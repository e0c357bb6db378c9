"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The oracle (oracle/oracle.cpp) built with -fsanitize=address,undefined
   runs the oracle's pin tests (tests/test_oracle_*.py, mutants excepted) in a
   child process that preloads the sanitizer runtime.
2. The C ABI's argument validation (block_scaled_gemm_amd/csrc/mm_api.cpp,
   host code instrumented, device code plain) runs
   tests/sanitized/host_validation.cpp: rejected and empty calls with the
   kernel launchers replaced by counting stubs.
Any sanitizer report ends the child with a non-zero status.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_gcc_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", lib, os.path.join(ROOT, "oracle", "oracle.cpp")],
                   check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _gcc_runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    env["ORACLE_LIB_PATH"] = lib
    files = ["test_oracle_fp8.py", "test_oracle_gemm.py", "test_oracle_atom.py", "test_oracle_fp4.py",
             "test_oracle_grouped.py", "test_oracle_grouped_layouts.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu"] +
                       [os.path.join(ROOT, "tests", f) for f in files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail


def test_host_validation_under_asan_ubsan(tmp_path):
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_scaled_gemm_amd", "csrc")]
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "host_validation")
    subprocess.run([HIPCC, "-x", "hip", "-c", os.path.join(ROOT, "block_scaled_gemm_amd", "csrc", "mm_api.cpp"),
                    "-o", api] + common, check=True, capture_output=True)
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-c",
                    os.path.join(ROOT, "tests", "sanitized", "host_validation.cpp"), "-o", drv] + common,
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fsanitize=undefined", api, drv, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in out, out[-4000:]
