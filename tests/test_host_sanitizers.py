"""The library's offline host code (pack.cpp: ternarise, pack, repack, unpack)
under the address + undefined-behaviour and the thread sanitizers, and the CPU
oracle (oracle/oracle.c) under the address + undefined-behaviour sanitizers.

tests/host/pack_sanitize.cpp drives round trips over many shapes and all three
scale granularities; tests/host/oracle_sanitize.c calls every oracle function on
exactly sized heap buffers and checks its products against a dense integer
product.  Both are built here with the host compilers (no device code) and must
run clean.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host", "pack_sanitize.cpp")
PACK = os.path.join(ROOT, "bit_gemv_i2_amd", "csrc", "pack.cpp")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


@pytest.mark.parametrize("sanitizers", ["address,undefined", "thread"])
def test_pack_code_runs_clean_under_sanitizers(tmp_path, sanitizers):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "pack_sanitize")
    cmd = ["g++", "-O1", "-g", "-std=c++17", f"-fsanitize={sanitizers}", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "bit_gemv_i2_amd", "csrc"), "-I" + ROCM_INCLUDE,
           DRIVER, PACK, "-o", exe, "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "cannot find" in build.stderr and "san" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "ok (0 failures)" in run.stdout
    assert "runtime error" not in run.stderr and "WARNING: ThreadSanitizer" not in run.stderr


ORACLE_DRIVER = os.path.join(ROOT, "tests", "host", "oracle_sanitize.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")


def test_oracle_runs_clean_under_address_and_undefined_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", ORACLE_DRIVER, ORACLE_SRC, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "cannot find" in build.stderr and "san" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "ok (0 failures)" in run.stdout
    assert "runtime error" not in run.stderr
