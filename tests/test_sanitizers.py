"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer).

Two host-only programs are compiled with gcc/g++ and the sanitizers and run
here, no GPU involved:
  * tests/sanitize/oracle_driver.c with oracle/kda_oracle.c: every oracle
    function on packed sequences with empty, one-token and ragged
    sequences, cross-checked (chunked == recurrent, decode == one-token
    recurrence, (I + A) T = I, restarts of the cumulative sum), and its
    argument checks;
  * tests/sanitize/abi_driver.cpp with the library's host code
    (csrc/kda_api.cpp): the C ABI's validation, workspace layout and launch
    sequencing against recording stubs of the kernel launchers.
Any sanitizer report aborts the program (-fno-sanitize-recover=all), so the
test fails on the first out-of-bounds access, overflow or other undefined
behaviour.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
# the sanitizer runtime need not come first when a preload is present; no
# leak checker under ptrace-restricted containers
ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(tmp_path, compiler, srcs, extra, libs=()):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / "drv")
    cmd = [compiler] + SAN + extra + ["-o", exe] + srcs + list(libs)
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{b.stderr[-4000:]}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"


def test_oracle_under_sanitizers(tmp_path):
    _build_and_run(tmp_path, "gcc",
                   [os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")],
                   ["-std=c11"], ["-lm"])


def test_abi_host_code_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "gated_delta_rule_chunked_amd", "csrc")
    _build_and_run(tmp_path, "g++",
                   [os.path.join(csrc, "kda_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")],
                   ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-w"])
