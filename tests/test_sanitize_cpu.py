"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two programs are built in a temporary directory and run:
  * the C oracle with tests/sanitize/oracle_driver.c (gcc, -fsanitize on the
    whole program): every oracle entry point on the test shapes and the
    method's edge cases, with exact-size heap buffers;
  * the C ABI (dequantizing_gemm_amd/csrc/api.cpp) with
    tests/sanitize/api_driver.cpp and the host stubs of
    tests/sanitize/stub_launchers.cpp in place of the kernel launchers
    (clang in HIP mode; the sanitizers apply to host code only): argument
    validation, overflow checks, size helpers, path choice, workspace checks
    and the per-thread error text.
Each driver also checks its own results and exits non-zero on a failed check;
a sanitizer report also makes it exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
GCC = shutil.which("gcc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\nstdout:\n{r.stdout}\nstderr:\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(GCC is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run([GCC, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "int4_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang++ not found")
def test_c_abi_under_sanitizers(tmp_path):
    hip = [CLANGXX, "-x", "hip", f"--offload-arch=gfx950", f"--rocm-path={ROCM}", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-c"]
    objs = []
    for src in (os.path.join(ROOT, "dequantizing_gemm_amd", "csrc", "api.cpp"),
                os.path.join(SAN, "stub_launchers.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(hip + [src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "api_driver.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-c", os.path.join(SAN, "api_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "api_san")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, drv, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-lpthread", "-o", exe])
    # (leak checking off: the HIP runtime keeps its own allocations to process exit)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout
