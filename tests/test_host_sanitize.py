"""The C ABI's host layer (csrc/api.hip: argument checks, launch planning, the profiling hook) run
under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.

api.hip is compiled for the host only with both sanitizers and linked with the stubs in
tests/host_sanitize/abi_driver.cpp in place of the kernel launchers, so every entry point runs its
checks and planning without a GPU; the driver exercises valid and invalid calls of every entry
point and checks the statuses and the planned launches. Any sanitizer report fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers not installed")

# host-only compilation; each sanitizer flag applies to the host side of the compile
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    common = ["-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              *SAN, "-I", os.path.join(ROOT, "include")]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "driver.o", "abi_driver"))
    _run([HIPCC, *common, "-c", os.path.join(ROOT, "kv_cache_sparsity_amd", "csrc", "api.hip"),
          "-o", api_o])
    _run([HIPCC, *common, "-c", os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp"),
          "-o", drv_o])
    # the link names no HIP source: the sanitizer runtimes are host libraries
    _run([CLANG, "-fsanitize=address,undefined", api_o, drv_o, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr
