"""The library's host code under AddressSanitizer (with leak detection) and
UndefinedBehaviorSanitizer, on the CPU.

spin.cpp is compiled with both sanitizers on its host side (its device side
holds no kernels) and linked with stand-ins for the kernel launchers
(`tests/host_sanitize/stubs.cpp`) and a driver (`tests/host_sanitize/
driver.cpp`) that calls every entry point needing no GPU: null and
malformed arguments, the five workloads' configurations, the edges of every
field's range and 200,000 seeded random configurations, and context creation
on host memory, whose failure at the first HIP call must free what it took.
A sanitizer report aborts the driver; the test requires a clean exit."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_tiered_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers not installed")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_code_is_clean_under_sanitizers(tmp_path):
    # each sanitizer flag applies to the host compilation only
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", f"-I{INC}", f"-I{CSRC}", "-x", "hip"]
    spin_o, stubs_o = str(tmp_path / "spin.o"), str(tmp_path / "stubs.o")
    driver_o, exe = str(tmp_path / "driver.o"), str(tmp_path / "driver")
    _run([HIPCC, *common, *host_san, "-c", os.path.join(CSRC, "spin.cpp"), "-o", spin_o])
    _run([HIPCC, *common, "-c", os.path.join(HERE, "stubs.cpp"), "-o", stubs_o])
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([CLANG, "-O1", "-g", "-std=c++17", *san, f"-I{INC}", "-c", os.path.join(HERE, "driver.cpp"),
          "-o", driver_o])
    _run([CLANG, *san, "-o", exe, driver_o, spin_o, stubs_o, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "Sanitizer" not in out, out
    assert "0 failures" in r.stdout, out
