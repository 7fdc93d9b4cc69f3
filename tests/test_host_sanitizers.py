"""AddressSanitizer / UndefinedBehaviorSanitizer build of the host code.

The mask compiler and the C ABI (static_block_sparse_amd/csrc/mask.cpp,
capi.cpp) are compiled with g++ -fsanitize=address,undefined together with
tests/sanitize/driver.cpp, which calls every host-side entry point over a
sweep of shapes, flags and mask variants with exactly sized caller buffers,
and tests/sanitize/fake_device.cpp, a host-memory stand-in for the HIP runtime
whose kernel launchers touch the first and last element of every range a
kernel would read or write.  Any heap overflow, leak, use after free or
undefined behaviour fails the run.  CPU only.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "static_block_sparse_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.fixture(scope="module")
def driver():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    tmp = tempfile.mkdtemp(prefix="radial_san_")
    exe = os.path.join(tmp, "driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mask.cpp"), os.path.join(CSRC, "capi.cpp"),
           os.path.join(SAN, "fake_device.cpp"), os.path.join(SAN, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        shutil.rmtree(tmp, ignore_errors=True)
        pytest.fail("sanitizer build failed:\n" + r.stdout + r.stderr)
    yield exe
    shutil.rmtree(tmp, ignore_errors=True)


def test_host_code_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), out[-4000:]
