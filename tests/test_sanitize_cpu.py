"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The planners (planner.cpp, chunking.cpp) and the host layer of the C ABI
(api.cpp: argument validation, plan tables, workspace layout, upload) are
compiled for the host alone with clang++ and both sanitizers, linked against
host stand-ins for the kernel launchers (tests/sanitize/stubs.cpp), and
driven with random valid and invalid inputs (tests/sanitize/driver.cpp).
The upload stand-in copies the tables into real host memory of exactly the
workspace size the library reports, so an overrun of the workspace layout
is an AddressSanitizer error.  No device code is built or run here."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segmented_causal_attention_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not available")
    out = str(tmp_path_factory.mktemp("sanitize") / "driver")
    srcs = [os.path.join(CSRC, f) for f in ("planner.cpp", "chunking.cpp", "api.cpp")]
    srcs += [os.path.join(HERE, f) for f in ("stubs.cpp", "driver.cpp")]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [CLANG, "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *srcs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_host_code_is_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "0 failures" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
