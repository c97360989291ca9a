"""The host side of libkvq (argument checks, partition plans, the table
checker; csrc/kvq_api.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers replaced by host
stubs that check the argument blocks the API builds
(tests/sanitize/host_stubs.cpp).  No GPU: two child processes (the
sanitizer runtime preloaded) run the ABI tests against that build and a
grid of valid calls of every entry point over formats, head counts,
batches, lengths, partition lengths and partition modes.  Any sanitizer
report or stub check aborts the child, failing the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_paged_kv_02_amd", "csrc")


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    return gxx


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    gxx = _gxx()
    out = str(tmp_path_factory.mktemp("san") / "libkvq_host_san.so")
    cmd = [gxx, "-std=c++17", "-fPIC", "-shared", "-g", "-O1", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", os.path.join(CSRC, "kvq_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", KVQ_TEST_LIB=out)
    return out, env


def test_abi_tests_under_sanitizers(sanitized_lib):
    lib, env = sanitized_lib
    # the noalloc entry point lives in a HIP source (not in this build);
    # the export checks read the real library
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k",
                        "not noalloc and not every_declared and not header_declares"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_valid_calls_under_sanitizers(sanitized_lib):
    lib, env = sanitized_lib
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize",
                                                     "drive_host_api.py"), lib],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "valid host calls" in r.stdout
