"""The library's host code (block managers v1 and v2, the grouping of
sharers) built with AddressSanitizer and UndefinedBehaviorSanitizer by g++,
and driven in a child process (the ASan runtime preloaded into Python) on
random operation sequences checked against the oracle's block managers, plus
edge and error paths (tests/sanitize_driver.py). Any sanitizer report fails
the child. The device kernels cannot be built this way (GPU sanitizers are
not used here); their bounds are covered by the GPU tests' poisoned inputs
and bad-entry cases.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    libasan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("no ASan runtime for g++")
    lib = str(tmp_path / "libpa_host_sanitized.so")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
             "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
             os.path.join(ROOT, "paged_kv_cache_410_amd", "csrc", "block_manager.cpp"), "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_driver.py"), lib,
                        "2024"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "sanitized host code: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
