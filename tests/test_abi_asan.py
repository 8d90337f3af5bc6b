"""The C ABI's host code (argument checks, workspace carving, launch order)
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven through
every entry point, its error paths and its success paths, with the kernel
launchers replaced by host stand-ins (tests/asan/stubs.cpp).  No GPU: the
sanitizers cover host code only."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

ASAN = os.path.join(ROOT, "tests", "asan")


def test_abi_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "abi_asan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "dsa_lightning_indexer_04_amd", "csrc", "abi.cpp"),
           os.path.join(ASAN, "stubs.cpp"), os.path.join(ASAN, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " 0 failed" in r.stdout
