"""The library's host C++ under AddressSanitizer and UBSan (CPU, no GPU).

tests/host/host_fuzz.cpp drives the KV pool manager and the decode planner
with random arguments, valid and not, and checks their documented promises
(no table word past max_blocks, nothing written by a failed request, plans
within plan_ints).  It is built here with g++ from the host sources only (no
device code), with both sanitizers, and any report fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_agnostic_kv_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("host_fuzz") / "host_fuzz")
    cmd = [cxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "cache_manager.cpp"), os.path.join(CSRC, "decode_plan.cpp"),
           os.path.join(ROOT, "tests", "host", "host_fuzz.cpp"), "-o", exe]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        if "asan" in res.stdout.lower() or "ubsan" in res.stdout.lower():
            pytest.skip("the sanitizer runtimes are not available: " + res.stdout[-300:])
        raise AssertionError(res.stdout)
    return exe


@pytest.mark.parametrize("seed", [12345, 777])
def test_host_code_is_clean_under_sanitizers(driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([driver, "300", str(seed)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, env=env, timeout=300)
    sys.stdout.write(res.stdout[-2000:])
    assert res.returncode == 0 and "ok:" in res.stdout, res.stdout[-4000:]
