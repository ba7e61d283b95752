"""The library's host C++ (tq_host.cpp) under AddressSanitizer, UBSan and
LeakSanitizer: built with g++ together with tests/host_sanitize_driver.cpp,
which drives every host path that runs without a GPU (rotations, Lloyd-Max
codebooks, cache layouts and descriptors, the argument checks of every entry
point).  The HIP runtime calls are stubbed to report no device."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "drv"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "host_sanitize_driver.cpp"),
           os.path.join(ROOT, "kv_cache_vector_encode_amd", "csrc", "tq_host.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
