"""Host code of the C ABI under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

The host source (validation, byte accounting, arena layout, state bookkeeping, export) is
built with g++ and the sanitizers, against host-memory stand-ins for the HIP runtime and
the kernel launchers (``tests/asan/host_stubs.cpp``), and driven by
``tests/asan/host_main.cpp``: valid and invalid configurations, the create / prefill /
decode / route / export / migration entry points, over a zeroed and over a random
"device" arena.  A memory error, undefined behaviour or a leak aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="needs g++ and the HIP headers")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "qv_host_asan"
    srcs = [os.path.join(ROOT, "recoverable_kv_cache_amd", "csrc", "qevict_host.cpp"),
            os.path.join(ROOT, "tests", "asan", "host_stubs.cpp"),
            os.path.join(ROOT, "tests", "asan", "host_main.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "recoverable_kv_cache_amd", "csrc"), *srcs, "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "host checks passed" in r.stdout
