"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``kvc_api.cpp`` and ``layout.cpp`` (config validation, buffer layout, step
protocol, split planning, page allocator, static steps, admits, timing) are
compiled with g++ and ``-fsanitize=address,undefined`` together with host
stand-ins for the HIP runtime and the kernel launchers
(``tests/host_sanitize/hip_host_stub.cpp``), then driven through the C ABI by
``tests/host_sanitize/protocol_driver.cpp`` over several cache shapes
(decode stack, rings with chunked prefill, mixed rows, paged, hybrid groups,
fp32 with a window mask, 300 rows).  The colibri PR "inkling: ring-buffer KV
cache", section "Tests done", builds its engine with extra warnings and checks
cache offsets for overflow; this is that check for the host side.  No GPU is
used.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cached_gqa_append_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "protocol_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(CSRC, "kvc_api.cpp"), os.path.join(CSRC, "layout.cpp"),
           os.path.join(HERE, "hip_host_stub.cpp"), os.path.join(HERE, "protocol_driver.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert run.stdout.startswith("ok:"), run.stdout
