"""The host layer (plan compiler, plan cache, one-shot upload bookkeeping, C ABI validation) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer against a HIP stand-in
(tests/host/mock_hip.cpp) and run: a forced hash collision still yields distinct plans, a repeated
one-shot call with one mask and workspace copies nothing, released or overwritten workspaces are
copied again, and every index of the compiled plans' device images is in range.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_softmax_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_harness")
    cmd = ["g++", "-std=c++17", "-O0", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{CSRC}", f"-I{HOST}",
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "plan_cache.cpp"), os.path.join(CSRC, "capi.cpp"),
           os.path.join(HOST, "mock_hip.cpp"), os.path.join(HOST, "harness.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
