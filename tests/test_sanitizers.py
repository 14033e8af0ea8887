"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer.

pool.cpp, sched.cpp and plan.cpp (the allocator, copy-on-write, the step
scheduler and the decode planning) are built with g++ and
-fsanitize=address,undefined, with tests/sanitize/hip_host_stub.cpp in place
of the HIP runtime and the kernels (no GPU code is built). The allocator,
scheduler and ABI tests, and the stub-runtime cases of
tests/sanitize/stub_device_cases.py, then run against that build in a child
process with the ASan runtime loaded first; any report fails the run. The
pool is externally synchronised ("无 vLLM 环境下的 Paged-KV 与连续批处理调度"
§3.1 guards its request map with a lock), so one thread is what is checked.
CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_62_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("pool.cpp", "sched.cpp", "plan.cpp")] + \
          [os.path.join(ROOT, "tests", "sanitize", "hip_host_stub.cpp")]
TESTS = ["tests/test_allocator.py", "tests/test_scheduler.py", "tests/test_abi.py",
         "tests/sanitize/stub_device_cases.py"]


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("asan") / "libpkv_host_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), *SOURCES, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def test_host_library_under_asan_and_ubsan(sanitized_lib):
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=libasan, PKV_LIB=sanitized_lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the build-entry test compiles the library and the oracle: not this run's subject
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not graft_entry", *TESTS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = (r.stdout[-6000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report
