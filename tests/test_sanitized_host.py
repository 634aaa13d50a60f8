"""The library's host code -- the block allocator and the C ABI (pool.cpp,
capi.cpp) -- built with AddressSanitizer and UndefinedBehaviorSanitizer, the
device launches replaced by stand-ins that fail (tests/sanitize/host_stubs.cpp),
and driven by the C-ABI CPU tests in a child process with the sanitizer
runtime preloaded: the golden allocator trace, hypothesis operation sequences
against the oracle's model (allocation, fork, append, prefix cache, swap),
swap-plan checks and every entry point's argument validation.  Any sanitizer
report fails the run."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_block_quantized_amd", "csrc")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    lib = tmp_path / "libpbq_host_sanitized.so"
    # (_GLIBCXX_SANITIZE_VECTOR: std::vector accesses past size() but within
    # capacity are reported too)
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D_GLIBCXX_SANITIZE_VECTOR", "-shared", "-fPIC",
             "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "pool.cpp"),
             os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
             "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    runtime = subprocess.check_output([gxx, "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, LD_PRELOAD=runtime, PBQ_LIB_PATH=str(lib),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # (-s: a report goes to stderr as the runtime aborts the child, not into
    # pytest's capture)
    r = subprocess.run([sys.executable, "-m", "pytest", "-s", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join("tests", "test_capi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
