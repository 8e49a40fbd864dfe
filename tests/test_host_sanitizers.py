"""The library's host C++ (page allocator, validators) under AddressSanitizer and
UndefinedBehaviorSanitizer: `tests/host/sanitize_driver.cpp` is built with g++ together with
`page_allocator.cpp` and `validate.cpp` and run on seeded random operation streams that include
out-of-range and hostile arguments; it checks the allocator's bookkeeping invariants after every
operation.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_pages_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_driver"
    sources = [os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"), os.path.join(CSRC, "page_allocator.cpp"),
               os.path.join(CSRC, "validate.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), *sources, "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "all checks passed" in run.stdout
    counts = dict(zip(run.stdout.split()[0:14:2], map(int, run.stdout.split()[1:14:2])))
    # every path was reached many times: admissions, successful and refused steps, releases,
    # refusals beyond the credits, rejected prefill layouts
    assert min(counts.values()) >= 20, counts
