"""The library's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

communication_compressed_optimizer_amd/csrc/onebit_host.hpp holds every
piece of libonebit.so's host logic that needs no GPU: the tensor table's
construction and its size bounds, the overlap check of a call's arrays,
byte counts, the workspace layout and the hyper-parameter domains.  It
includes no HIP header, so tests/native/host_check.cc compiles it with g++
and the sanitizers and fuzzes it against brute-force references (random
ragged tables checked element by element and segment by segment, sizes at
the chunk bounds (2^30 - 1 chunks, and under 2^32 work-items per launch) and at
int64 overflow, pointer ranges near the top
of the address space, random hyper-parameter structs)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "communication_compressed_optimizer_amd", "csrc"),
           "-o", str(exe), os.path.join(ROOT, "tests", "native", "host_check.cc")]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    assert "warning" not in build.stderr, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "host check ok" in res.stdout
