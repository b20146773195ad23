"""The host segment allocator under the address and undefined-behaviour sanitizers: its source
(allocator.cpp, plain C++ with no GPU code) and the stress driver tests/native/allocator_stress.cpp
are compiled with the host compiler and -fsanitize=address,undefined (no recovery, so any report
ends the run with an error), then run on random operation sequences of several shapes while the
driver checks the state reported through the C ABI on a bitmap of the pool. Host only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def stress_exe(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path_factory.mktemp("asan") / "allocator_stress"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "attention_segmented_kv_amd", "csrc", "allocator.cpp"),
           os.path.join(ROOT, "tests", "native", "allocator_stress.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("the host compiler has no sanitizers")
    assert r.returncode == 0, r.stderr
    return exe


# (seed, steps, pool slots, requests, largest growth, granule): a roomy pool, a tight one, a tiny
# one where most growth fails, many requests with a coarse granule
CASES = [(1, 20000, 3000, 40, 200, 16), (2, 20000, 500, 8, 40, 1), (3, 5000, 64, 5, 30, 1),
         (4, 20000, 4000, 100, 12, 64), (5, 10000, 1 << 16, 300, 900, 7)]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_allocator_under_sanitizers(stress_exe, case):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(stress_exe), *map(str, case)], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
