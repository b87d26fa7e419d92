"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The allocator (allocator.cpp with host_api.cpp, the library's HIP-free part) and the
oracle (oracle.c) are built with g++ / gcc -fsanitize=address,undefined (undefined
behaviour is fatal), then the allocator tests (the hypothesis comparison with the model
allocator, all-or-nothing batches, out-of-blocks, monitoring figures, host checks) and the
oracle pins run in a child process that loads those builds (PA_LIBRARY, ORACLE_LIBRARY)
with the ASan runtime preloaded.  A sanitizer report, or any failing test, fails this one
("PagedAttention" concept report (compassingai.com) §13: bounds checks and an explicit
out-of-memory path instead of corrupting running work).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_308_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
FLAGS = ["-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer"]


def _runtime():
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_builds():
    asan = _runtime()
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libpa_host_asan.so")
    orc = os.path.join(OUT, "liboracle_asan.so")
    subprocess.run(["g++", "-std=c++17", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "allocator.cpp"), os.path.join(CSRC, "host_api.cpp"), "-o", lib], check=True)
    subprocess.run(["gcc", "-std=c99", *FLAGS, "-fno-fast-math", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", orc], check=True)
    return asan, lib, orc


def test_allocator_and_oracle_under_asan_and_ubsan(sanitized_builds):
    asan, lib, orc = sanitized_builds
    env = dict(os.environ, LD_PRELOAD=asan, PA_LIBRARY=lib, ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    select = ("matches_model or replays_workload or out_of_blocks or midway or monitoring_rates "
              "or invalid_calls or check_tables or check_copy_pairs or test_pin")
    # -s: a sanitizer aborts the child at once, so its report must not sit in pytest's capture
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        "tests/test_native_host.py", "tests/test_oracle_pins.py", "-k", select],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]
