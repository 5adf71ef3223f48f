"""The host core (rq_host.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/native/host_sanitize_main.cpp builds every
session kind's tables with g++ -fsanitize=address,undefined (any report
aborts the run), and its table digests must equal those of the tables the
built library returns through rq_host_params."""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_vector_norm_amd", "csrc")


def _fnv(h, data):
    for b in data:
        h ^= b
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


@pytest.fixture(scope="module")
def sanitized_run(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("asan") / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "native", "host_sanitize_main.cpp"), os.path.join(CSRC, "rq_host.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    return r


def test_host_core_is_clean_under_asan_and_ubsan(sanitized_run):
    r = sanitized_run
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "failures 0" in r.stdout


def test_sanitized_tables_equal_the_library_tables(sanitized_run):
    import kv_cache_vector_norm_amd as K
    got = {}
    for line in sanitized_run.stdout.splitlines():
        if line.startswith("tables "):
            _, b, m, h = line.split()
            got[(int(b.split("=")[1]), int(m.split("=")[1]))] = int(h, 16)
    assert len(got) == 15
    for (bits, mode), h in got.items():
        p = K.rq_host_params(128, bits, 0, mode)
        x = 1469598103934665603
        for key in ("rotors", "rotmats", "centroids", "boundaries", "pi", "s"):
            if key in p and p[key].size:
                x = _fnv(x, np.ascontiguousarray(p[key]).tobytes())
        assert x == h, (bits, mode)
