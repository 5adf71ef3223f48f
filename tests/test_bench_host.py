"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
machine-code digest that ties measured HBM counters to the kernel they were
taken on."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_code_digest():
    if not os.path.exists(os.path.join(ROOT, "kv_cache_vector_norm_amd", "librq.so")):
        pytest.skip("librq.so not built")
    import bench
    d1 = bench.kernel_code_digest(bench.ROUNDTRIP_SYMBOL)
    d2 = bench.kernel_code_digest(bench.ROUNDTRIP_SYMBOL)
    assert re.fullmatch(r"[0-9a-f]{16}", d1) and d1 == d2
    assert bench.kernel_code_digest() != d1          # the whole offload section is another digest
