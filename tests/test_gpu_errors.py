"""Failure handling of the C ABI on the GPU: a device allocation refused in
the middle of rq_init (the RQ_TEST_FAIL_ALLOC hook makes the k-th one fail)
returns RQ_ENOMEM, leaves *out NULL, frees what was already allocated, and
leaves the library usable.  A refused allocation is an ordinary error
return, not a fault."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _init(K, bits, mode):
    h = ctypes.c_void_p(0x1234)
    rc = K.lib().rq_init(128, bits, 0, mode, ctypes.byref(h))
    return rc, h.value


@pytest.mark.parametrize("bits,mode", [(3, 0), (3, 1), (4, 2), (3, 3), (4, 4)])
def test_refused_allocation_in_init(K, bits, mode):
    try:
        # every allocation position in turn, until the session needs fewer
        fails = 0
        for k in range(1, 64):
            os.environ["RQ_TEST_FAIL_ALLOC"] = str(k)
            rc, h = _init(K, bits, mode)
            if rc == K.RQ_OK:
                K.rq_free(h)
                break
            assert rc == K.RQ_ENOMEM, K.rq_last_error()
            assert h is None
            assert "device allocation failed" in K.rq_last_error()
            fails += 1
        else:
            pytest.fail("rq_init never succeeded")
        assert fails >= 3
        # the failing path many times over: nothing stays allocated
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        os.environ["RQ_TEST_FAIL_ALLOC"] = str(fails)     # the last allocation fails
        for _ in range(100):
            rc, h = _init(K, bits, mode)
            assert rc == K.RQ_ENOMEM and h is None
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        assert free0 - free1 < 8 << 20, f"{(free0 - free1) >> 20} MiB not returned"
    finally:
        os.environ.pop("RQ_TEST_FAIL_ALLOC", None)
    # and the library still works
    c = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    x = torch.randn((64, 128), device="cuda").to(torch.float16)
    rec, y = c.roundtrip(x, dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.isfinite(y.cpu().numpy()).all()
