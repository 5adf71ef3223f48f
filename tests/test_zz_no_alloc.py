"""rq_attend_noalloc (the fixed-scratch variant of rq_attend for callers that
cannot allocate) against rq_attend with a caller workspace, through the C
ABI: both run the same kernels in the same order, so their outputs must be
identical bit for bit.  Two calls in a row on the fixed array, the second
with a smaller input, then a size beyond the array's limit, which must be
refused without touching the output."""
import ctypes

import numpy as np
import pytest

from kv_cache_vector_norm_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _records(K, codec, n, seed):
    x = torch.from_numpy(W.gaussian(n, seed=seed, dtype=np.float16)).cuda()
    return codec.quantize(x)


def _both(K, kc, vc, krec, vrec, q, group, t, kv_stride, scale):
    hq = q.shape[0]
    ref = torch.full((hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full((hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    need = K.rq_attend_workspace(hq, group, t)
    assert 0 < need <= K.RQ_ATTEND_NOALLOC_BYTES
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    base = ws.data_ptr()
    wsp = base + ((-base) % 256)
    parts = (krec.codes, krec.norms, krec.signs, krec.rnorms, vrec.codes, vrec.norms, vrec.signs, vrec.rnorms)
    K.rq_attend(kc.ctx, vc.ctx, q, hq, group, *parts, t, kv_stride, scale, wsp, need, ref, 128)
    K.rq_attend_noalloc(kc.ctx, vc.ctx, q, hq, group, *parts, t, kv_stride, scale, got, 128)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_equals_rq_attend_two_calls(K):
    kc = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    vc = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    scale = 1.0 / np.sqrt(128.0)
    # first call: 4 KV heads x 20,000 keys, GQA 8:1 (32 query rows)
    heads, t, group = 4, 20000, 8
    krec = _records(K, kc, heads * t, 11)
    vrec = _records(K, vc, heads * t, 12)
    q = torch.from_numpy(W.queries(heads * group, seed=13)).cuda()
    ref, got = _both(K, kc, vc, krec, vrec, q, group, t, t, scale)
    assert np.all(np.isfinite(ref))
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    # second call, smaller: 2 KV heads x 777 keys, GQA 4:1, rows strided by 1,000
    heads2, t2, group2, stride2 = 2, 777, 4, 1000
    krec2 = _records(K, kc, heads2 * stride2, 21)
    vrec2 = _records(K, vc, heads2 * stride2, 22)
    q2 = torch.from_numpy(W.queries(heads2 * group2, seed=23)).cuda()
    ref2, got2 = _both(K, kc, vc, krec2, vrec2, q2, group2, t2, stride2, scale)
    assert np.all(np.isfinite(ref2))
    assert np.array_equal(ref2.view(np.uint32), got2.view(np.uint32))


def test_noalloc_mixed_sessions(K):
    """Dense QJL keys with rotor MSE values (other value and key passes)."""
    kc = K.Codec(bits=4, seed=0, mode=K.RQ_DENSE | K.RQ_QJL)
    vc = K.Codec(bits=2, seed=0, mode=K.RQ_MSE)
    t, group = 3000, 16
    krec = _records(K, kc, t, 31)
    vrec = _records(K, vc, t, 32)
    q = torch.from_numpy(W.queries(group, seed=33)).cuda()
    ref, got = _both(K, kc, vc, krec, vrec, q, group, t, t, 0.1)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_noalloc_refuses_sizes_beyond_its_scratch(K):
    kc = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    hq, group, t = 256, 256, 1 << 16          # 64 MB of estimates alone
    assert K.rq_attend_workspace(hq, group, t) > K.RQ_ATTEND_NOALLOC_BYTES
    rec = kc.alloc_record(t, "cuda")
    q = torch.zeros((hq, 128), dtype=torch.float32, device="cuda")
    out = torch.full((hq, 128), 7.0, dtype=torch.float32, device="cuda")
    parts = (rec.codes, rec.norms, rec.signs, rec.rnorms) * 2
    rc = K.lib().rq_attend_noalloc(kc.ctx, kc.ctx, q.data_ptr(), hq, group,
                                   *[p.data_ptr() for p in parts], t, t, ctypes.c_float(0.1), out.data_ptr(), 128,
                                   None)
    assert rc == K.RQ_EINVAL
    assert "RQ_ATTEND_NOALLOC_BYTES" in K.rq_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
