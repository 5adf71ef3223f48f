"""GPU parity of rq_score (q.k estimates from compressed keys, grouped-query
attention) against the oracle's plain definition, on the GPU's own records."""
import numpy as np
import pytest

import parity as PR
from oracle import codec as OC
from oracle import params as OP
from kv_cache_vector_norm_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _score_case(K, bits, mode, t, hq, group, kv_stride=None, seed=0):
    kv_heads = hq // group
    kv_stride = t if kv_stride is None else kv_stride
    n = kv_stride * (kv_heads - 1) + t
    keys = W.gaussian(n, seed=seed + 21, dtype=np.float16)
    q = W.queries(hq, seed=seed + 22)
    c = K.Codec(bits=bits, seed=0, mode=mode)
    rec = c.quantize(torch.from_numpy(keys).cuda())
    s = c.score(torch.from_numpy(q).cuda(), rec, group, t, kv_stride)
    torch.cuda.synchronize()
    p = OP.Params(D, bits, 0, mode)
    hrec = PR.record_from_host(*rec.host())
    ref = OC.score_gqa(p, q.astype(np.float64), hrec, group, t, kv_stride)
    got = s.cpu().numpy().astype(np.float64)
    qn = np.linalg.norm(q.astype(np.float64), axis=1)
    nh = np.zeros((hq, t))
    for h in range(hq):
        j = h // group
        nh[h] = OC.half_value(hrec.norms[j * kv_stride: j * kv_stride + t])
    lim = PR.SCORE_TOL * qn[:, None] * nh + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= lim), f"worst {np.max(err / lim):.3g} x tolerance"
    return float(np.max(err / lim))


@pytest.mark.parametrize("bits,mode", [(3, OP.QJL), (2, OP.QJL), (5, OP.QJL), (3, OP.MSE), (1, OP.MSE), (4, OP.MSE)])
def test_score_single_head(K, bits, mode):
    _score_case(K, bits, mode, t=1000, hq=8, group=8)


@pytest.mark.parametrize("t,hq,group,stride", [
    (1, 1, 1, None), (63, 4, 4, None), (65, 8, 4, 80), (640, 16, 8, 700), (300, 64, 64, None),
    (257, 100, 100, None), (129, 6, 1, 130), (2048, 32, 4, 2048),
    # around the 16-row (16x16x32) and 32-row tiles: 16 / 17 / 32 / 33 rows a group
    (700, 32, 16, None), (333, 34, 17, None), (200, 64, 32, 256), (96, 33, 33, None)])
def test_score_gqa_shapes(K, t, hq, group, stride):
    _score_case(K, 3, OP.QJL, t, hq, group, stride)


def test_score_65536_keys_64_queries(K):
    """64 queries against 65,536 keys of one head (2-bit codes + QJL)."""
    _score_case(K, 3, OP.QJL, t=65536, hq=64, group=64, seed=1)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("t", [512, 2048, 8192])
def test_needle(K, bits, t):
    """Synthetic needle: the planted key must have the top estimated score."""
    keys, q, idx = W.needle_keys(t, seed=bits * 100 + t)
    c = K.Codec(bits=bits, seed=0, mode=OP.QJL)
    rec = c.quantize(torch.from_numpy(keys).cuda())
    s = c.score(torch.from_numpy(q[None]).cuda(), rec, 1, t)
    torch.cuda.synchronize()
    assert int(torch.argmax(s[0]).item()) == idx


def test_score_rejects_bad_group(K):
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)
    rec = c.alloc_record(10)
    q = torch.zeros((6, D), device="cuda")
    with pytest.raises(K.RQError):
        c.score(q, rec, 4, 10)


@pytest.mark.parametrize("col0,pad", [(0, 4), (4, 8), (1, 6), (3, 1), (2, 2)])
def test_score_into_strided_rows(K, col0, pad):
    """Scores written into columns col0 .. col0 + t of wider rows equal the
    dense output bit for bit, and nothing outside those columns changes
    (rows wider than t, and rows that are not 16-byte aligned)."""
    t, hq, group = 1000, 8, 4
    keys = W.gaussian(2 * t, seed=31, dtype=np.float16)
    q = torch.from_numpy(W.queries(hq, seed=32)).cuda()
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)
    rec = c.quantize(torch.from_numpy(keys).cuda())
    dense = c.score(q, rec, group, t)
    big = torch.full((hq, col0 + t + pad), float("nan"), device="cuda")
    out = big[:, col0:col0 + t]
    c.score(q, rec, group, t, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    assert torch.isnan(big[:, :col0]).all() and torch.isnan(big[:, col0 + t:]).all()
