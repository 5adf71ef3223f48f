"""GPU parity of QJL-only sessions (one bit per coordinate in total, no MSE
stage: the record is the norm, sign(S x_u) and gamma = ||x_u||) against the
oracle, through the C ABI: quantise, dequantise, roundtrip, scoring and
attention with QJL-only keys."""
import numpy as np
import pytest

import parity as PR
from oracle import codec as OC
from oracle import params as OP
from kv_cache_vector_norm_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128
MODES = [OP.QJL, OP.QJL | OP.DENSE]


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _check_record(p, x, rec):
    codes, norms, signs, rnorms = rec.host()
    assert codes.shape == (x.shape[0], 0)
    orec, diag = OC.quantize(p, x.astype(np.float64))
    PR.compare_halves(norms, diag.n, "norms")
    PR.compare_halves(rnorms, diag.gamma, "gamma")
    PR.compare_signs(p, signs, diag, np.zeros(x.shape[0], dtype=bool))
    return PR.record_from_host(codes, norms, signs, rnorms)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n", [1, 65, 1000])
@pytest.mark.parametrize("in_dtype", [np.float16, np.float32])
def test_qjl1_quantize_dequantize_roundtrip(K, mode, n, in_dtype):
    x = W.gaussian(n, seed=90 + n, dtype=in_dtype)
    x[n // 2] = 0
    c = K.Codec(bits=1, seed=0, mode=mode)
    assert c.layout["record_bytes"] == 20
    xt = torch.from_numpy(x).cuda()
    rec = c.quantize(xt)
    rec2, y32 = c.roundtrip(xt, dtype=torch.float32)
    y16 = c.roundtrip(xt, dtype=torch.float16)[1]
    d32 = c.dequantize(rec, dtype=torch.float32)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, mode)
    hrec = _check_record(p, x, rec)
    for a, b in zip(rec.host(), rec2.host()):
        assert np.array_equal(a, b)
    assert torch.equal(y32, d32)
    assert torch.equal(y16, d32.to(torch.float16))
    assert torch.all(d32[n // 2] == 0)
    PR.compare_recon(d32.cpu().numpy(), OC.dequantize(p, hrec), OC.half_value(hrec.norms), "qjl1 dequantize")


def test_qjl1_65536_keys(K):
    """The 65,536 fp16 N(0,1) keys at one bit: 20 B per key (12.8x)."""
    x = W.keys_65536()
    c = K.Codec(bits=1, seed=0, mode=OP.QJL)
    rec, y = c.roundtrip(torch.from_numpy(x).cuda(), dtype=torch.float32)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, OP.QJL)
    hrec = _check_record(p, x, rec)
    PR.compare_recon(y.cpu().numpy(), OC.dequantize(p, hrec), OC.half_value(hrec.norms), "qjl1 roundtrip")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("t,hq,group", [(1, 1, 1), (300, 8, 4), (2049, 32, 8), (640, 40, 40)])
def test_qjl1_score(K, mode, t, hq, group):
    kvh = hq // group
    keys = W.gaussian(kvh * t, seed=95, dtype=np.float16)
    q = W.queries(hq, seed=96)
    c = K.Codec(bits=1, seed=0, mode=mode)
    rec = c.quantize(torch.from_numpy(keys).cuda())
    s = c.score(torch.from_numpy(q).cuda(), rec, group, t)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, mode)
    hrec = PR.record_from_host(*rec.host())
    ref = OC.score_gqa(p, q.astype(np.float64), hrec, group, t)
    qn = np.linalg.norm(q.astype(np.float64), axis=1)[:, None]
    nh = np.stack([OC.half_value(hrec.norms[(h // group) * t:(h // group + 1) * t]) for h in range(hq)])
    PR.compare_scores(s.cpu().numpy(), ref, qn, nh, "qjl1 scores")


def test_qjl1_keys_in_attention(K):
    t, hq, group = 777, 8, 4
    kc, vc = K.Codec(bits=1, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    keys = W.gaussian(2 * t, seed=97, dtype=np.float16)
    vals = W.gaussian(2 * t, seed=98, dtype=np.float16)
    q = W.queries(hq, seed=99)
    krec = kc.quantize(torch.from_numpy(keys).cuda())
    vrec = vc.quantize(torch.from_numpy(vals).cuda())
    qd = torch.from_numpy(q).cuda()
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, qd, krec, vrec, group, t, t, scale)
    torch.cuda.synchronize()
    pk, pv = OP.Params(D, 1, 0, OP.QJL), OP.Params(D, 3, 0, OP.MSE)
    hk, hv = PR.record_from_host(*krec.host()), PR.record_from_host(*vrec.host())
    ref = OC.attend(pk, pv, q.astype(np.float64), hk, hv, group, t, scale)
    got = out.cpu().numpy()
    for h in range(hq):
        j = h // group
        xv = OC.dequantize(pv, OC._rows(hv, slice(j * t, (j + 1) * t)))
        nmax = OC.half_value(hk.norms[j * t:(j + 1) * t]).max()
        lim = (2e-4 * scale * np.linalg.norm(q[h]) * nmax + 1e-5) * np.abs(xv).max()
        assert np.abs(got[h] - ref[h]).max() <= lim
    # values need an MSE stage
    with pytest.raises(K.RQError):
        K.attend(vc, kc, qd, vrec, krec, group, t)
