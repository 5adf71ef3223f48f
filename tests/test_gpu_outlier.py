"""GPU parity of outlier-channel separation for QJL-only keys against the
oracle (oracle/outlier.py), through the C ABI: the channel choice per head,
the record (inlier sketch + exact outlier halves), dequantisation and
grouped-query scoring, on keys with planted x10 channels and on the
low-rank + outlier generator of the model-shaped caches.

Rules (tests/parity.py): norms and gamma as halves, sign bits outside the
1e-6 band as for the plain QJL-only codec (the oracle quantises the same
inlier rows); outlier halves and reconstructed outlier channels bit-exact;
the other channels within 1e-5 n^; scores within 1e-4 ||q|| (n^ + ||o^||),
the key's norm being split between its inlier part (n^) and its outlier
values."""
import numpy as np
import pytest

import parity as PR
from oracle import codec as OC
from oracle import outlier as OO
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


def _planted(heads, rows, seed, k=4, dtype=np.float16):
    """heads x rows keys, each head with its own k channels scaled by 10."""
    rng = np.random.default_rng(seed)
    x = W.gaussian(heads * rows, seed=seed).astype(np.float64)
    chans = np.stack([np.sort(rng.choice(D, size=k, replace=False)) for _ in range(heads)])
    for h in range(heads):
        x[h * rows:(h + 1) * rows, chans[h]] *= 10.0
    return x.astype(np.float16).astype(dtype), chans


def _select(K, x, heads, rows, k):
    xd = torch.from_numpy(x).cuda()
    ch = torch.zeros((max(heads, 1), max(k, 1)), dtype=torch.uint8, device="cuda")
    K.rq_outlier_channels(xd, K.RQ_F16 if x.dtype == np.float16 else K.RQ_F32, heads, rows, x.shape[1], k, ch)
    torch.cuda.synchronize()
    return ch[:heads, :k].cpu().numpy().astype(np.int64)


def _quantize(K, c, x, head_rows, k, chans):
    n = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    rec = c.alloc_record(n, "cuda")
    out = torch.zeros((n, max(k, 1)), dtype=torch.int16, device="cuda")
    ch = torch.from_numpy(np.ascontiguousarray(chans.astype(np.uint8))).cuda() if k else None
    K.rq_quantize_outliers(c.ctx, xd, K.RQ_F16 if x.dtype == np.float16 else K.RQ_F32, n, x.shape[1], head_rows, k,
                           ch, rec.norms, rec.signs, rec.rnorms, out if k else None)
    return rec, out, ch


def _check(p, x, head_rows, chans, rec, out):
    """Record vs the oracle's quantisation of the same rows and channels
    (a ragged last head is padded with zero rows for the oracle and cut off
    again).  Returns the GPU record as an oracle Record and its outlier
    halves."""
    n, k = x.shape[0], chans.shape[1]
    _, norms, signs, rnorms = rec.host()
    rows = chans.shape[0] * head_rows
    xp = np.concatenate([x.astype(np.float64), np.zeros((rows - n, D))])
    _, oout, _ = OO.quantize_heads(p, xp, head_rows, chans)
    xin = xp.copy()
    for h in range(chans.shape[0]):
        xin[h * head_rows:(h + 1) * head_rows][:, chans[h]] = 0.0
    _, diag = OC.quantize(p, xin[:n])
    PR.compare_halves(norms, diag.n, "inlier norms")
    PR.compare_halves(rnorms, diag.gamma, "gamma")
    PR.compare_signs(p, signs, diag, np.zeros(n, dtype=bool))
    got_out = out.cpu().numpy().view(np.uint16)[:, :k]
    assert np.array_equal(got_out, oout[:n])
    return PR.record_from_host(np.zeros((n, 0), np.uint32), norms, signs, rnorms), got_out


def test_channel_choice_per_head(K):
    for dtype in (np.float16, np.float32):
        x, planted = _planted(5, 999, seed=11, dtype=dtype)
        got = _select(K, x, 5, 999, 4)
        assert np.array_equal(got, planted)
        assert np.array_equal(got, OO.select_channels_heads(x.astype(np.float64), 999, 4))
        # other k: the oracle's choice wherever its mean |x| leaves a clear gap at the cut
        for k in (1, 7, 16):
            got = _select(K, x, 5, 999, k)
            for h in range(5):
                m = np.mean(np.abs(x[h * 999:(h + 1) * 999].astype(np.float64)), axis=0)
                srt = np.sort(m)[::-1]
                ref = OO.select_channels(x[h * 999:(h + 1) * 999], k)
                if srt[k - 1] - srt[k] > 1e-5 * srt[k - 1]:
                    assert np.array_equal(got[h], ref)
                assert np.all(np.diff(got[h]) > 0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,head_rows", [(65, 65), (1000, 300), (4096, 1024)])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_quantize_dequantize(K, mode, n, head_rows, dtype):
    heads = -(-n // head_rows)
    x, planted = _planted(heads, head_rows, seed=n + head_rows, dtype=dtype)
    x = x[:n]
    c = K.Codec(bits=1, seed=0, mode=mode)
    rec, out, ch = _quantize(K, c, x, head_rows, 4, planted)
    y = torch.full((n, D), float("nan"), dtype=torch.float32, device="cuda")
    y16 = torch.full((n, D), float("nan"), dtype=torch.float16, device="cuda")
    K.rq_dequantize_outliers(c.ctx, rec.norms, rec.signs, rec.rnorms, out, n, head_rows, 4, ch, y, K.RQ_F32, D)
    K.rq_dequantize_outliers(c.ctx, rec.norms, rec.signs, rec.rnorms, out, n, head_rows, 4, ch, y16, K.RQ_F16, D)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, mode)
    hrec, got_out = _check(p, x, head_rows, planted, rec, out)
    ref = np.concatenate([OO.dequantize(p, OC._rows(hrec, slice(h * head_rows, min(n, (h + 1) * head_rows))),
                                        got_out[h * head_rows:min(n, (h + 1) * head_rows)], planted[h])
                          for h in range(heads)])
    got = y.cpu().numpy().astype(np.float64)
    for h in range(heads):
        rows = slice(h * head_rows, min(n, (h + 1) * head_rows))
        assert np.array_equal(got[rows][:, planted[h]], x[rows][:, planted[h]].astype(np.float16).astype(np.float64))
    PR.compare_recon(got, ref, OC.half_value(hrec.norms), "outlier dequantize")
    assert torch.equal(y16, y.to(torch.float16))


def test_zero_channels_equal_the_plain_codec(K):
    x = W.gaussian(500, seed=21, dtype=np.float16)
    c = K.Codec(bits=1, seed=0, mode=OP.QJL)
    rec, _, _ = _quantize(K, c, x, 500, 0, np.zeros((1, 0), np.int64))
    ref = c.quantize(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    for a, b in zip(rec.host()[1:], ref.host()[1:]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("t,hq,group,k", [(1, 1, 1, 4), (300, 8, 4, 4), (2049, 32, 8, 16), (640, 40, 40, 3),
                                          (1000, 128, 64, 5)])
def test_score(K, mode, t, hq, group, k):
    kvh = hq // group
    stride = t + 7
    x, planted = _planted(kvh, stride, seed=31 + t, k=k)
    q = W.queries(hq, seed=32).astype(np.float64)
    for h in range(hq):
        q[h, planted[h // group]] *= 10.0
    q = q.astype(np.float32)
    c = K.Codec(bits=1, seed=0, mode=mode)
    rec, out, ch = _quantize(K, c, x, stride, k, planted)
    s = torch.full((hq, t), float("nan"), dtype=torch.float32, device="cuda")
    K.rq_score_outliers(c.ctx, torch.from_numpy(q).cuda(), hq, group, rec.norms, rec.signs, rec.rnorms, out, k, ch, t,
                        stride, s, t)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, mode)
    hrec, got_out = _check(p, x, stride, planted, rec, out)
    ref = OO.score_gqa(p, q.astype(np.float64), hrec, got_out, planted, group, t, stride)
    qn = np.linalg.norm(q.astype(np.float64), axis=1)[:, None]
    kn = np.stack([OC.half_value(hrec.norms[(h // group) * stride:(h // group) * stride + t])
                   + np.linalg.norm(OC.half_value(got_out[(h // group) * stride:(h // group) * stride + t]), axis=1)
                   for h in range(hq)])
    PR.compare_scores(s.cpu().numpy(), ref, qn, kn, "outlier scores")


def test_qwen_shaped_keys(K):
    """Keys of a few (layer, KV head) blocks of the Qwen2.5-3B-shaped cache
    generator (rank 16 + noise + four x10 channels): the choice finds the
    planted channels, and records and GQA scores (8 query rows per head)
    match the oracle."""
    spec = W.QWEN25_3B
    T, group = 4096, spec["q_heads"] // spec["kv_heads"]
    ks, qs = [], []
    for layer in range(2):
        for h in range(spec["kv_heads"]):
            k, _, q = W.lowrank_head(T, W.cache_seed(1, layer, h), with_query_heads=group, torch=torch)
            ks.append(k.numpy())
            qs.append(q.numpy())
    x = np.concatenate(ks)
    q = np.concatenate(qs).astype(np.float32)
    heads = len(ks)
    got = _select(K, x, heads, T, 4)
    assert np.array_equal(got, OO.select_channels_heads(x.astype(np.float64), T, 4))
    c = K.Codec(bits=1, seed=0, mode=OP.QJL)
    rec, out, ch = _quantize(K, c, x, T, 4, got)
    s = torch.empty((heads * group, T), dtype=torch.float32, device="cuda")
    K.rq_score_outliers(c.ctx, torch.from_numpy(q).cuda(), heads * group, group, rec.norms, rec.signs, rec.rnorms,
                        out, 4, ch, T, T, s, T)
    torch.cuda.synchronize()
    p = OP.Params(D, 1, 0, OP.QJL)
    hrec, got_out = _check(p, x, T, got, rec, out)
    ref = OO.score_gqa(p, q.astype(np.float64), hrec, got_out, got, group, T)
    qn = np.linalg.norm(q.astype(np.float64), axis=1)[:, None]
    kn = np.stack([OC.half_value(hrec.norms[(h // group) * T:(h // group + 1) * T])
                   + np.linalg.norm(OC.half_value(got_out[(h // group) * T:(h // group + 1) * T]), axis=1)
                   for h in range(heads * group)])
    PR.compare_scores(s.cpu().numpy(), ref, qn, kn, "qwen-shaped outlier scores")


def test_argument_checks(K):
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)          # not QJL-only
    rec = c.alloc_record(64, "cuda")
    x = torch.zeros((64, D), dtype=torch.float16, device="cuda")
    out = torch.zeros((64, 4), dtype=torch.int16, device="cuda")
    ch = torch.zeros((1, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(K.RQError):
        K.rq_quantize_outliers(c.ctx, x, K.RQ_F16, 64, D, 64, 4, ch, rec.norms, rec.signs, rec.rnorms, out)
    c1 = K.Codec(bits=1, seed=0, mode=OP.QJL)
    r1 = c1.alloc_record(64, "cuda")
    with pytest.raises(K.RQError):      # k beyond the limit
        K.rq_quantize_outliers(c1.ctx, x, K.RQ_F16, 64, D, 64, 17, ch, r1.norms, r1.signs, r1.rnorms, out)
    with pytest.raises(K.RQError):      # k > 0 without arrays
        K.rq_quantize_outliers(c1.ctx, x, K.RQ_F16, 64, D, 64, 4, None, r1.norms, r1.signs, r1.rnorms, None)
    with pytest.raises(K.RQError):
        K.rq_outlier_channels(x, K.RQ_F16, 1, 0, D, 4, ch)
