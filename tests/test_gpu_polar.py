"""GPU parity of PolarQuant sessions (RQ_POLAR) against the oracle, through
the C ABI: quantise (angle codes of four levels and the eight half radii),
dequantise, the fused roundtrip and GQA scoring.  Rules in tests/parity.py:
angle codes equal except for points within 1e-6 of a decision ray, radius
halves equal except near rounding midpoints, reconstructions within
1e-5 * ||r^|| and scores within 1e-4 * ||q|| * ||r^|| (r^ the stored radii,
whose norm is the norm of the dequantised vector)."""
import numpy as np
import pytest

import parity as PR
from oracle import polar as PQ
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


@pytest.fixture(scope="module")
def P():
    return PQ.PolarParams(D, 0)


def _words(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n", [1, 65, 1000, 4097])
@pytest.mark.parametrize("in_dtype", [np.float16, np.float32])
def test_polar_quantize_dequantize_roundtrip(K, P, n, in_dtype):
    x = W.gaussian(n, seed=110 + n, dtype=in_dtype)
    x[n // 2] = 0
    if n > 3:
        x[1] *= 40.0                       # norms other than ~sqrt(128)
        x[2] *= 1e-3
    c = K.PolarCodec(seed=0)
    assert c.layout["record_bytes"] == 64
    xt = torch.from_numpy(x).cuda()
    words = c.quantize(xt)
    w2, y32 = c.roundtrip(xt, dtype=torch.float32)
    y16 = c.roundtrip(xt, dtype=torch.float16)[1]
    d32 = c.dequantize(words, dtype=torch.float32)
    d16 = c.dequantize(words, dtype=torch.float16)
    torch.cuda.synchronize()
    gw = _words(words)
    rep = PR.check_polar_words(P, x, gw)
    assert np.array_equal(gw, _words(w2))
    assert np.all(gw[:, 11] >> 16 == 0)
    assert torch.equal(y32, d32)
    assert torch.equal(y16, d32.to(torch.float16)) and torch.equal(d16, y16)
    assert np.all(gw[n // 2] == 0) and torch.all(d32[n // 2] == 0)
    rn = PR.polar_radius_norm(gw)
    PR.compare_recon(d32.cpu().numpy(), PQ.dequantize(P, gw), rn, "polar dequantize")
    assert rep["angles"] == 120 * (n - 1)


def test_polar_keys_65536(K, P):
    """The 65,536 fp16 N(0,1) keys with their norms, fused roundtrip: 64 B
    per key (4.13x over fp16 by the article's 496-bit count)."""
    x = W.keys_65536()
    c = K.PolarCodec(seed=0)
    words, y = c.roundtrip(torch.from_numpy(x).cuda(), dtype=torch.float32)
    torch.cuda.synchronize()
    gw = _words(words)
    rep = PR.check_polar_words(P, x, gw)
    rn = PR.polar_radius_norm(gw)
    rows = W.sample_rows(x.shape[0], 0.05, seed=111)
    PR.compare_recon(y.cpu().numpy()[rows], PQ.dequantize(P, gw[rows]), rn[rows], "polar roundtrip")
    # the dequantised norm is the norm of the stored radii
    yn = np.linalg.norm(y.cpu().numpy().astype(np.float64), axis=1)
    assert np.abs(yn - rn).max() <= 1e-5 * rn.max()
    assert rep["band_count"] <= 1e-4 * rep["angles"] + 3 * np.sqrt(1e-4 * rep["angles"])


@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.float16, torch.float16), (torch.float16, torch.float32),
                                                (torch.float32, torch.float32)])
def test_polar_several_tiles_per_wave(K, P, in_dtype, out_dtype):
    """300,000 keys: every wave of the quantiser, the fused roundtrip and the
    dequantiser walks several 32-vector tiles (the next tile's input is
    fetched during the current one, each tile's output is stored after the
    next tile's input or record has arrived).  The roundtrip's records equal
    pq_quantize's and its output equals pq_dequantize of them, bit for bit;
    rows sampled from the first and the last 65,536 match the oracle."""
    n = 300_000
    c = K.PolarCodec(seed=0)
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((n, D), generator=g, device="cuda").to(in_dtype)
    words, y = c.roundtrip(x, dtype=out_dtype)
    w2 = c.quantize(x)
    d = c.dequantize(words, dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(words, w2)
    assert torch.equal(y, d)
    rows = np.concatenate([W.sample_rows(65536, 1 / 32, seed=120),
                           n - 65536 + W.sample_rows(65536, 1 / 32, seed=121)])
    idx = torch.from_numpy(rows).cuda()
    xs = x[idx].float().cpu().numpy()
    gw = _words(words[idx])
    PR.check_polar_words(P, xs, gw)
    tol = PR.RECON_TOL + (2.0 ** -11 if out_dtype == torch.float16 else 0.0)
    PR.compare_recon(y[idx].float().cpu().numpy(), PQ.dequantize(P, gw), PR.polar_radius_norm(gw),
                     "polar roundtrip sample", tol=tol)


@pytest.mark.parametrize("t,hq,group", [(1, 1, 1), (300, 8, 4), (2049, 32, 8), (640, 40, 40), (777, 66, 33),
                                        (4096, 32, 4)])
def test_polar_score(K, P, t, hq, group):
    kvh = hq // group
    keys = W.gaussian(kvh * t, seed=112, dtype=np.float16)
    q = W.queries(hq, seed=113)
    c = K.PolarCodec(seed=0)
    words = c.quantize(torch.from_numpy(keys).cuda())
    s = c.score(torch.from_numpy(q).cuda(), words, group, t)
    torch.cuda.synchronize()
    gw = _words(words)
    got = s.cpu().numpy()
    qn = np.linalg.norm(q.astype(np.float64), axis=1)[:, None]
    for j in range(kvh):
        rows = slice(j * group, (j + 1) * group)
        kw = gw[j * t:(j + 1) * t]
        ref = PQ.score(P, q[rows].astype(np.float64), kw)
        PR.compare_scores(got[rows], ref, qn[rows], PR.polar_radius_norm(kw)[None, :], "polar scores")


def test_polar_score_strided_heads(K, P):
    """Head j's keys start at record row j * kv_stride; rows beyond t are not read."""
    t, stride, kvh, group = 200, 256, 3, 4
    keys = W.gaussian(kvh * stride, seed=114, dtype=np.float16)
    q = W.queries(kvh * group, seed=115)
    c = K.PolarCodec(seed=0)
    words = c.quantize(torch.from_numpy(keys).cuda())
    out = torch.full((kvh * group, 260), 7.0, device="cuda")
    c.score(torch.from_numpy(q).cuda(), words, group, t, kv_stride=stride, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, t:] == 7.0)
    gw = _words(words)
    qn = np.linalg.norm(q.astype(np.float64), axis=1)[:, None]
    for j in range(kvh):
        rows = slice(j * group, (j + 1) * group)
        kw = gw[j * stride:j * stride + t]
        ref = PQ.score(P, q[rows].astype(np.float64), kw)
        PR.compare_scores(got[rows, :t], ref, qn[rows], PR.polar_radius_norm(kw)[None, :], "strided polar scores")


def test_polar_sessions_are_separate(K):
    c = K.PolarCodec(seed=0)
    r = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    x = torch.from_numpy(W.gaussian(64, seed=116, dtype=np.float16)).cuda()
    rec = r.alloc_record(64)
    with pytest.raises(K.RQError):
        K.rq_quantize(c.ctx, x, K.RQ_F16, 64, 128, rec.codes, rec.norms, rec.signs, rec.rnorms)
    with pytest.raises(K.RQError):
        K.pq_quantize(r.ctx, x, K.RQ_F16, 64, 128, c.alloc_words(64))
    with pytest.raises(K.RQError):
        K.Cache(c, r, layers=1, kv_heads=1)
    # seeds give different Pi, hence different records
    w0 = c.quantize(x)
    w1 = K.PolarCodec(seed=1).quantize(x)
    torch.cuda.synchronize()
    assert not torch.equal(w0, w1)


def test_polar_strided_rows_and_empty_calls(K, P):
    """Row pitches above 128 elements read and write only the first 128;
    n = 0 and t = 0 are no-ops; bad arguments are rejected before any launch."""
    n, ld = 300, 136
    xs = np.full((n, ld), 9.0, dtype=np.float32)
    xs[:, :D] = W.gaussian(n, seed=117, dtype=np.float32)
    c = K.PolarCodec(seed=0)
    xt = torch.from_numpy(xs).cuda()
    words = c.alloc_words(n)
    y = torch.full((n, ld), 5.0, device="cuda")
    K.pq_roundtrip(c.ctx, xt, K.RQ_F32, n, ld, words, y, K.RQ_F32, ld)
    torch.cuda.synchronize()
    gw = _words(words)
    PR.check_polar_words(P, xs[:, :D], gw)
    assert torch.all(y[:, D:] == 5.0)
    ref = c.dequantize(c.quantize(torch.from_numpy(np.ascontiguousarray(xs[:, :D])).cuda()), dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :D], ref)
    # empty calls touch nothing
    w0 = torch.full((1, 16), 3, dtype=torch.int32, device="cuda")
    K.pq_quantize(c.ctx, xt, K.RQ_F32, 0, ld, w0)
    K.pq_dequantize(c.ctx, w0, 0, y, K.RQ_F32, ld)
    s0 = torch.full((2, 4), 1.5, device="cuda")
    q = torch.from_numpy(W.queries(2, seed=118)).cuda()
    K.pq_score(c.ctx, q, 2, 2, w0, 0, 0, s0, 4)
    torch.cuda.synchronize()
    assert torch.all(w0 == 3) and torch.all(s0 == 1.5)
    # argument checks
    with pytest.raises(K.RQError):
        K.pq_quantize(c.ctx, xt, K.RQ_F32, n, 100, words)                  # ld < 128
    with pytest.raises(K.RQError):
        K.pq_roundtrip(c.ctx, xt, K.RQ_F32, n, ld, words, xt, K.RQ_F32, ld)   # x and y overlap
    with pytest.raises(K.RQError):
        K.pq_score(c.ctx, q, 2, 3, words, n, n, s0, 4)                      # hq % group != 0
    with pytest.raises(K.RQError):
        K.pq_score(c.ctx, q, 2, 1, words, 10, 5, torch.empty((2, 10), device="cuda"), 10)   # kv_stride < t
    with pytest.raises(K.RQError):
        K.pq_score(c.ctx, q, 2, 2, words, 10, 10, torch.empty((2, 10), device="cuda"), 8)   # ld < t


@pytest.mark.parametrize("t,kvh,group,vspec", [(777, 2, 4, (3, "mse")), (2049, 4, 8, (3, "qjl")), (100, 1, 40, (4, "dense"))])
def test_attention_over_polar_keys(K, P, t, kvh, group, vspec):
    """rq_attend with PolarQuant keys: end to end against the oracle within
    the bound the score tolerance implies (a score error e moves the
    softmax weights by at most 2 scale e in total), and with the GPU's own
    polar scores within 1e-5 of the largest value coordinate."""
    from oracle import codec as OC
    from oracle import params as OP
    mode = {"mse": OP.MSE, "qjl": OP.QJL, "dense": OP.DENSE}[vspec[1]]
    kc, vc = K.PolarCodec(seed=0), K.Codec(bits=vspec[0], seed=0, mode=mode)
    keys = W.gaussian(kvh * t, seed=119, dtype=np.float16)
    vals = W.gaussian(kvh * t, seed=120, dtype=np.float16)
    q = W.queries(kvh * group, seed=121)
    kw = kc.quantize(torch.from_numpy(keys).cuda())
    vrec = vc.quantize(torch.from_numpy(vals).cuda())
    qd = torch.from_numpy(q).cuda()
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, qd, kw, vrec, group, t, t, scale)
    s = kc.score(qd, kw, group, t)
    torch.cuda.synchronize()
    pv = OP.Params(D, vspec[0], 0, mode)
    gw = _words(kw)
    hv = PR.record_from_host(*vrec.host())
    ref = PQ.attend(P, pv, q.astype(np.float64), gw, hv, group, t, scale)
    got = out.cpu().numpy().astype(np.float64)
    sg = s.cpu().numpy().astype(np.float64)
    for h in range(kvh * group):
        j = h // group
        xv = OC.dequantize(pv, OC._rows(hv, slice(j * t, (j + 1) * t)))
        vmax = np.abs(xv).max()
        rmax = PR.polar_radius_norm(gw[j * t:(j + 1) * t]).max()
        lim = (2e-4 * scale * np.linalg.norm(q[h]) * rmax + 1e-5) * vmax
        assert np.abs(got[h] - ref[h]).max() <= lim, (h, np.abs(got[h] - ref[h]).max() / lim)
        z = scale * sg[h]
        wgt = np.exp(z - z.max())
        assert np.abs(got[h] - (wgt / wgt.sum()) @ xv).max() <= 1e-5 * vmax, h
    # keys must come as word records only
    with pytest.raises(K.RQError):
        K.rq_attend(kc.ctx, vc.ctx, qd, kvh * group, group, kw, vrec.norms, None, None, vrec.codes, vrec.norms,
                    vrec.signs, vrec.rnorms, t, t, scale, 0, 0, out, D)


@pytest.mark.parametrize("t,kvh,group", [(1000, 2, 4), (63, 3, 1), (4097, 1, 8), (200, 2, 32), (130, 1, 40)])
@pytest.mark.parametrize("kspec", ["polar", "rotor+qjl3", "dense2"])
def test_attention_over_polar_values(K, P, t, kvh, group, kspec):
    """rq_attend with PolarQuant values (keys: PolarQuant, rotor with QJL,
    TurboQuant dense): end to end against the oracle within the bound the
    score tolerance implies, and with the GPU's own estimates within 1e-5
    of the largest value coordinate of the decoded values."""
    from oracle import codec as OC
    from oracle import params as OP
    pv = PQ.PolarParams(D, 3)
    vc = K.PolarCodec(seed=3)
    keys = W.gaussian(kvh * t, seed=131, dtype=np.float16)
    vals = W.gaussian(kvh * t, seed=132, dtype=np.float16)
    q = W.queries(kvh * group, seed=133)
    if kspec == "polar":
        kc, pk = K.PolarCodec(seed=0), P
    else:
        bits, mode = (3, OP.QJL) if kspec == "rotor+qjl3" else (2, OP.DENSE)
        kc, pk = K.Codec(bits=bits, seed=0, mode=mode), OP.Params(D, bits, 0, mode)
    kd = kc.quantize(torch.from_numpy(keys).cuda())
    vw = vc.quantize(torch.from_numpy(vals).cuda())
    qd = torch.from_numpy(q).cuda()
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, qd, kd, vw, group, t, t, scale)
    s = kc.score(qd, kd, group, t)
    torch.cuda.synchronize()
    if kspec == "polar":
        hk = _words(kd)
        knorm = PR.polar_radius_norm(hk)
    else:
        hk = PR.record_from_host(*kd.host())
        knorm = OC.half_value(hk.norms)
    hv = _words(vw)
    ref = PQ.attend_values(pk, pv, q.astype(np.float64), hk, hv, group, t, scale)
    got = out.cpu().numpy().astype(np.float64)
    sg = s.cpu().numpy().astype(np.float64)
    for h in range(kvh * group):
        j = h // group
        xv = PQ.dequantize(pv, hv[j * t:(j + 1) * t])
        vmax = np.abs(xv).max()
        kmax = knorm[j * t:(j + 1) * t].max()
        lim = (2e-4 * scale * np.linalg.norm(q[h]) * kmax + 1e-5) * vmax
        assert np.abs(got[h] - ref[h]).max() <= lim, (h, np.abs(got[h] - ref[h]).max() / lim)
        z = scale * sg[h]
        wgt = np.exp(z - z.max())
        assert np.abs(got[h] - (wgt / wgt.sum()) @ xv).max() <= 1e-5 * vmax, h


def test_attention_polar_values_argument_checks(K):
    """PolarQuant values come as word records only."""
    kc, vc = K.Codec(bits=3, seed=0, mode=K.RQ_QJL), K.PolarCodec(seed=3)
    t = 64
    kd = kc.quantize(torch.zeros((t, D), dtype=torch.float16, device="cuda"))
    vw = vc.quantize(torch.zeros((t, D), dtype=torch.float16, device="cuda"))
    qd = torch.zeros((2, D), device="cuda")
    out = torch.empty((2, D), device="cuda")
    ws = torch.empty(K.rq_attend_workspace(2, 2, t) + 256, dtype=torch.uint8, device="cuda")
    base = ws.data_ptr() + ((-ws.data_ptr()) % 256)
    with pytest.raises(K.RQError):
        K.rq_attend(kc.ctx, vc.ctx, qd, 2, 2, kd.codes, kd.norms, kd.signs, kd.rnorms, vw, kd.norms, None, None,
                    t, t, 1.0, base, ws.numel() - 256, out, D)
    K.rq_attend(kc.ctx, vc.ctx, qd, 2, 2, kd.codes, kd.norms, kd.signs, kd.rnorms, vw, None, None, None,
                t, t, 1.0, base, ws.numel() - 256, out, D)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_attention_polar_values_strided_heads(K, P):
    """PolarQuant keys and values of three KV heads 130 rows apart, 100 keys
    each (the rows between heads hold other data)."""
    t, stride, kvh, group = 100, 130, 3, 2
    pv = PQ.PolarParams(D, 3)
    kc, vc = K.PolarCodec(seed=0), K.PolarCodec(seed=3)
    keys = W.gaussian(kvh * stride, seed=141, dtype=np.float16)
    vals = W.gaussian(kvh * stride, seed=142, dtype=np.float16)
    q = W.queries(kvh * group, seed=143)
    kw = kc.quantize(torch.from_numpy(keys).cuda())
    vw = vc.quantize(torch.from_numpy(vals).cuda())
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, torch.from_numpy(q).cuda(), kw, vw, group, t, stride, scale)
    torch.cuda.synchronize()
    hk, hv = _words(kw), _words(vw)
    ref = PQ.attend_values(P, pv, q.astype(np.float64), hk, hv, group, t, scale, stride)
    got = out.cpu().numpy().astype(np.float64)
    for h in range(kvh * group):
        j = h // group
        xv = PQ.dequantize(pv, hv[j * stride:j * stride + t])
        vmax = np.abs(xv).max()
        kmax = PR.polar_radius_norm(hk[j * stride:j * stride + t]).max()
        lim = (2e-4 * scale * np.linalg.norm(q[h]) * kmax + 1e-5) * vmax
        assert np.abs(got[h] - ref[h]).max() <= lim, h


@pytest.mark.parametrize("t,kvh,group", [(40000, 1, 4), (40000, 2, 4)])
def test_attention_polar_values_several_tiles_per_wave(K, P, t, kvh, group):
    """PolarQuant values over 40,000 keys per KV head: with at most 64 key
    slices per (KV head, row block), each wave of the value pass carries its
    sums across two or three 64-key tiles (the loop that reuses the staging
    LDS and the row weights).  Against softmax of the GPU's own estimates
    times the oracle's dequantised values, in float64."""
    pv = PQ.PolarParams(D, 3)
    kc, vc = K.Codec(bits=3, seed=0, mode=K.RQ_QJL), K.PolarCodec(seed=3)
    plan_slices = min(64, 512 // kvh)
    assert -(-t // 64) > 4 * plan_slices          # more tiles than waves: several per wave
    keys = W.gaussian(kvh * t, seed=151, dtype=np.float16)
    vals = W.gaussian(kvh * t, seed=152, dtype=np.float16)
    q = W.queries(kvh * group, seed=153)
    kd = kc.quantize(torch.from_numpy(keys).cuda())
    vw = vc.quantize(torch.from_numpy(vals).cuda())
    qd = torch.from_numpy(q).cuda()
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, qd, kd, vw, group, t, t, scale)
    s = kc.score(qd, kd, group, t)
    torch.cuda.synchronize()
    hv = _words(vw)
    got = out.cpu().numpy().astype(np.float64)
    sg = s.cpu().numpy().astype(np.float64)
    for j in range(kvh):
        xv = PQ.dequantize(pv, hv[j * t:(j + 1) * t])
        vmax = np.abs(xv).max()
        for h in range(j * group, (j + 1) * group):
            z = scale * sg[h]
            wgt = np.exp(z - z.max())
            assert np.abs(got[h] - (wgt / wgt.sum()) @ xv).max() <= 1e-5 * vmax, h
