"""GPU tests of the paged compressed KV cache (rq_cache_*), through the C ABI.

The cache only moves records (quantised per vector, so position-independent)
into pages and reads them through a page table, so its contents and its
attention must equal the dense path bit for bit: records read back equal
rq_quantize of the same vectors, and rq_cache_attend equals rq_attend over
those dense records (same kernels, same tiles in the same order).  The
current-token variant is checked against the oracle's definition.
"""
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


def _kv(kv_heads, t, seed, dtype=np.float16):
    k = W.gaussian(kv_heads * t, seed=seed, dtype=dtype).reshape(kv_heads, t, D)
    v = W.gaussian(kv_heads * t, seed=seed + 1, dtype=dtype).reshape(kv_heads, t, D)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def _same_record(a, b):
    for x, y in zip(a.host(), b.host()):
        if x is None:
            assert y is None
        else:
            assert np.array_equal(x, y)


@pytest.mark.parametrize("page,kv_heads,group,t0,steps,kspec,vspec,stage", [
    (64, 2, 4, 130, 5, (3, OP.QJL), (3, OP.MSE), 65536),
    (256, 8, 4, 1000, 3, (3, OP.QJL), (2, OP.QJL), 65536),
    (128, 1, 8, 0, 70, (1, OP.QJL), (4, OP.MSE), 65536),
    (64, 4, 2, 700, 2, (4, OP.DENSE | OP.QJL), (3, OP.DENSE), 100),   # chunked prefill
])
def test_cache_matches_dense_path(K, page, kv_heads, group, t0, steps, kspec, vspec, stage):
    kc = K.Codec(bits=kspec[0], seed=0, mode=kspec[1])
    vc = K.Codec(bits=vspec[0], seed=0, mode=vspec[1])
    cache = K.Cache(kc, vc, layers=2, kv_heads=kv_heads, page_tokens=page, max_pages=4096, stage_tokens=stage)
    t = t0 + steps
    seq = cache.open(t)
    kk, vv = _kv(kv_heads, t, 60 + t0)
    if t0:
        cache.append(seq, 1, kk[:, :t0].contiguous(), vv[:, :t0].contiguous())     # bulk prefill
    for i in range(t0, t):
        cache.append(seq, 1, kk[:, i:i + 1].contiguous(), vv[:, i:i + 1].contiguous())   # decode steps
    assert cache.length(seq, 1) == t and cache.length(seq, 0) == 0
    krec = cache.read(seq, 1, 0)
    vrec = cache.read(seq, 1, 1)
    kd = kc.quantize(kk.reshape(-1, D))
    vd = vc.quantize(vv.reshape(-1, D))
    torch.cuda.synchronize()
    _same_record(krec, kd)
    _same_record(vrec, vd)
    hq = kv_heads * group
    q = torch.from_numpy(W.queries(hq, seed=61)).cuda()
    a = cache.attend(seq, 1, q)
    b = K.attend(kc, vc, q, kd, vd, group, t, t)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("t", [0, 1, 300])
def test_cache_attend_with_current_token(K, t):
    kv_heads, group = 2, 4
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    cache = K.Cache(kc, vc, layers=1, kv_heads=kv_heads, page_tokens=64, max_pages=64)
    seq = cache.open(512)
    kk, vv = _kv(kv_heads, max(t, 1), 62)
    if t:
        cache.append(seq, 0, kk[:, :t].contiguous(), vv[:, :t].contiguous())
    kcur = torch.from_numpy(W.gaussian(kv_heads, seed=63, dtype=np.float32)).cuda()
    vcur = torch.from_numpy(W.gaussian(kv_heads, seed=64, dtype=np.float32)).cuda()
    q = torch.from_numpy(W.queries(kv_heads * group, seed=65)).cuda()
    scale = 1 / np.sqrt(D)
    out = cache.attend(seq, 0, q, scale, k_cur=kcur, v_cur=vcur)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    pk, pv = OP.Params(D, 3, 0, OP.QJL), OP.Params(D, 3, 0, OP.MSE)
    if t:
        hk = PR.record_from_host(*cache.read(seq, 0, 0).host())
        hv = PR.record_from_host(*cache.read(seq, 0, 1).host())
    else:
        hk = hv = None
    qh = q.cpu().numpy().astype(np.float64)
    ref = OC.attend_with_current(pk, pv, qh, hk, hv, group, t, scale, kcur.cpu().numpy(), vcur.cpu().numpy())
    for h in range(kv_heads * group):
        j = h // group
        vals = [np.abs(vcur[j].cpu().numpy()).max()]
        nmax = 0.0
        if t:
            vals.append(np.abs(OC.dequantize(pv, OC._rows(hv, slice(j * t, (j + 1) * t)))).max())
            nmax = OC.half_value(hk.norms[j * t:(j + 1) * t]).max()
        lim = (2e-4 * scale * np.linalg.norm(qh[h]) * nmax + 1e-5) * max(vals)
        assert np.abs(got[h] - ref[h]).max() <= lim, (h, np.abs(got[h] - ref[h]).max() / lim)


def test_cache_sequences_share_the_pool(K):
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    layers, kv_heads, page = 2, 2, 64
    cache = K.Cache(kc, vc, layers=layers, kv_heads=kv_heads, page_tokens=page, max_pages=40)
    assert cache.free_pages() == 40
    a = cache.open(300)                     # 5 pages per (layer, head): 20
    assert cache.free_pages() == 20
    b = cache.open(200)                     # 4 pages per (layer, head): 16
    assert cache.free_pages() == 4
    with pytest.raises(K.RQError):
        cache.open(100)                     # needs 8, 4 left
    ka, va = _kv(kv_heads, 300, 66)
    kb, vb = _kv(kv_heads, 200, 67)
    for layer in range(layers):
        cache.append(a, layer, ka[:, :150].contiguous(), va[:, :150].contiguous())
        cache.append(b, layer, kb[:, :200].contiguous(), vb[:, :200].contiguous())
        cache.append(a, layer, ka[:, 150:].contiguous(), va[:, 150:].contiguous())
    # b reserved whole pages: 4 x 64 = 256 tokens, 200 used
    kx, vx = _kv(kv_heads, 57, 70)
    with pytest.raises(K.RQError):
        cache.append(b, 0, kx.contiguous(), vx.contiguous())                 # 257 > 256
    cache.close(a)
    assert cache.free_pages() == 24
    c = cache.open(256)                     # reuses a's pages
    kc_, vc_ = _kv(kv_heads, 256, 68)
    cache.append(c, 1, kc_.contiguous(), vc_.contiguous())
    torch.cuda.synchronize()
    _same_record(cache.read(b, 1, 0), kc.quantize(kb.reshape(-1, D)))
    _same_record(cache.read(c, 1, 1), vc.quantize(vc_.reshape(-1, D)))


def test_cache_rejects_bad_use(K):
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    with pytest.raises(K.RQError):
        K.Cache(kc, vc, layers=1, kv_heads=2, page_tokens=100)              # not a power of two
    with pytest.raises(K.RQError):
        K.Cache(kc, K.Codec(bits=1, seed=0, mode=OP.QJL), layers=1, kv_heads=2)   # values need MSE bits
    cache = K.Cache(kc, vc, layers=1, kv_heads=2, page_tokens=64, max_pages=8)
    seq = cache.open(64)
    q = torch.zeros((4, D), device="cuda")
    with pytest.raises(K.RQError):
        cache.attend(seq, 0, q)                                            # nothing cached, no current token
    with pytest.raises(K.RQError):
        cache.attend(seq, 1, q)                                            # no such layer
    kk, vv = _kv(2, 65, 69)
    with pytest.raises(K.RQError):
        cache.append(seq, 0, kk.contiguous(), vv.contiguous())            # 65 > 64 reserved


@pytest.mark.parametrize("layers,l0,nl,kv_heads,group,t0,steps,kspec,vspec,stage,cur", [
    (4, 1, 3, 2, 8, 130, 3, (3, OP.QJL), (3, OP.MSE), 65536, True),
    (36, 0, 36, 2, 8, 600, 2, (3, OP.QJL), (3, OP.MSE), 65536, True),     # Qwen2.5-3B-shaped step
    (3, 0, 3, 4, 2, 300, 2, (1, OP.QJL), (4, OP.MSE), 65536, False),
    (2, 0, 2, 2, 4, 200, 1, (4, OP.DENSE | OP.QJL), (3, OP.DENSE), 128, True),   # chunked staging
])
def test_all_layers_calls_equal_per_layer_calls(K, layers, l0, nl, kv_heads, group, t0, steps, kspec, vspec, stage,
                                                cur):
    """rq_cache_append_layers / rq_cache_attend_layers over layers l0 .. l0+nl-1
    give the same records and the same attention, bit for bit, as one
    rq_cache_append / rq_cache_attend per layer on a twin cache."""
    kc = K.Codec(bits=kspec[0], seed=0, mode=kspec[1])
    vc = K.Codec(bits=vspec[0], seed=0, mode=vspec[1])
    mk = lambda: K.Cache(kc, vc, layers=layers, kv_heads=kv_heads, page_tokens=64, max_pages=4096,
                         stage_tokens=stage)
    a, b = mk(), mk()
    t = t0 + steps
    sa, sb = a.open(t + 64), b.open(t + 64)
    kk = torch.stack([_kv(kv_heads, t, 80 + l)[0] for l in range(nl)])
    vv = torch.stack([_kv(kv_heads, t, 80 + l)[1] for l in range(nl)])
    hq = kv_heads * group
    scale = 1 / np.sqrt(D)
    chunks = [(0, t0)] + [(i, i + 1) for i in range(t0, t)]
    for step, (i0, i1) in enumerate(chunks):
        a.append_layers(sa, l0, kk[:, :, i0:i1].contiguous(), vv[:, :, i0:i1].contiguous())
        for l in range(nl):
            b.append(sb, l0 + l, kk[l, :, i0:i1].contiguous(), vv[l, :, i0:i1].contiguous())
        q = torch.from_numpy(W.queries(nl * hq, seed=90 + step)).cuda().reshape(nl, hq, D)
        kcur = vcur = None
        if cur:
            kcur = torch.from_numpy(W.gaussian(nl * kv_heads, seed=91 + step, dtype=np.float32)).cuda()
            vcur = torch.from_numpy(W.gaussian(nl * kv_heads, seed=92 + step, dtype=np.float32)).cuda()
            kcur, vcur = kcur.reshape(nl, kv_heads, D), vcur.reshape(nl, kv_heads, D)
        got = a.attend_layers(sa, l0, q, scale, k_cur=kcur, v_cur=vcur)
        ref = torch.cat([b.attend(sb, l0 + l, q[l].contiguous(), scale,
                                  k_cur=None if kcur is None else kcur[l].contiguous(),
                                  v_cur=None if vcur is None else vcur[l].contiguous()) for l in range(nl)])
        torch.cuda.synchronize()
        assert torch.equal(got, ref), step
    for l in range(layers):
        assert a.length(sa, l) == (t if l0 <= l < l0 + nl else 0)
    for l in range(l0, l0 + nl):
        for which in (0, 1):
            _same_record(a.read(sa, l, which), b.read(sb, l, which))


def test_all_layers_calls_reject_bad_use(K):
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    cache = K.Cache(kc, vc, layers=3, kv_heads=2, page_tokens=64, max_pages=64)
    seq = cache.open(128)
    kk, vv = _kv(2, 10, 95)
    k3, v3 = torch.stack([kk] * 3), torch.stack([vv] * 3)
    with pytest.raises(K.RQError):
        cache.append_layers(seq, 1, k3.contiguous(), v3.contiguous())        # layers 1..3 of 3
    cache.append(seq, 0, kk.contiguous(), vv.contiguous())
    q = torch.from_numpy(W.queries(3 * 8, seed=96)).cuda().reshape(3, 8, D)
    with pytest.raises(K.RQError):
        cache.attend_layers(seq, 0, q)                                       # layer 0 holds 10, the rest 0
    with pytest.raises(K.RQError):
        cache.append_layers(seq, 0, k3.contiguous(), v3.contiguous())        # unequal lengths
    cache.append_layers(seq, 1, k3[:2].contiguous(), v3[:2].contiguous())    # now all hold 10
    out = cache.attend_layers(seq, 0, q)
    torch.cuda.synchronize()
    assert out.shape == (24, D) and torch.isfinite(out).all()
    with pytest.raises(K.RQError):
        cache.attend_layers(seq, 0, q[:, :7].contiguous())                   # hq not a multiple of kv_heads
