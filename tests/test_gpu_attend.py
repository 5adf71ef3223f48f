"""GPU parity of rq_attend (decode attention read from compressed keys and
values) against the oracle's plain definition, through the C ABI.

Two comparisons per case:
* against the oracle end to end, within the bound the score tolerance
  implies: a score error of at most 1e-4 ||q|| n^ moves the softmax weights
  by at most 2 scale max|ds| in total, so
      |out - ref| <= (2e-4 scale ||q|| max n^ + 1e-5) max_t |v~_t|;
* against softmax(scale * s_gpu) . dequantize_oracle(v) with the GPU's own
  estimates (rq_score, the same kernel rq_attend runs first), which isolates
  the value pass, the row statistics and the combine: within
  1e-5 max_t |v~_t|.
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
OUT_TOL = 1e-5


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _check(K, kc, vc, kmode, kbits, vmode, vbits, keys, vals, q, group, t, kv_stride, scale):
    """keys/vals: host fp16 arrays laid out for the call; q host fp32."""
    krec = kc.quantize(torch.from_numpy(keys).cuda())
    vrec = vc.quantize(torch.from_numpy(vals).cuda())
    qd = torch.from_numpy(q).cuda()
    out = K.attend(kc, vc, qd, krec, vrec, group, t, kv_stride, scale)
    s_gpu = kc.score(qd, krec, group, t, kv_stride)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    pk, pv = OP.Params(D, kbits, 0, kmode), OP.Params(D, vbits, 0, vmode)
    hk, hv = PR.record_from_host(*krec.host()), PR.record_from_host(*vrec.host())
    ref = OC.attend(pk, pv, q.astype(np.float64), hk, hv, group, t, scale, kv_stride)
    sg = s_gpu.cpu().numpy().astype(np.float64)
    worst = [0.0, 0.0]
    for h in range(q.shape[0]):
        j = h // group
        sl = slice(j * kv_stride, j * kv_stride + t)
        xv = OC.dequantize(pv, OC._rows(hv, sl))
        vmax = np.abs(xv).max() + 1e-30
        nmax = OC.half_value(hk.norms[sl]).max()
        lim = (2e-4 * abs(scale) * np.linalg.norm(q[h]) * nmax + OUT_TOL) * vmax
        e1 = np.abs(got[h] - ref[h]).max() / lim
        z = scale * sg[h]
        p = np.exp(z - z.max())
        ref2 = (p / p.sum()) @ xv
        e2 = np.abs(got[h] - ref2).max() / (OUT_TOL * vmax)
        worst = [max(worst[0], e1), max(worst[1], e2)]
    assert worst[0] <= 1.0 and worst[1] <= 1.0, f"worst {worst} x tolerance"
    return worst


CODECS = [
    ((3, OP.QJL), (2, OP.MSE)),
    ((3, OP.QJL), (3, OP.QJL)),
    ((2, OP.MSE), (4, OP.MSE)),
    ((4, OP.DENSE | OP.QJL), (3, OP.DENSE)),
    ((3, OP.MSE), (3, OP.DENSE | OP.QJL)),
    ((5, OP.QJL), (1, OP.MSE)),
    # value codes of every width with and without signs (1- and 2-bit codes
    # go through the transposed four-key tables, 3- and 4-bit ones by pairs)
    ((3, OP.QJL), (2, OP.QJL)),
    ((3, OP.QJL), (4, OP.QJL)),
    ((2, OP.QJL), (3, OP.MSE)),
    ((3, OP.MSE), (5, OP.DENSE | OP.QJL)),
    ((3, OP.QJL), (2, OP.DENSE | OP.QJL)),
]


@pytest.mark.parametrize("kspec,vspec", CODECS)
@pytest.mark.parametrize("t", [1, 65, 1000])
def test_attend_codecs(K, kspec, vspec, t):
    (kb, km), (vb, vm) = kspec, vspec
    kc, vc = K.Codec(bits=kb, seed=0, mode=km), K.Codec(bits=vb, seed=0, mode=vm)
    hq, group = 8, 4
    keys = W.gaussian(2 * t, seed=70 + t, dtype=np.float16)
    vals = W.gaussian(2 * t, seed=71 + t, dtype=np.float16)
    q = W.queries(hq, seed=72)
    _check(K, kc, vc, km, kb, vm, vb, keys, vals, q, group, t, t, 1 / np.sqrt(D))


@pytest.mark.parametrize("t,hq,group,stride", [(63, 4, 4, None), (130, 6, 1, 140), (257, 16, 8, 300),
                                                (700, 40, 40, None), (64, 64, 32, 64), (2049, 8, 2, None),
                                                (300, 16, 16, None), (129, 48, 16, 140), (200, 9, 3, None),
                                                (150, 17, 17, None)])
def test_attend_shapes(K, t, hq, group, stride):
    stride = t if stride is None else stride
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    kvh = hq // group
    n = stride * (kvh - 1) + t
    keys = W.gaussian(n, seed=73, dtype=np.float16)
    vals = W.gaussian(n, seed=74, dtype=np.float16)
    q = W.queries(hq, seed=75)
    _check(K, kc, vc, OP.QJL, 3, OP.MSE, 3, keys, vals, q, group, t, stride, 1 / np.sqrt(D))


@pytest.mark.parametrize("vspec", [(2, OP.QJL), (4, OP.QJL), (5, OP.DENSE | OP.QJL), (3, OP.QJL)])
def test_attend_several_tiles_per_wave(K, vspec):
    """20,000 keys per KV head (two heads, GQA 4:1): some waves of the value
    pass walk two 64-key tiles, carrying their sums and the staged tables
    from one tile to the next (value codes 1 to 4 bits with signs)."""
    vb, vm = vspec
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=vb, seed=0, mode=vm)
    t, hq, group = 20000, 8, 4
    keys = W.gaussian(2 * t, seed=84, dtype=np.float16)
    vals = W.gaussian(2 * t, seed=85, dtype=np.float16)
    q = W.queries(hq, seed=86)
    _check(K, kc, vc, OP.QJL, 3, vm, vb, keys, vals, q, group, t, t, 1 / np.sqrt(D))


@pytest.mark.parametrize("scale", [0.0, 1.0, -0.3])
def test_attend_scales(K, scale):
    """scale 0 is the plain mean; scale 1 makes the softmax sharp."""
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=2, seed=0, mode=OP.QJL)
    t = 500
    keys = W.gaussian(t, seed=76, dtype=np.float16)
    vals = W.gaussian(t, seed=77, dtype=np.float16)
    q = W.queries(4, seed=78)
    _check(K, kc, vc, OP.QJL, 3, OP.QJL, 2, keys, vals, q, 4, t, t, scale)


def test_attend_lowrank_cache(K):
    """A Qwen2.5-3B-shaped layer (2 KV heads, 16 query heads) of the low-rank
    + outlier generator at 4,096 tokens, K 3-bit + QJL, V 3-bit MSE."""
    k, v, q = [], [], []
    for h in range(2):
        kh, vh, qh = W.lowrank_head(4096, W.cache_seed(9, 0, h), with_query_heads=8, torch=torch)
        k.append(kh)
        v.append(vh)
        q.append(qh)
    keys = torch.cat(k).numpy()
    vals = torch.cat(v).numpy()
    qs = torch.cat(q).numpy().astype(np.float32)
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    _check(K, kc, vc, OP.QJL, 3, OP.MSE, 3, keys, vals, qs, 8, 4096, 4096, 1 / np.sqrt(D))


def test_attend_deterministic_and_workspace(K):
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    t, hq, group = 3000, 16, 4
    krec = kc.quantize(torch.from_numpy(W.gaussian(4 * t, seed=79)).cuda())
    vrec = vc.quantize(torch.from_numpy(W.gaussian(4 * t, seed=80)).cuda())
    q = torch.from_numpy(W.queries(hq, seed=81)).cuda()
    need = K.rq_attend_workspace(hq, group, t)
    ws = torch.full((need + 256,), 0x5A, dtype=torch.uint8, device="cuda")
    a = K.attend(kc, vc, q, krec, vrec, group, t, workspace=ws)
    ws.fill_(0xFF)
    b = K.attend(kc, vc, q, krec, vrec, group, t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attend_rejects_bad_arguments(K):
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    krec, vrec = kc.alloc_record(10), vc.alloc_record(10)
    q = torch.zeros((4, D), device="cuda")
    with pytest.raises(K.RQError):
        K.attend(kc, vc, q, krec, vrec, 4, 0)                       # no keys
    with pytest.raises(K.RQError):
        K.attend(kc, vc, q, krec, vrec, 3, 10)                      # hq % group
    with pytest.raises(K.RQError):
        K.attend(kc, vc, q, krec, krec, 4, 10)                      # value record of the wrong kind
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(K.RQError):
        K.attend(kc, vc, q, krec, vrec, 4, 10, workspace=small)     # workspace too small
    assert K.rq_attend_workspace(4, 3, 10) == -1


def test_attend_at_the_key_limit(K):
    """t = RQ_ATTEND_MAX_KEYS (2^23 keys for one KV head, 4 query rows):
    the output equals softmax(scale * s_gpu) . dequantize(v) evaluated in
    float64 on the device from the GPU's own estimates and dequantised
    values (chunks of 2^20 values), within 1e-5 max |v~|; one key more is
    rejected before any launch."""
    t, group = 1 << 23, 4
    assert K.rq_attend_workspace(4, 4, t) > 0
    kc, vc = K.Codec(bits=3, seed=0, mode=OP.QJL), K.Codec(bits=3, seed=0, mode=OP.MSE)
    g = torch.Generator(device="cuda").manual_seed(82)
    krec = kc.quantize(torch.randn((t, D), generator=g, device="cuda").to(torch.float16))
    vrec = vc.quantize(torch.randn((t, D), generator=g, device="cuda").to(torch.float16))
    q = torch.from_numpy(W.queries(group, seed=83)).cuda()
    scale = 1 / np.sqrt(D)
    out = K.attend(kc, vc, q, krec, vrec, group, t, t, scale)
    s = kc.score(q, krec, group, t).to(torch.float64)
    z = scale * s
    p = torch.exp(z - z.max(dim=1, keepdim=True).values)
    p = p / p.sum(dim=1, keepdim=True)
    ref = torch.zeros((group, D), dtype=torch.float64, device="cuda")
    vmax = 0.0
    step = 1 << 20
    for i in range(0, t, step):
        sub = K.Record(vrec.codes[i:i + step], vrec.norms[i:i + step])
        xv = vc.dequantize(sub, dtype=torch.float32).to(torch.float64)
        ref += p[:, i:i + step] @ xv
        vmax = max(vmax, float(xv.abs().max()))
    torch.cuda.synchronize()
    err = float((out.to(torch.float64) - ref).abs().max())
    assert err <= OUT_TOL * vmax, (err, vmax)
    with pytest.raises(K.RQError):
        K.attend(kc, vc, q, krec, vrec, group, t + 1, t + 1, scale)
    assert K.rq_attend_workspace(4, 4, t + 1) == -1
