"""GPU parity at the shapes of the pages' workloads, through the C ABI.

* 262,144 fp16 N(0,1) keys: the TurboQuant dense path at 2/3/4 bits with and
  without QJL (hyper.ai Algorithms 1 and 2), and the rotor path on the same
  keys (README "MSE Quality");
* a Qwen2.5-3B-shaped K/V cache (36 layers x 2 KV heads x 32,768 tokens,
  16 query heads, GQA 8:1; README "Background", "Real Model Validation") and
  a Llama-3.1-8B-shaped one (32 layers x 8 KV heads x 131,072 tokens, 32
  query heads, GQA 4:1; PolarQuant article on the KV-cache problem), both
  from the low-rank + outlier generator, quantised in bulk with 3 bits
  (2-bit codes + QJL) and scored for one decode step.

At these sizes the float64 oracle checks seeded samples of rows (every
output of a sampled row is compared); every output is also checked at full
size against properties that hold at any size: the roundtrip output equals
the dequantisation of its own record bit for bit, each score equals the
inner product of its query with the dequantised key (the estimator is that
inner product by construction), the bulk call equals per-layer calls, and
the MSE-only distortion of N(0,1) keys sits at the Lloyd-Max values.
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
DEV = "cuda"


def _sync():
    if DEV == "cuda":
        torch.cuda.synchronize()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _gather(rec, idx):
    """Host copies of the record rows at the given indices."""
    it = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(DEV)

    def g(t, dt):
        return None if t is None else t.index_select(0, it).cpu().numpy().view(dt)
    return g(rec.codes, np.uint32), g(rec.norms, np.uint16), g(rec.signs, np.uint32), g(rec.rnorms, np.uint16)


def _nhat_dev(norms):
    return norms.view(torch.float16).to(torch.float64)


def _check_score_property(codec, q, rec, scores, group, t):
    """scores[h, i] == <q_h, dequant(k_i)> within SCORE_TOL * ||q_h|| * n^_i,
    for hq query heads over hq / group KV heads of t keys each (contiguous)."""
    xt = codec.dequantize(rec, dtype=torch.float32).to(torch.float64)
    nh = _nhat_dev(rec.norms)
    hq = q.shape[0]
    qd = q.to(torch.float64)
    qn = torch.linalg.norm(qd, dim=1)
    worst = 0.0
    for j in range(hq // group):
        sl = slice(j * t, (j + 1) * t)
        ref = qd[j * group:(j + 1) * group] @ xt[sl].T
        lim = PR.SCORE_TOL * qn[j * group:(j + 1) * group, None] * nh[None, sl] + 1e-30
        ratio = (scores[j * group:(j + 1) * group].to(torch.float64) - ref).abs() / lim
        worst = max(worst, float(ratio.max()))
    assert worst <= 1.0, f"score vs dequantised key: worst {worst:.3g} x tolerance"
    return worst


def _check_sampled_scores(p, q_host, scores, rec, rows, kv_heads, t, group):
    """Oracle scores of sampled keys against all query heads of their group.

    `rows` index the K records laid out [layer][kv_head][token];
    `scores` is [layers, q_heads, t] on the GPU."""
    layer = rows // (kv_heads * t)
    head = (rows // t) % kv_heads
    tok = rows % t
    codes, norms, signs, rnorms = _gather(rec, rows)
    li = torch.from_numpy(layer).to(DEV)[:, None]
    hi = torch.from_numpy(head * group).to(DEV)[:, None] + torch.arange(group, device=DEV)[None, :]
    ti = torch.from_numpy(tok).to(DEV)[:, None]
    got = scores[li, hi, ti].cpu().numpy().astype(np.float64)          # [m, group]
    worst = 0.0
    keys = layer * kv_heads + head
    for key in np.unique(keys):
        sel = keys == key
        l, j = divmod(int(key), kv_heads)
        sub = OC.Record(codes[sel], norms[sel], signs[sel] if signs is not None else None,
                        rnorms[sel] if rnorms is not None else None)
        qh = q_host[l, j * group:(j + 1) * group].astype(np.float64)
        ref = OC.score(p, qh, sub)                                      # [group, m_sel]
        qn = np.linalg.norm(qh, axis=1)[:, None]
        worst = max(worst, PR.compare_scores(got[sel].T, ref, qn, OC.half_value(norms[sel])[None, :],
                                             f"layer {l} kv head {j}"))
    return worst


# ------------------------------------------- 262,144 keys, dense sweep ----
N_262144 = 262144
MODES_262144 = ([(b, OP.DENSE) for b in (2, 3, 4)] + [(b, OP.DENSE | OP.QJL) for b in (2, 3, 4, 5)]
            + [(b, OP.MSE) for b in (2, 3, 4)] + [(3, OP.QJL)])
# Unit-vector distortion of the Lloyd-Max codebooks (README "MSE Quality";
# hyper.ai Theorem 1 table) at 2/3/4 bits.
LLOYD_MAX_MSE = {2: 0.1160, 3: 0.0340, 4: 0.0093}


@pytest.fixture(scope="module")
def keys_262144_fixture(K):
    x = W.keys_262144()
    return x, torch.from_numpy(x).to(DEV)


@pytest.mark.parametrize("bits,mode", MODES_262144)
def test_262144_keys_sweep(K, keys_262144_fixture, bits, mode):
    x, xd = keys_262144_fixture
    print(f"262,144-key sweep bits={bits} mode={mode}", flush=True)
    c = K.Codec(bits=bits, seed=0, mode=mode)
    rec, y = c.roundtrip(xd, dtype=torch.float32)
    d = c.dequantize(rec, dtype=torch.float32)
    _sync()
    assert torch.equal(y, d)
    if not mode & OP.QJL:
        xs = xd.to(torch.float64)
        rel = (((xs - y.to(torch.float64)) ** 2).sum(1) / (xs ** 2).sum(1)).mean().item()
        assert abs(rel - LLOYD_MAX_MSE[bits]) < 0.01 * LLOYD_MAX_MSE[bits] + 2e-4, rel
    idx = W.sample_rows(N_262144, 1 / 16, seed=100 + 10 * bits + mode)
    codes, norms, signs, rnorms = _gather(rec, idx)
    p = OP.Params(D, bits, 0, mode)
    PR.check_records(p, x[idx], codes, norms, signs, rnorms)
    hrec = PR.record_from_host(codes, norms, signs, rnorms)
    PR.compare_recon(y[torch.from_numpy(idx).to(DEV)].cpu().numpy(), OC.dequantize(p, hrec),
                     OC.half_value(norms), "dequantize")


# ------------------------------------------------- model-shaped caches ----
def _bulk(K, spec, seed):
    """Generate the cache on the GPU, quantise K and V of every layer in one
    call, then score one decode step per layer.  Records are laid out
    [K|V][layer][kv_head][token]."""
    L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
    group = HQ // H
    print(f"{spec['name']}: generating {2 * L * H * T} vectors", flush=True)
    kv, q = W.kv_cache(spec, device=DEV, base_seed=seed, torch=torch)
    flat = kv.view(-1, D)
    assert flat.shape[0] == 2 * L * H * T and q.shape == (L, HQ, D)
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)
    rec = c.quantize(flat)
    scores = torch.empty((L, HQ, T), dtype=torch.float32, device=DEV)
    per_layer = H * T
    for layer in range(L):
        sl = slice(layer * per_layer, (layer + 1) * per_layer)
        sub = K.Record(rec.codes[sl], rec.norms[sl], rec.signs[sl], rec.rnorms[sl])
        c.score(q[layer], sub, group, T, T, out=scores[layer])
    _sync()
    print(f"{spec['name']}: quantised and scored", flush=True)
    return dict(spec=spec, codec=c, flat=flat, q=q, q_host=q.cpu().numpy(), rec=rec, scores=scores,
                group=group, p=OP.Params(D, 3, 0, OP.QJL))


def _layer_record(K, st, which, layer):
    spec = st["spec"]
    per_layer = spec["kv_heads"] * spec["tokens"]
    base = (which * spec["layers"] + layer) * per_layer
    sl = slice(base, base + per_layer)
    r = st["rec"]
    return K.Record(r.codes[sl], r.norms[sl], r.signs[sl], r.rnorms[sl]), sl


def _check_sample(st, rows, dequant=False):
    p = st["p"]
    codes, norms, signs, rnorms = _gather(st["rec"], rows)
    it = torch.from_numpy(rows).to(DEV)
    x = st["flat"].index_select(0, it).cpu().numpy()
    _, _, excl, rep = PR.check_records(p, x, codes, norms, signs, rnorms)
    if dequant:
        sub = st["codec"].dequantize(type(st["rec"])(*(None if a is None else a.index_select(0, it) for a in
                                                        (st["rec"].codes, st["rec"].norms, st["rec"].signs,
                                                         st["rec"].rnorms))), dtype=torch.float32)
        PR.compare_recon(sub.cpu().numpy(), OC.dequantize(p, PR.record_from_host(codes, norms, signs, rnorms)),
                         OC.half_value(norms), "dequantize")
    spec = st["spec"]
    n_k = spec["layers"] * spec["kv_heads"] * spec["tokens"]
    k_rows = rows[rows < n_k]
    worst = _check_sampled_scores(p, st["q_host"], st["scores"], st["rec"], k_rows, spec["kv_heads"],
                                  spec["tokens"], st["group"])
    return rep, worst


# Qwen2.5-3B shape: 36 x 2 x 32,768 x 128, K and V (4,718,592 vectors).
@pytest.fixture(scope="module")
def qwen(K):
    st = _bulk(K, W.QWEN25_3B, seed=3)
    yield st
    st.clear()
    if DEV == "cuda":
        torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_qwen_cache_sample(K, qwen, part):
    """A seeded 2% of all K and V rows (a quarter per case) against the oracle:
    codes, norms, signs, residual norms, dequantisation, and the 8 query heads'
    scores of every sampled key."""
    n = qwen["flat"].shape[0]
    rows = np.array_split(W.sample_rows(n, 0.02, seed=5), 4)[part]
    print(f"qwen sample part {part}: {rows.size} rows", flush=True)
    _check_sample(qwen, rows, dequant=(part == 0))


def test_qwen_scores_full(K, qwen):
    """All 18,874,368 scores of the decode step against q . dequant(k)."""
    spec = qwen["spec"]
    for layer in range(spec["layers"]):
        rec, _ = _layer_record(K, qwen, 0, layer)
        _check_score_property(qwen["codec"], qwen["q"][layer], rec, qwen["scores"][layer], qwen["group"],
                              spec["tokens"])


def test_qwen_bulk_equals_per_layer(K, qwen):
    """One call over the whole cache writes the same bytes as a call per layer."""
    c = qwen["codec"]
    for which, layer in ((0, 0), (0, 17), (1, 35)):
        bulk, sl = _layer_record(K, qwen, which, layer)
        own = c.quantize(qwen["flat"][sl])
        _sync()
        for a, b in zip((bulk.codes, bulk.norms, bulk.signs, bulk.rnorms),
                        (own.codes, own.norms, own.signs, own.rnorms)):
            assert torch.equal(a, b)


# Llama-3.1-8B shape: 32 x 8 x 131,072 x 128, K and V (67,108,864 vectors,
# 17.2 GB of fp16), quantised in one call.
@pytest.fixture(scope="module")
def llama(K):
    st = _bulk(K, W.LLAMA31_8B, seed=4)
    yield st
    st.clear()
    if DEV == "cuda":
        torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(6))
def test_llama_cache_sample(K, llama, part):
    """A seeded 1% of all K and V rows (671,089; a sixth per case) against the
    oracle, with the 4 query heads' scores of every sampled key."""
    n = llama["flat"].shape[0]
    rows = np.array_split(W.sample_rows(n, 0.01, seed=6), 6)[part]
    print(f"llama sample part {part}: {rows.size} rows", flush=True)
    _check_sample(llama, rows, dequant=(part == 0))


def test_llama_scores_full(K, llama):
    """All 134,217,728 decode scores (32 layers) against q . dequant(k)."""
    spec = llama["spec"]
    for layer in range(spec["layers"]):
        rec, _ = _layer_record(K, llama, 0, layer)
        _check_score_property(llama["codec"], llama["q"][layer], rec, llama["scores"][layer], llama["group"],
                              spec["tokens"])


@pytest.mark.parametrize("which", ["qwen", "llama"])
def test_decode_step_in_one_call(K, which, request):
    """The whole decode step as one rq_score call: query row l * HQ + h reads
    KV head l * H + h / group, i.e. layer l's records, so the scores equal the
    per-layer calls bit for bit."""
    st = request.getfixturevalue(which)
    spec = st["spec"]
    L, HQ, T = spec["layers"], spec["q_heads"], spec["tokens"]
    n_k = L * spec["kv_heads"] * T
    r = st["rec"]
    krec = K.Record(r.codes[:n_k], r.norms[:n_k], r.signs[:n_k], r.rnorms[:n_k])
    out = torch.empty((L * HQ, T), dtype=torch.float32, device=DEV)
    st["codec"].score(st["q"].view(L * HQ, D), krec, st["group"], T, T, out=out)
    _sync()
    assert torch.equal(out.view(L, HQ, T), st["scores"])


@pytest.mark.parametrize("which,nrows", [("qwen", 4), ("llama", 3)])
def test_attention_decode_step(K, which, nrows, request):
    """Decode attention of the whole cache in one rq_attend call (keys and
    values of every layer, GQA), sampled query rows against the oracle:
    end to end within the bound the score tolerance implies, and with the
    GPU's own estimates within 1e-5 of the largest value coordinate."""
    st = request.getfixturevalue(which)
    spec = st["spec"]
    L, H, HQ, T = spec["layers"], spec["kv_heads"], spec["q_heads"], spec["tokens"]
    g = st["group"]
    n_k = L * H * T
    r = st["rec"]
    krec = K.Record(r.codes[:n_k], r.norms[:n_k], r.signs[:n_k], r.rnorms[:n_k])
    vrec = K.Record(r.codes[n_k:], r.norms[n_k:], r.signs[n_k:], r.rnorms[n_k:])
    q = st["q"].view(L * HQ, D)
    scale = 1 / np.sqrt(D)
    out = K.attend(st["codec"], st["codec"], q, krec, vrec, g, T, T, scale)
    _sync()
    p = st["p"]
    rows = np.sort(np.random.Generator(np.random.PCG64(7)).choice(L * HQ, size=nrows, replace=False))
    got = out[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    for i, row in enumerate(rows):
        j = row // g                                    # KV head over all layers: layer * H + head
        sl = slice(j * T, (j + 1) * T)
        kr = OC.Record(*_gather(krec, np.arange(sl.start, sl.stop)))
        vr = OC.Record(*_gather(vrec, np.arange(sl.start, sl.stop)))
        qh = st["q_host"].reshape(L * HQ, D)[row:row + 1].astype(np.float64)
        s = OC.score(p, qh, kr)[0]
        xv = OC.dequantize(p, vr)
        vmax = np.abs(xv).max()
        z = scale * s
        w = np.exp(z - z.max())
        ref = (w / w.sum()) @ xv
        lim = (2e-4 * scale * np.linalg.norm(qh) * OC.half_value(kr.norms).max() + 1e-5) * vmax
        assert np.abs(got[i] - ref).max() <= lim, (row, np.abs(got[i] - ref).max() / lim)
        sg = st["scores"].view(L * HQ, T)[row].cpu().numpy().astype(np.float64)
        zg = scale * sg
        wg = np.exp(zg - zg.max())
        assert np.abs(got[i] - (wg / wg.sum()) @ xv).max() <= 1e-5 * vmax, row


# ------------------------------------- PolarQuant keys at the Qwen shape ----
@pytest.fixture(scope="module")
def qwen_polar(K, qwen):
    """The Qwen-shaped cache's keys (all layers, 2,359,296 vectors) as
    PolarQuant records in one call, and one decode step of all layers'
    scores in one pq_score call (query row l * HQ + h reads KV head
    l * H + h / group)."""
    from oracle import polar as PQ
    spec = qwen["spec"]
    L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
    n_k = L * H * T
    c = K.PolarCodec(seed=0)
    words = c.quantize(qwen["flat"][:n_k])
    scores = torch.empty((L * HQ, T), dtype=torch.float32, device=DEV)
    c.score(qwen["q"].view(L * HQ, D), words, qwen["group"], T, T, out=scores)
    _sync()
    st = dict(codec=c, words=words, scores=scores, n_k=n_k, p=PQ.PolarParams(D, 0))
    yield st
    st.clear()


def test_qwen_polar_sample(K, qwen, qwen_polar):
    """A seeded 1% of the key rows against the oracle: angle codes, radii,
    dequantisation, and the 8 query heads' scores of every sampled key."""
    from oracle import polar as PQ
    st, spec = qwen_polar, qwen["spec"]
    H, T, HQ, g = spec["kv_heads"], spec["tokens"], spec["q_heads"], qwen["group"]
    rows = W.sample_rows(st["n_k"], 0.01, seed=8)
    it = torch.from_numpy(rows).to(DEV)
    words = st["words"].index_select(0, it).cpu().numpy().view(np.uint32)
    x = qwen["flat"].index_select(0, it).cpu().numpy()
    rep = PR.check_polar_words(st["p"], x, words)
    print(f"qwen polar sample: {rows.size} keys, {rep}", flush=True)
    y = st["codec"].dequantize(st["words"].index_select(0, it), dtype=torch.float32).cpu().numpy()
    rn = PR.polar_radius_norm(words)
    PR.compare_recon(y, PQ.dequantize(st["p"], words), rn, "polar dequantize")
    layer, head, tok = rows // (H * T), (rows // T) % H, rows % T
    qrows = (layer * HQ + head * g)[:, None] + np.arange(g)[None, :]
    got = st["scores"][torch.from_numpy(qrows).to(DEV), torch.from_numpy(tok).to(DEV)[:, None]]
    got = got.cpu().numpy().astype(np.float64)
    qh = qwen["q_host"].reshape(-1, D).astype(np.float64)
    for key in np.unique(layer * H + head):
        sel = (layer * H + head) == key
        qk = qh[qrows[sel][0]]
        ref = PQ.score(st["p"], qk, words[sel])
        PR.compare_scores(got[sel].T, ref, np.linalg.norm(qk, axis=1)[:, None], rn[sel][None, :],
                          f"polar kv head {key}")


def test_qwen_polar_scores_full(K, qwen, qwen_polar):
    """All 18,874,368 polar decode scores against q . dequant(k), within
    1e-4 * ||q|| * ||r^||."""
    st, spec = qwen_polar, qwen["spec"]
    L, H, T, HQ, g = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"], qwen["group"]
    q = qwen["q"].view(L * HQ, D).to(torch.float64)
    qn = torch.linalg.norm(q, dim=1)
    worst = 0.0
    for j in range(L * H):
        w = st["words"][j * T:(j + 1) * T]
        xt = st["codec"].dequantize(w, dtype=torch.float32).to(torch.float64)
        rb = w[:, 12:16].contiguous().view(torch.float16).to(torch.float64)
        rn = torch.linalg.norm(rb, dim=1)
        ref = q[j * g:(j + 1) * g] @ xt.T
        lim = PR.SCORE_TOL * qn[j * g:(j + 1) * g, None] * rn[None, :] + 1e-30
        ratio = (st["scores"][j * g:(j + 1) * g].to(torch.float64) - ref).abs() / lim
        worst = max(worst, float(ratio.max()))
    assert worst <= 1.0, f"polar score vs dequantised key: worst {worst:.3g} x tolerance"


# ------------------------------------ PolarQuant keys at the Llama shape ----
def test_llama_polar_sample(K, llama):
    """The Llama-shaped cache's keys (all 32 layers, 33,554,432 vectors: 8.6
    GB of fp16 input and 2.1 GB of records, so row offsets pass 2^32 bytes)
    as PolarQuant records in one call, and one decode step of all layers'
    scores in one pq_score call.  A seeded 0.1% of the key rows against the
    oracle: angle codes, radii, dequantisation and the 4 query heads' scores
    of every sampled key."""
    from oracle import polar as PQ
    spec = llama["spec"]
    L, H, T, HQ, g = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"], llama["group"]
    n_k = L * H * T
    c = K.PolarCodec(seed=0)
    p = PQ.PolarParams(D, 0)
    words = c.quantize(llama["flat"][:n_k])
    scores = torch.empty((L * HQ, T), dtype=torch.float32, device=DEV)
    c.score(llama["q"].view(L * HQ, D), words, g, T, T, out=scores)
    _sync()
    rows = W.sample_rows(n_k, 0.001, seed=9)
    it = torch.from_numpy(rows).to(DEV)
    gw = words.index_select(0, it).cpu().numpy().view(np.uint32)
    x = llama["flat"].index_select(0, it).cpu().numpy()
    rep = PR.check_polar_words(p, x, gw)
    print(f"llama polar sample: {rows.size} keys, {rep}", flush=True)
    y = c.dequantize(words.index_select(0, it), dtype=torch.float32).cpu().numpy()
    rn = PR.polar_radius_norm(gw)
    PR.compare_recon(y, PQ.dequantize(p, gw), rn, "polar dequantize")
    layer, head, tok = rows // (H * T), (rows // T) % H, rows % T
    qrows = (layer * HQ + head * g)[:, None] + np.arange(g)[None, :]
    got = scores[torch.from_numpy(qrows).to(DEV), torch.from_numpy(tok).to(DEV)[:, None]]
    got = got.cpu().numpy().astype(np.float64)
    qh = llama["q_host"].reshape(-1, D).astype(np.float64)
    for key in np.unique(layer * H + head):
        sel = (layer * H + head) == key
        qk = qh[qrows[sel][0]]
        ref = PQ.score(p, qk, gw[sel])
        PR.compare_scores(got[sel].T, ref, np.linalg.norm(qk, axis=1)[:, None], rn[sel][None, :],
                          f"polar kv head {key}")
    del words, scores
