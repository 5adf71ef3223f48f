"""Seeded synthetic inputs shaped like the pages' workloads.

This module draws inputs only; it holds none of the codec's arithmetic, so
both the HIP path and the CPU oracle can be fed from it.

Shapes follow the pages:
* unit-vector and N(0,1) key/value sets at head dim 128 (README "MSE
  Quality" and "Triton Kernel Speed": d = 128, up to 65,536 vectors);
* KV caches shaped like Qwen2.5-3B (36 layers, 2 KV heads, 16 query heads;
  README "Background" and "Real Model Validation") and Llama-3.1-8B
  (32 layers, 8 KV heads, 32 query heads, 128K context; PolarQuant article,
  "Проблема KV-кэша").  Real caches live on "low-rank manifolds" with
  "massive outliers" (podcast page; blog on Lemma 1), so the cache generator
  is rank-16 Gaussian factors plus N(0, 0.1^2) noise plus four outlier
  channels per head scaled by 10.  These stand in for the real models'
  caches, which need weights that are not used here.
"""
import numpy as np

HEAD_DIM = 128
LOWRANK = 16
NOISE_STD = 0.1
N_OUTLIERS = 4
OUTLIER_SCALE = 10.0


def gaussian(n, d=HEAD_DIM, seed=0, dtype=np.float16):
    """n x d i.i.d. N(0,1) from numpy PCG64(seed), cast once to dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((n, d)).astype(dtype)


def unit_gaussian(n, d=HEAD_DIM, seed=0, dtype=np.float32):
    """N(0,1) rows normalised in float64, then cast once to dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return x.astype(dtype)


def queries(h, d=HEAD_DIM, seed=1):
    """h x d float32 N(0,1) query rows."""
    return gaussian(h, d, seed, np.float32)


def unit_vectors_1024():
    """1,024 fp32 unit vectors (N(0,1) then normalised), seed 0."""
    return unit_gaussian(1024, seed=0, dtype=np.float32)


def keys_65536():
    """65,536 fp16 N(0,1) vectors (norms near sqrt(128)), seed 0."""
    return gaussian(65536, seed=0, dtype=np.float16)


def queries_64():
    return queries(64, seed=1)


def keys_262144():
    return gaussian(262144, seed=0, dtype=np.float16)


# ------------------------------------------------------------ KV caches ----
QWEN25_3B = dict(name="qwen2.5-3b", layers=36, kv_heads=2, q_heads=16, tokens=32768)
LLAMA31_8B = dict(name="llama3.1-8b", layers=32, kv_heads=8, q_heads=32, tokens=131072)


def lowrank_head(tokens, seed, device="cpu", with_query_heads=0, torch=None):
    """One (layer, head) block of a synthetic cache, as torch tensors.

    Returns (K [tokens, 128] fp16, V [tokens, 128] fp16, Q [q, 128] fp32).
    K = U_k W_k^T / 4 + 0.1 eps, V likewise with its own factors; then four
    channels (a seeded choice per head, shared by K, V and the queries) are
    multiplied by 10.  Queries are W_k u / 4 + 0.1 eps with fresh u, so they
    live near the keys' subspace, with the same outlier channels scaled.
    """
    if torch is None:
        import torch  # noqa: F811
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    d = HEAD_DIM
    perm = torch.randperm(d, generator=g, device=device)[:N_OUTLIERS]
    scale = torch.ones(d, device=device)
    scale[perm] = OUTLIER_SCALE

    def block(n):
        w = torch.randn(d, LOWRANK, generator=g, device=device)
        u = torch.randn(n, LOWRANK, generator=g, device=device)
        x = u @ w.T / 4.0 + NOISE_STD * torch.randn(n, d, generator=g, device=device)
        return x * scale, w

    k, wk = block(tokens)
    v, _ = block(tokens)
    q = None
    if with_query_heads:
        uq = torch.randn(with_query_heads, LOWRANK, generator=g, device=device)
        q = (uq @ wk.T / 4.0 + NOISE_STD * torch.randn(with_query_heads, d, generator=g, device=device)) * scale
    return k.to(torch.float16), v.to(torch.float16), q


def cache_seed(base_seed, layer, head):
    return (base_seed * 1_000_003 + layer * 1009 + head) & 0x7FFFFFFFFFFF


def needle_keys(t, d=HEAD_DIM, seed=7, cos=0.6):
    """t random fp32 keys and one query whose best match is a planted key.

    Keys are N(0,1); the query is N(0,1).  The key at a seeded position is
    replaced by a vector of norm sqrt(d) at cosine `cos` to the query, which
    puts its true score well above the largest of the random keys (about
    four standard deviations for t = 8192) but not out of reach of the
    quantisation noise.  Returns (keys [t, d], query [d], needle index).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    keys = rng.standard_normal((t, d))
    q = rng.standard_normal(d)
    qu = q / np.linalg.norm(q)
    w = rng.standard_normal(d)
    w -= (w @ qu) * qu
    w /= np.linalg.norm(w)
    idx = int(rng.integers(t))
    keys[idx] = np.sqrt(d) * (cos * qu + np.sqrt(1.0 - cos * cos) * w)
    return keys.astype(np.float32), q.astype(np.float32), idx


def kv_cache(spec, device="cpu", base_seed=0, torch=None):
    """A whole synthetic cache of a model shape, filled head by head.

    Returns (kv [2, layers, kv_heads, tokens, 128] fp16 with K at index 0 and
    V at 1, q [layers, q_heads, 128] fp32).  Query heads h of a layer come
    from the generator of KV head h // (q_heads / kv_heads), so each group of
    query heads sits near its own keys' subspace.
    """
    if torch is None:
        import torch  # noqa: F811
    L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
    group = HQ // H
    kv = torch.empty((2, L, H, T, HEAD_DIM), dtype=torch.float16, device=device)
    q = torch.empty((L, HQ, HEAD_DIM), dtype=torch.float32, device=device)
    for layer in range(L):
        for h in range(H):
            k, v, qh = lowrank_head(T, cache_seed(base_seed, layer, h), device=device,
                                    with_query_heads=group, torch=torch)
            kv[0, layer, h].copy_(k)
            kv[1, layer, h].copy_(v)
            q[layer, h * group:(h + 1) * group].copy_(qh)
    return kv, q


def sample_rows(n, fraction, seed):
    """Sorted seeded sample of round(fraction * n) distinct row indices."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = max(1, int(round(fraction * n)))
    return np.sort(rng.choice(n, size=m, replace=False))
