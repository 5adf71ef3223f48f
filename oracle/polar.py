"""PolarQuant, stated plainly in float64 (test infrastructure only).

Follows the PolarQuant article ("TurboQuant и PolarQuant: математика
квантизации KV-кэша в LLM"), sections "PolarQuant: ключевая идея",
"Полярное преобразование: от декартовых к полярным координатам",
"Алгоритм PolarQuant на практике" and "Степень сжатия":

  1. Preconditioning: y = Pi x with Pi orthogonal from Gram-Schmidt of a
     seeded Gaussian matrix (the same Pi as the TurboQuant session of the
     same seed).
  2. Recursive polar transform, four levels: level 1 pairs coordinates
     (y_2i, y_2i+1) -> angle atan2(y_2i+1, y_2i) taken in [0, 2 pi) and
     radius sqrt(y_2i^2 + y_2i+1^2); each later level pairs the previous
     radii the same way, so its angles lie in [0, pi/2].  128 -> 64 -> 32
     -> 16 -> 8 radii.
  3. Per-level codebooks from Lloyd's algorithm on the known angle law:
     level 1 uniform on [0, 2 pi) with 4 bits; level l >= 2 with density
     Gamma(k) / (2^(k-2) Gamma(k/2)^2) sin^(k-1)(2 theta) on [0, pi/2],
     k = 2^(l-1) coordinates behind each paired radius, 2 bits.
  4. Record: the angle codes (64 x 4 + 32 x 2 + 16 x 2 + 8 x 2 = 368 bits)
     and the 8 remaining radii as IEEE halves: 496 bits of content.
  Dequantisation walks the levels back from the 8 radii with the centroid
  angles, then x~ = Pi^T y~.  The score is <q, x~>.

Layout (this codec's own; the article gives none): 16 u32 words per
vector, words 0..11 the code stream LSB-first (level 1 codes, then levels
2, 3, 4; bits 368..383 zero), words 12..15 the radii, radius 2i in the low
half of word 12 + i.
"""
import math

import numpy as np
from scipy import integrate

from .params import f32, pi_matrix

D = 128
LEVEL_BITS = (4, 2, 2, 2)
N_LEVELS = 4
N_RADII = D >> N_LEVELS          # 8
WORDS = 16
CODE_BITS = sum((D >> (l + 1)) * b for l, b in enumerate(LEVEL_BITS))   # 368


def level_range(level):
    return (0.0, 2.0 * math.pi) if level == 0 else (0.0, math.pi / 2.0)


def level_density(level):
    """Density of the level's angle for a Gaussian input (0-based level)."""
    lo, hi = level_range(level)
    if level == 0:
        return lambda th: 1.0 / (hi - lo)
    k = 2 ** level
    const = math.gamma(k) / (2.0 ** (k - 2) * math.gamma(k / 2.0) ** 2)
    return lambda th: const * math.sin(2.0 * th) ** (k - 1)


def lloyd(density, lo, hi, levels, tol=1e-14, max_iter=10000):
    """Lloyd's algorithm on [lo, hi]: centroids = conditional means of
    their cells, boundaries = midpoints, from a uniform start."""
    c = lo + (np.arange(levels) + 0.5) * (hi - lo) / levels
    for _ in range(max_iter):
        t = np.concatenate([[lo], (c[:-1] + c[1:]) / 2.0, [hi]])
        new = np.empty(levels)
        for i in range(levels):
            mass = integrate.quad(density, t[i], t[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
            mom = integrate.quad(lambda th: th * density(th), t[i], t[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
            new[i] = mom / mass if mass > 0 else (t[i] + t[i + 1]) / 2.0
        done = np.max(np.abs(new - c)) < tol
        c = new
        if done:
            break
    return c, (c[:-1] + c[1:]) / 2.0


_CODEBOOKS = None


def codebooks():
    """[(centroids, boundaries)] per level, each rounded once to fp32."""
    global _CODEBOOKS
    if _CODEBOOKS is None:
        out = []
        for level, bits in enumerate(LEVEL_BITS):
            lo, hi = level_range(level)
            c, t = lloyd(level_density(level), lo, hi, 1 << bits)
            out.append((f32(c), f32(t)))
        _CODEBOOKS = out
    return _CODEBOOKS


class PolarParams:
    def __init__(self, d=D, seed=0):
        if d != D:
            raise ValueError("PolarQuant here is specified for d = 128 (four levels, eight radii)")
        self.d = d
        self.seed = seed
        self.pi = pi_matrix(d, seed)
        self.books = codebooks()


def polar_pairs(y):
    """The pairs each level's angles are taken of, and the final radii.

    A level turns a vector of n coordinates into n/2 (angle, radius) pairs:
    coordinate 2i is paired with coordinate 2i + 1 (the PolarQuant article's
    polar transform takes consecutive coordinates two at a time), and the
    next level does the same to the n/2 radii.  Returns ([pairs of level
    1..4, each [N, n_l, 2]], radii [N, 8])."""
    v = np.asarray(y, dtype=np.float64)
    pairs = []
    for _ in range(N_LEVELS):
        pr = v.reshape(v.shape[0], v.shape[1] // 2, 2)
        pairs.append(pr)
        v = np.hypot(pr[..., 0], pr[..., 1])
    return pairs, v


def polar_transform(y):
    """(angles per level, final radii) of rows of y, float64.  The angle of a
    pair (first, second) is the polar angle of the point with those Cartesian
    coordinates; level-1 angles are taken in [0, 2 pi), later levels pair
    non-negative radii, so their angles lie in [0, pi/2]."""
    pairs, radii = polar_pairs(y)
    angles = []
    for level, pr in enumerate(pairs):
        th = np.arctan2(pr[..., 1], pr[..., 0])
        if level == 0:
            th = np.where(th < 0.0, th + 2.0 * math.pi, th)
        angles.append(th)
    return angles, radii


def polar_inverse(angles, radii):
    """Walks the levels back: each radius r with angle th is the pair
    (r cos th, r sin th) of the level below."""
    r = np.asarray(radii, dtype=np.float64)
    for level in reversed(range(N_LEVELS)):
        th = angles[level]
        r = np.stack([r * np.cos(th), r * np.sin(th)], axis=-1).reshape(r.shape[0], 2 * r.shape[1])
    return r


def _half_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _half_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def pack(codes, radius_bits):
    """codes: per level [N, n_l] ints; radius_bits [N, 8] uint16 -> [N, 16] uint32."""
    n = radius_bits.shape[0]
    bits = np.zeros((n, 32 * WORDS), dtype=np.uint64)
    pos = 0
    for level, b in enumerate(LEVEL_BITS):
        c = np.asarray(codes[level], dtype=np.uint64)
        for i in range(c.shape[1]):
            for k in range(b):
                bits[:, pos + b * i + k] = (c[:, i] >> np.uint64(k)) & np.uint64(1)
        pos += b * c.shape[1]
    rb = np.asarray(radius_bits, dtype=np.uint64)
    for i in range(N_RADII):
        for k in range(16):
            bits[:, 32 * 12 + 16 * i + k] = (rb[:, i] >> np.uint64(k)) & np.uint64(1)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (bits.reshape(n, WORDS, 32) * weights).sum(axis=2).astype(np.uint32)


def unpack(words):
    """[N, 16] uint32 -> (codes per level, radius bits [N, 8])."""
    w = np.asarray(words, dtype=np.uint64)
    n = w.shape[0]
    bits = ((w[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).reshape(n, 32 * WORDS)
    codes, pos = [], 0
    for level, b in enumerate(LEVEL_BITS):
        m = D >> (level + 1)
        c = np.zeros((n, m), dtype=np.int64)
        for k in range(b):
            c += (bits[:, pos + b * np.arange(m) + k] << np.uint64(k)).astype(np.int64)
        codes.append(c)
        pos += b * m
    rb = np.zeros((n, N_RADII), dtype=np.int64)
    for k in range(16):
        rb += (bits[:, 32 * 12 + 16 * np.arange(N_RADII) + k] << np.uint64(k)).astype(np.int64)
    return codes, rb.astype(np.uint16)


class PolarDiagnostics:
    def __init__(self, angles, radii):
        self.angles = angles      # per level, float64
        self.radii = radii        # final radii, float64


def quantize(p: PolarParams, x):
    x = np.asarray(x, dtype=np.float64)
    y = x @ p.pi.T
    angles, radii = polar_transform(y)
    codes = [(angles[l][..., None] > p.books[l][1]).sum(axis=-1) for l in range(N_LEVELS)]
    return pack(codes, _half_bits(radii)), PolarDiagnostics(angles, radii)


def dequantize(p: PolarParams, words):
    codes, rb = unpack(words)
    angles = [p.books[l][0][codes[l]] for l in range(N_LEVELS)]
    y = polar_inverse(angles, _half_value(rb))
    return y @ p.pi


def score(p: PolarParams, q, words):
    """[H, T] inner products of query rows with the dequantised keys."""
    return np.asarray(q, dtype=np.float64) @ dequantize(p, words).T


def boundary_distance(p: PolarParams, diag: PolarDiagnostics):
    """Per level, each angle's distance to its nearest decision boundary.
    Level 1 angles live on a circle: 0 = 2 pi is where code 0 meets code 15."""
    out = []
    for l in range(N_LEVELS):
        t = p.books[l][1]
        if l == 0:
            t = np.concatenate([[0.0], t, [2.0 * math.pi]])
        out.append(np.min(np.abs(diag.angles[l][..., None] - t), axis=-1))
    return out


def attend(p: PolarParams, pv, q, words, vrec, group, t, scale, kv_stride=None):
    """Decode attention over PolarQuant keys: softmax(scale * <q_h, x~_t>)
    weighs the values, decoded with their own session (the KV-cache
    section's softmax(Q K^T / sqrt(d)) V, with the keys read from their
    PolarQuant records).  Query head h reads KV head j = h // group, whose
    keys and values start at row j * kv_stride.  Returns [H, d]."""
    from . import codec as OC
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], D))
    for h in range(q.shape[0]):
        j = h // group
        rows = slice(j * kv_stride, j * kv_stride + t)
        s = scale * score(p, q[h:h + 1], np.asarray(words)[rows])[0]
        e = np.exp(s - s.max())
        out[h] = (e / e.sum()) @ OC.dequantize(pv, OC._rows(vrec, rows))
    return out


def attend_values(pk, pv, q, keys, vwords, group, t, scale, kv_stride=None):
    """Decode attention with PolarQuant values: softmax(scale * <q_h, k~_t>)
    weighs the values decoded from their PolarQuant records (pv, the value
    session), the KV-cache section's softmax(Q K^T / sqrt(d)) V with V read
    from its PolarQuant records.  Keys are scored by their own session: pk a
    PolarParams (keys: 16-word records) or a codec Params (keys: a codec
    Record, scored by the codec's estimator).  Query head h reads KV head
    j = h // group, whose keys and values start at row j * kv_stride.
    Returns [H, d]."""
    from . import codec as OC
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], D))
    for h in range(q.shape[0]):
        j = h // group
        rows = slice(j * kv_stride, j * kv_stride + t)
        if isinstance(pk, PolarParams):
            s = score(pk, q[h:h + 1], np.asarray(keys)[rows])[0]
        else:
            s = OC.score(pk, q[h:h + 1], OC._rows(keys, rows))[0]
        s = scale * s
        e = np.exp(s - s.max())
        out[h] = (e / e.sum()) @ dequantize(pv, np.asarray(vwords)[rows])
    return out
