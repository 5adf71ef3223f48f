"""Pins for the oracle's PolarQuant (CPU only), against what the PolarQuant
article fixes: the lemma's angle density and its normalising constant, its
mean pi/4, the level each density belongs to (Monte Carlo over Gaussian
vectors), the uniform level-1 codebook, the exact inverse of the polar
transform, and the article's bit budget (496 bits per token, 4.13x)."""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import polar as PQ
from kv_cache_vector_norm_amd import workloads as W


@pytest.mark.parametrize("level", [1, 2, 3])
def test_lemma_density_is_normalised_with_mean_pi_over_4(level):
    f = PQ.level_density(level)
    mass = integrate.quad(f, 0, math.pi / 2, epsrel=1e-13)[0]
    mean = integrate.quad(lambda t: t * f(t), 0, math.pi / 2, epsrel=1e-13)[0]
    assert abs(mass - 1.0) < 1e-12
    assert abs(mean - math.pi / 4) < 1e-12


def test_level_one_codebook_is_uniform():
    c, t = PQ.codebooks()[0]
    assert np.allclose(c, (np.arange(16) + 0.5) * math.pi / 8, atol=2e-7)
    assert np.allclose(t, np.arange(1, 16) * math.pi / 8, atol=2e-7)


@pytest.mark.parametrize("level", [1, 2, 3])
def test_later_codebooks_are_symmetric_about_pi_over_4(level):
    c, t = PQ.codebooks()[level]
    assert c.shape == (4,) and t.shape == (3,)
    assert np.allclose(c + c[::-1], math.pi / 2, atol=4e-7)
    assert abs(t[1] - math.pi / 4) < 2e-7
    # tighter levels: the cells shrink toward pi/4 as k grows
    if level > 1:
        assert c[0] > PQ.codebooks()[level - 1][0][0]


def test_angle_laws_per_level_monte_carlo():
    """Angles of N(0, 1) vectors: level 1 uniform on [0, 2 pi), level l >= 2
    the lemma's law with k = 2^(l-1) (mean pi/4, its variance)."""
    y = np.random.Generator(np.random.PCG64(3)).standard_normal((4000, 128))
    angles, _ = PQ.polar_transform(y)
    a0 = angles[0].ravel()
    assert abs(a0.mean() - math.pi) < 4 * (2 * math.pi / math.sqrt(12)) / math.sqrt(a0.size)
    assert abs(a0.var() - (2 * math.pi) ** 2 / 12) < 0.05 * (2 * math.pi) ** 2 / 12
    for level in (1, 2, 3):
        f = PQ.level_density(level)
        var = integrate.quad(lambda t: (t - math.pi / 4) ** 2 * f(t), 0, math.pi / 2)[0]
        th = angles[level].ravel()
        assert abs(th.mean() - math.pi / 4) < 4 * math.sqrt(var / th.size)
        assert abs(th.var() / var - 1) < 0.06


def test_polar_transform_inverts_exactly():
    y = W.gaussian(20, seed=4).astype(np.float64)
    angles, radii = PQ.polar_transform(y)
    assert radii.shape == (20, 8)
    assert np.abs(PQ.polar_inverse(angles, radii) - y).max() < 1e-12
    assert np.allclose(np.linalg.norm(radii, axis=1), np.linalg.norm(y, axis=1))


def test_bit_budget_of_the_article():
    bits = PQ.CODE_BITS + 16 * PQ.N_RADII
    assert PQ.CODE_BITS == 64 * 4 + 32 * 2 + 16 * 2 + 8 * 2 == 368
    assert bits == 496
    assert round(128 * 16 / bits, 2) == 4.13


def test_quantise_dequantise_roundtrip():
    p = PQ.PolarParams(128, 0)
    x = W.gaussian(200, seed=5).astype(np.float64)
    x[3] = 0.0
    words, diag = PQ.quantize(p, x)
    assert words.shape == (200, 16) and np.all(words[:, 11] >> 16 == 0)
    codes, rb = PQ.unpack(words)
    for l, (c, b) in enumerate(zip(codes, PQ.LEVEL_BITS)):
        assert c.min() >= 0 and c.max() < (1 << b)
    assert np.array_equal(PQ.pack(codes, rb), words)
    xt = PQ.dequantize(p, words)
    assert np.all(xt[3] == 0.0)
    rel = np.linalg.norm(xt - x, axis=1) / np.maximum(np.linalg.norm(x, axis=1), 1e-30)
    rel = np.delete(rel, 3)
    # four angle levels of 4 / 2 / 2 / 2 bits: a coarse but bounded error
    assert rel.max() < 0.8 and 0.05 < rel.mean() < 0.5
    # more levels of the radius tree decoded exactly -> exact vector
    ex = PQ.polar_inverse(diag.angles, PQ._half_value(rb)) @ p.pi
    assert np.abs(ex - x).max() < 1e-2 * np.abs(x).max()


def test_codes_are_the_nearest_centroid():
    """code = #{k : theta > t_k} with midpoint boundaries is the index of the
    nearest centroid (circular distance on level 1), by brute force."""
    p = PQ.PolarParams(128, 0)
    x = W.gaussian(300, seed=6).astype(np.float64)
    words, diag = PQ.quantize(p, x)
    codes, _ = PQ.unpack(words)
    for level in range(PQ.N_LEVELS):
        c = p.books[level][0]
        d = np.abs(diag.angles[level][..., None] - c)
        if level == 0:
            d = np.minimum(d, 2 * math.pi - d)
        assert np.array_equal(codes[level], np.argmin(d, axis=-1))


def test_score_reads_rotated_coordinates():
    """With q = Pi^T e_j the score is coordinate j of the decoded polar
    vector y~ (Pi orthogonal): a transposed Pi or a misplaced level fails."""
    p = PQ.PolarParams(128, 0)
    x = W.gaussian(40, seed=7).astype(np.float64)
    words, _ = PQ.quantize(p, x)
    codes, rb = PQ.unpack(words)
    angles = [p.books[l][0][codes[l]] for l in range(PQ.N_LEVELS)]
    yt = PQ.polar_inverse(angles, PQ._half_value(rb))
    s = PQ.score(p, p.pi[[3, 77]], words)             # rows of Pi = (Pi^T e_j)^T
    assert np.abs(s - yt[:, [3, 77]].T).max() < 1e-5 * np.abs(yt).max()


def test_attention_over_polar_keys():
    """The polar-key attention is the softmax of the scaled polar scores
    applied to the decoded values: a dominant key returns its value, scale 0
    the mean of the values (per GQA head)."""
    from oracle import codec as OC
    from oracle import params as OP
    p = PQ.PolarParams(128, 0)
    pv = OP.Params(128, 3, 0, OP.MSE)
    t, kvh, group = 20, 2, 3
    k = W.gaussian(kvh * t, seed=8).astype(np.float64)
    q = W.queries(kvh * group, seed=9).astype(np.float64)
    k[7] = 4.0 * q[0]                                   # head 0's dominant key for query row 0
    words, _ = PQ.quantize(p, k)
    vrec, _ = OC.quantize(pv, W.gaussian(kvh * t, seed=10).astype(np.float64))
    xv = OC.dequantize(pv, vrec)
    out0 = PQ.attend(p, pv, q, words, vrec, group, t, 0.0)
    for h in range(kvh * group):
        j = h // group
        assert np.abs(out0[h] - xv[j * t:(j + 1) * t].mean(0)).max() < 1e-14
    out = PQ.attend(p, pv, q, words, vrec, group, t, 1.0)
    s = PQ.score(p, q[:1], words[:t])[0]
    gap = s[7] - np.max(np.delete(s, 7))
    assert gap > 30
    assert np.abs(out[0] - xv[7]).max() < t * np.exp(-gap) * np.abs(xv).max() + 1e-12


def test_attention_over_polar_values():
    """PolarQuant values: scale 0 gives the mean of the decoded values, a
    single key its decoded value, and a dominant key its value (per GQA
    head; rotor-scored and polar-scored keys)."""
    from oracle import codec as OC
    from oracle import params as OP
    pv = PQ.PolarParams(128, 3)
    t, kvh, group = 20, 2, 3
    vw, _ = PQ.quantize(pv, W.gaussian(kvh * t, seed=11).astype(np.float64))
    xv = PQ.dequantize(pv, vw)
    q = W.queries(kvh * group, seed=12).astype(np.float64)
    k = W.gaussian(kvh * t, seed=13).astype(np.float64)
    k[5] = 4.0 * q[0]                                    # head 0's dominant key for query row 0
    pk_rotor = OP.Params(128, 3, 0, OP.QJL)
    krec, _ = OC.quantize(pk_rotor, k)
    pk_polar = PQ.PolarParams(128, 0)
    kw, _ = PQ.quantize(pk_polar, k)
    for pk, keys in ((pk_rotor, krec), (pk_polar, kw)):
        out0 = PQ.attend_values(pk, pv, q, keys, vw, group, t, 0.0)
        for h in range(kvh * group):
            j = h // group
            assert np.abs(out0[h] - xv[j * t:(j + 1) * t].mean(0)).max() < 1e-14
        one = PQ.attend_values(pk, pv, q[:group], keys, vw, group, 1, 1.0)
        assert np.abs(one - xv[:1]).max() < 1e-14
        out = PQ.attend_values(pk, pv, q, keys, vw, group, t, 1.0)
        if isinstance(pk, PQ.PolarParams):
            s = PQ.score(pk, q[:1], kw[:t])[0]
        else:
            s = OC.score(pk, q[:1], OC._rows(krec, slice(0, t)))[0]
        gap = s[5] - np.max(np.delete(s, 5))
        assert gap > 30
        assert np.abs(out[0] - xv[5]).max() < t * np.exp(-gap) * np.abs(xv).max() + 1e-12


@pytest.mark.parametrize("level", [1, 2, 3])
def test_later_codebooks_are_cell_means_by_gauss_legendre(level):
    """The centroid condition of Lloyd's algorithm checked by a quadrature
    other than the one the oracle iterates with: on every cell
    [t_(i-1), t_i] of levels 2..4 the centroid is the mean angle of the
    article's law sin^(k-1)(2 theta), k = 2^(l-1) (normalising constants
    cancel), from 200-point Gauss-Legendre rules on 16 sub-intervals; the
    boundaries are the centroids' midpoints.  Stored values are fp32, hence
    the tolerance."""
    c, t = PQ.codebooks()[level]
    k = 2 ** level
    lo = np.r_[0.0, t]
    hi = np.r_[t, math.pi / 2.0]
    xg, wg = np.polynomial.legendre.leggauss(200)
    for i in range(len(c)):
        edges = np.linspace(lo[i], hi[i], 17)
        m0 = m1 = 0.0
        for a, b in zip(edges[:-1], edges[1:]):
            th = 0.5 * (b - a) * xg + 0.5 * (b + a)
            w = 0.5 * (b - a) * wg * np.sin(2.0 * th) ** (k - 1)
            m0 += w.sum()
            m1 += (w * th).sum()
        assert abs(m1 / m0 - c[i]) <= 2e-7 * abs(c[i])
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=2e-7, atol=0)
