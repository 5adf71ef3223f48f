"""Pins for the oracle's Lloyd-Max codebooks and the theorems (CPU only)."""
import math

import numpy as np
import pytest
from scipy import integrate

from conftest import golden
from oracle import lloyd_max as L
from oracle import theory as T

D = 128


@pytest.fixture(scope="module")
def books():
    return {b: L.beta_codebook(b, D) for b in range(1, 5)}


def test_density_is_the_unit_sphere_coordinate_law():
    # integrates to 1 and has variance 1/d (E[sum y_i^2] = 1 over d coordinates)
    tot, _ = integrate.quad(lambda x: L.beta_coord_pdf(x, D), -1, 1, epsabs=1e-14)
    var, _ = integrate.quad(lambda x: x * x * L.beta_coord_pdf(x, D), -1, 1, epsabs=1e-14)
    assert math.isclose(tot, 1.0, rel_tol=1e-12)
    assert math.isclose(var, 1.0 / D, rel_tol=1e-10)
    # Monte Carlo: first coordinate of normalised Gaussians
    rng = np.random.default_rng(0)
    x = rng.normal(size=(200000, D))
    c1 = x[:, 0] / np.linalg.norm(x, axis=1)
    from scipy import stats
    assert stats.kstest(c1, lambda t: L.beta_coord_cdf(t, D)).pvalue > 1e-3


def test_one_bit_closed_form(books):
    c, t = books[1]
    e = T.mean_abs_coord(D)
    assert np.allclose(c, [-e, e], atol=1e-12, rtol=0)
    assert t[0] == 0.0
    assert math.isclose(L.beta_unit_mse(c, D), T.one_bit_distortion(D), rel_tol=1e-10)
    assert math.isclose(T.one_bit_distortion(D), 0.360889, abs_tol=5e-7)


def test_centroids_are_cell_means_by_quadrature(books):
    # checks the closed-form numerator and the incomplete-beta denominator
    for b in (2, 3):
        c, t = books[b]
        lo = np.r_[-1.0, t]
        hi = np.r_[t, 1.0]
        for k in range(len(c)):
            m0, _ = integrate.quad(lambda x: L.beta_coord_pdf(x, D), lo[k], hi[k], epsabs=1e-15)
            m1, _ = integrate.quad(lambda x: x * L.beta_coord_pdf(x, D), lo[k], hi[k], epsabs=1e-15)
            assert math.isclose(m1 / m0, c[k], rel_tol=1e-9, abs_tol=1e-12)
        assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)


def test_fixed_point_unique_from_two_starts(books):
    for b in range(1, 5):
        c2, _ = L.beta_codebook(b, D, init_scale=0.4)
        assert np.abs(books[b][0] - c2).max() < 1e-12


def test_codebook_symmetric_and_sorted(books):
    for b, (c, t) in books.items():
        assert np.all(np.diff(c) > 0)
        assert np.array_equal(c, -c[::-1])


def test_readme_mse_table(books):
    g = golden("readme_mse_table.json")
    for row in g["rows"]:
        mse = L.beta_unit_mse(books[row["bits"]][0], D)
        assert round(mse, 3) == row["mse"], (row, mse)
        # cosine of a unit vector with its reconstruction, E <x, x~>/|x~|:
        # the centroid condition gives <x, x~> = |x~|^2, so cos ~ sqrt(1 - D)
        assert abs(math.sqrt(1 - mse) - row["cosine"]) < 1.5e-3


def test_mse_matches_monte_carlo(books):
    rng = np.random.default_rng(1)
    x = rng.normal(size=(20000, D))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    for b in (2, 3):
        c, t = books[b]
        q = c[(x[..., None] > t).sum(-1)]
        err = ((x - q) ** 2).sum(1)
        se = err.std() / math.sqrt(len(err))
        assert abs(err.mean() - L.beta_unit_mse(c, D)) < 4 * se


def test_theorem1_and_theorem3_bounds(books):
    g = golden("theorems.json")
    assert math.isclose(T.THM1_CONSTANT_DERIVED, g["thm1_constant_derived"], rel_tol=1e-15)
    assert math.isclose(T.THM1_CONSTANT_PRINTED, g["thm1_constant_printed"], rel_tol=1e-15)
    ratios = []
    for b in range(1, 5):
        dd = L.beta_unit_mse(books[b][0], D)
        assert T.thm3_lower(b) <= dd <= T.thm1_upper(b)
        ratios.append(dd * 4 ** b)
    # the constant grows with b toward the large-b value, ~1.45 at b = 1
    assert np.all(np.diff(ratios) > 0)
    assert abs(ratios[0] - g["b1_constant_remark"]) < 0.01
    assert ratios[-1] < g["large_b_constant_remark"] + 0.03
    # the printed constant sqrt(3 pi)/2 is contradicted by the MSE table
    assert L.beta_unit_mse(books[2][0], D) > T.thm1_upper(2, T.THM1_CONSTANT_PRINTED)


def test_max1960_gaussian_levels():
    g = golden("max1960_gaussian.json")
    c4, _ = L.gaussian_codebook(2, 1.0)
    c8, _ = L.gaussian_codebook(3, 1.0)
    assert np.allclose(c4[2:], g["levels_4"], atol=g["tolerance"])
    assert np.allclose(c8[4:], g["levels_8"], atol=g["tolerance"])


def test_readme_codebook_fix_numbers():
    g = golden("readme_codebook_fix.json")
    assert round(1 / math.sqrt(g["d_eff_old"]), 3) == g["sigma_old"]
    assert round(1 / math.sqrt(g["d"]), 3) == g["sigma_new"]
    c, _ = L.gaussian_codebook(3, g["d_eff_old"])
    assert round(c[-1], 3) == g["outer_centroid_old_3bit"]


def test_one_bit_shrinkage_limit():
    g = golden("theorems.json")
    assert math.isclose(T.one_bit_shrinkage(D), 0.63911, abs_tol=5e-6)
    assert abs(T.one_bit_shrinkage(100000) - g["shrinkage_limit"]) < 1e-5
