"""Lloyd-Max scalar codebooks (test infrastructure only).

Sources:
* Blog "TurboQuant 论文解读", section "Beta 分布" and "MSE 标量量化
  (Theorem 1)": after a uniformly random rotation each coordinate of a unit
  vector follows a fixed Beta-type law, so an optimal 2^b-level scalar
  quantizer can be precomputed offline.
* hyper.ai summary, section "方法": the centroids for that law are found
  with the Max-Lloyd algorithm and stored in a codebook.
* PolarQuant article, "Шаг 3": the Lloyd iteration itself -- cell
  boundaries at the midpoints of neighbouring centroids, then each centroid
  re-set to the probability-weighted mean of its cell, repeated until it
  settles.
* RotorQuant README, "Codebook Calibration Fix": the codebook must be built
  for d_eff = d (the vector dimension) on unit-normalised vectors.  The old
  Gaussian form with d_eff = 344 is kept as a variant to check the printed
  sigma and +-0.116.

The density of one coordinate of a uniform unit vector in R^d is
    f(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),
on [-1, 1]; x^2 ~ Beta(1/2, (d-1)/2), so the CDF is
    F(x) = 1/2 + sign(x)/2 * I_{x^2}(1/2, (d-1)/2).
The cell mean has a closed-form numerator:
    int_a^b x (1-x^2)^k dx = [(1-a^2)^(k+1) - (1-b^2)^(k+1)] / (2(k+1)).
"""
import math

import numpy as np
from scipy import special, stats


def beta_coord_pdf(x, d):
    x = np.asarray(x, dtype=np.float64)
    lc = special.gammaln(d / 2.0) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2.0)
    return np.where(np.abs(x) < 1.0, np.exp(lc) * np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2.0), 0.0)


def beta_coord_cdf(x, d):
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(x) * special.betainc(0.5, (d - 1) / 2.0, x * x)


def _beta_cell_moments(lo, hi, d):
    """(P(lo < X < hi), E[X; lo < X < hi]) for the coordinate law."""
    mass = beta_coord_cdf(hi, d) - beta_coord_cdf(lo, d)
    lc = special.gammaln(d / 2.0) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2.0)
    kp1 = (d - 1) / 2.0
    first = np.exp(lc) * ((1.0 - lo * lo) ** kp1 - (1.0 - hi * hi) ** kp1) / (2.0 * kp1)
    return mass, first


def _gauss_cell_moments(lo, hi, sigma):
    a, b = lo / sigma, hi / sigma
    mass = stats.norm.cdf(b) - stats.norm.cdf(a)
    first = sigma * (stats.norm.pdf(a) - stats.norm.pdf(b))
    return mass, first


def lloyd_max(levels, moments, support, init, tol=1e-15, max_iter=200000):
    """Lloyd iteration for a symmetric density.

    `moments(lo, hi)` returns arrays (mass, first moment) per cell.  Starting
    from `init`, alternate: boundaries = midpoints of neighbours; centroids =
    first moment / mass of each cell.  The density is symmetric and so is the
    fixed point; the centroids are symmetrised after every step so that
    rounding cannot break the symmetry.  Stops when the largest centroid
    change is below `tol`.
    """
    c = np.array(init, dtype=np.float64)
    for it in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-support], t))
        hi = np.concatenate((t, [support]))
        mass, first = moments(lo, hi)
        new = first / mass
        new = 0.5 * (new - new[::-1])
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it + 1


def beta_codebook(bits, d=128, tol=1e-15, init_scale=1.0):
    """Float64 Lloyd-Max centroids and midpoint boundaries, 2^bits levels.

    The start is the Gaussian N(0, 1/d) quantiles at (k + 1/2) / L, scaled by
    `init_scale` (a second start is used to check uniqueness).
    """
    levels = 1 << bits
    p = (np.arange(levels) + 0.5) / levels
    init = init_scale * stats.norm.ppf(p) / math.sqrt(d)
    c, t, _ = lloyd_max(levels, lambda lo, hi: _beta_cell_moments(lo, hi, d), 1.0, init, tol)
    return c, t


def gaussian_codebook(bits, d_eff, tol=1e-15):
    """Lloyd-Max for N(0, 1/d_eff) (the pre-fix reading of the README)."""
    levels = 1 << bits
    sigma = 1.0 / math.sqrt(d_eff)
    p = (np.arange(levels) + 0.5) / levels
    init = sigma * stats.norm.ppf(p)
    c, t, _ = lloyd_max(levels, lambda lo, hi: _gauss_cell_moments(lo, hi, sigma), np.inf, init, tol)
    return c, t


def beta_unit_mse(centroids, d=128):
    """Expected ||x - x~||^2 for a uniform unit vector, d coordinates.

    Uses the per-coordinate distortion E[(X - q(X))^2] summed over d
    coordinates, with q the nearest-centroid map (boundaries at midpoints).
    Computed from the second moment directly, not from the centroid
    condition, so it also holds for a codebook that is not a fixed point.
    """
    c = np.asarray(centroids, dtype=np.float64)
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    mass, first = _beta_cell_moments(lo, hi, d)
    # E[X^2; cell] = E[X^2] contributions: total E[X^2] = 1/d; per cell by quadrature.
    second = np.array([_beta_second(a, b, d) for a, b in zip(lo, hi)])
    per_coord = np.sum(second - 2.0 * c * first + c * c * mass)
    return d * per_coord


def _beta_second(a, b, d):
    """E[X^2; a < X < b] via the identity x^2 f = f - (1-x^2) f and the
    Beta(1/2, (d+1)/2) law of a coordinate in dimension d + 2."""
    # (1 - x^2) f_d(x) = c_d / c_{d+2} * f_{d+2}(x), with c_d the normaliser.
    lcd = special.gammaln(d / 2.0) - special.gammaln((d - 1) / 2.0)
    lcd2 = special.gammaln((d + 2) / 2.0) - special.gammaln((d + 1) / 2.0)
    ratio = math.exp(lcd - lcd2)
    mass_d = beta_coord_cdf(b, d) - beta_coord_cdf(a, d)
    mass_d2 = beta_coord_cdf(b, d + 2) - beta_coord_cdf(a, d + 2)
    return mass_d - ratio * mass_d2
