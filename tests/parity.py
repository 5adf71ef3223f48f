"""GPU-versus-oracle comparison rules shared by the GPU tests.

The oracle works in float64 and the kernels in fp32, so a decision taken
within rounding distance of a boundary may go either way.  The rules:

* codes: every coordinate whose code differs must have the oracle's rotated
  coordinate y within BAND (1e-6, unit-vector domain) of a decision
  boundary; the fraction of coordinates inside the band must be <= 1e-4.
  The band count is a property of the data (about 2e-5 to 8e-5 of all
  coordinates at 2 to 4 MSE bits), so on batches of fewer than ~1e6
  coordinates the bound is applied with its Poisson allowance,
  1e-4 N + 3 sqrt(1e-4 N), and never below BAND_FLOOR coordinates;
* sign bits: the same rule on the oracle's z = S r with boundary 0, checked
  on vectors with no coordinate in the code band (their residual is defined
  by the same codes on both sides);
* half-precision norms / residual norms: bit-equal unless the float64 value
  is within 1e-6 (relative) of a half rounding midpoint;
* reconstructions (fp32): |gpu - oracle| <= 1e-5 * n^ per vector;
* scores: |gpu - oracle| <= 1e-4 * ||q|| * n^.
"""
import numpy as np

from oracle import codec as K

BAND = 1e-6
BAND_FRACTION = 1e-4
BAND_FLOOR = 3
RECON_TOL = 1e-5
SCORE_TOL = 1e-4


def half_midpoint_distance(v):
    """Relative distance of float64 values to the nearest half rounding midpoint."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    h = v.astype(np.float16).astype(np.float64)
    up = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h.astype(np.float16), np.float16(0)).astype(np.float64)
    mids = np.stack([(h + up) / 2, (h + dn) / 2])
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.min(np.abs(mids - v), axis=0) / np.where(v > 0, v, 1.0)
    return rel


def compare_halves(gpu_bits, oracle_values, what):
    """Half bit patterns equal except near rounding midpoints."""
    exp = K.half_bits(oracle_values)
    bad = (gpu_bits != exp) & (half_midpoint_distance(oracle_values) > 1e-6)
    assert not bad.any(), f"{what}: {bad.sum()} mismatches outside the midpoint band, first at {np.argmax(bad)}"
    return int((gpu_bits != exp).sum())


def compare_codes(p, gpu_words, diag):
    """Returns (band mask per vector, report).  Asserts the code rule."""
    gc = K.unpack_codes(gpu_words, p.b_m, p.n_coords)
    oc = K.scalar_quantize(p, diag.y)
    dist = K.boundary_distance(p, diag.y)
    in_band = dist < BAND
    mism = gc != oc
    outside = mism & ~in_band
    assert not outside.any(), (
        f"{outside.sum()} code mismatches outside the band; first vector "
        f"{np.argwhere(outside)[0]} gpu {gc[outside][:5]} oracle {oc[outside][:5]} dist {dist[outside][:5]}")
    frac = in_band.mean()
    expected = BAND_FRACTION * in_band.size
    allowed = expected + (3.0 * np.sqrt(expected) if in_band.size < 1_000_000 else 0.0)
    assert in_band.sum() <= max(allowed, BAND_FLOOR), (
        f"{in_band.sum()} of {in_band.size} coordinates within {BAND} of a boundary")
    return in_band.any(axis=1), {"band_fraction": float(frac), "code_mismatches": int(mism.sum()),
                                 "band_count": int(in_band.sum())}


def compare_signs(p, gpu_words, diag, exclude):
    gs = K.unpack_signs(gpu_words, p.m)
    os_ = (diag.z >= 0.0).astype(np.int64)
    mism = (gs != os_) & ~exclude[:, None]
    outside = mism & (np.abs(diag.z) >= BAND)
    assert not outside.any(), f"{outside.sum()} sign mismatches outside the band (z = {diag.z[outside][:5]})"
    return int(mism.sum())


def compare_recon(gpu, oracle, nhat, what="reconstruction", tol=RECON_TOL, rows=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    oracle = np.asarray(oracle, dtype=np.float64)
    err = np.abs(gpu - oracle).max(axis=1)
    lim = tol * np.maximum(nhat, 1e-30) + 0.0
    if rows is not None:
        err = err[rows]
        lim = lim[rows]
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} vectors over tolerance; worst {np.max(err / np.maximum(lim, 1e-300))}x"
    return float(np.max(err / np.maximum(lim, 1e-300))) if err.size else 0.0


def record_from_host(codes, norms, signs, rnorms):
    return K.Record(codes.astype(np.uint32), norms.astype(np.uint16),
                    None if signs is None else signs.astype(np.uint32),
                    None if rnorms is None else rnorms.astype(np.uint16))


def check_records(p, x, codes, norms, signs, rnorms):
    """Codes, norms, sign bits and residual norms of GPU records against the
    oracle's quantisation of the same input rows.  Returns (oracle record,
    diagnostics, band mask per vector, code report)."""
    orec, diag = K.quantize(p, np.asarray(x, dtype=np.float64))
    excl, rep = compare_codes(p, codes, diag)
    compare_halves(norms, diag.n, "norms")
    if p.qjl:
        compare_signs(p, signs, diag, excl)
        compare_halves(rnorms[~excl], diag.gamma[~excl], "rnorms")
    return orec, diag, excl, rep


def compare_scores(got, ref, qnorm, nhat, what="scores"):
    """|gpu - oracle| <= SCORE_TOL * ||q|| * n^ elementwise (broadcasting)."""
    got = np.asarray(got, dtype=np.float64)
    lim = SCORE_TOL * qnorm * nhat + 1e-30
    err = np.abs(got - ref)
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} over tolerance, worst {np.max(err / lim):.3g}x"
    return float(np.max(err / lim)) if err.size else 0.0


# ---------------------------------------------------------------- PolarQuant --
# Angle codes: a code that differs from the oracle's must have the oracle's
# pair point (a, b) of that level (unit-vector domain, y = Pi x / ||x||)
# within BAND of its nearest decision ray (perpendicular distance
# r |sin(theta - t)|; level 1 also has the ray at angle 0); the fraction of
# points inside the band obeys the same bound as the codec's coordinates.
# The kernel's point carries the rotation's error (a few 1e-7 in this domain)
# plus the fp32 rounding of its boundary constants, below BAND.
# Radii: half bits equal unless the float64 radius lies within
# POLAR_RADIUS_BAND (relative) of a half rounding midpoint; the kernel's
# radius carries the rotation's error through up to 16 coordinates and the
# fp32 norm (about 1e-6 relative at worst), hence twice the codec's 1e-6.
POLAR_RADIUS_BAND = 2e-6


def polar_level_points(p, x):
    """Per level, (a, b) of every pair in the unit-vector domain, float64."""
    from oracle import polar as PQ
    x = np.asarray(x, dtype=np.float64)
    nrm = np.linalg.norm(x, axis=1)
    y = (x @ p.pi.T) / np.where(nrm > 0, nrm, 1.0)[:, None]
    pairs, _ = PQ.polar_pairs(y)
    return [(pr[..., 0], pr[..., 1]) for pr in pairs]


def polar_ray_distance(p, level, a, b):
    """Perpendicular distance of (a, b) to the nearest decision ray of the level."""
    t = np.asarray(p.books[level][1], dtype=np.float64)
    if level == 0:
        t = np.concatenate([[0.0], t])
    th = np.arctan2(b, a)
    r = np.sqrt(a * a + b * b)
    d = np.abs(np.mod(th[..., None] - t + np.pi, 2.0 * np.pi) - np.pi).min(axis=-1)
    return r * np.sin(np.minimum(d, np.pi / 2.0))


def check_polar_words(p, x, gpu_words):
    """GPU PolarQuant records against the oracle's quantisation of x.
    Returns a report."""
    from oracle import polar as PQ
    x = np.asarray(x, dtype=np.float64)
    owords, diag = PQ.quantize(p, x)
    gc, grb = PQ.unpack(gpu_words)
    oc, orb = PQ.unpack(owords)
    pts = polar_level_points(p, x)
    zero = np.linalg.norm(x, axis=1) == 0      # every angle 0 on both sides: exact, not banded
    n_band = n_mism = n_all = 0
    for level in range(PQ.N_LEVELS):
        assert np.all(gc[level][zero] == 0) and np.all(oc[level][zero] == 0)
        dist = polar_ray_distance(p, level, *pts[level])[~zero]
        in_band = dist < BAND
        mism = (gc[level] != oc[level])[~zero]
        outside = mism & ~in_band
        assert not outside.any(), (
            f"level {level + 1}: {outside.sum()} angle codes differ outside the band; first at "
            f"{np.argwhere(outside)[0]} gpu {gc[level][outside][:5]} oracle {oc[level][outside][:5]} "
            f"distance {dist[outside][:5]}")
        n_band += int(in_band.sum())
        n_mism += int(mism.sum())
        n_all += in_band.size
    expected = BAND_FRACTION * n_all
    allowed = expected + (3.0 * np.sqrt(expected) if n_all < 1_000_000 else 0.0)
    assert n_band <= max(allowed, BAND_FLOOR), f"{n_band} of {n_all} angles within {BAND} of a decision ray"
    rel = half_midpoint_distance(diag.radii)
    bad = (grb != orb) & (rel > POLAR_RADIUS_BAND)
    assert not bad.any(), f"{bad.sum()} radius halves differ away from a rounding midpoint"
    return {"band_count": n_band, "code_mismatches": n_mism, "radius_mismatches": int((grb != orb).sum()),
            "angles": n_all}


def polar_radius_norm(words):
    from oracle import polar as PQ
    _, rb = PQ.unpack(words)
    r = rb.view(np.float16).astype(np.float64)
    return np.linalg.norm(r, axis=1)
