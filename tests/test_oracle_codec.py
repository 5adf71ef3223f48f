"""Pins for the oracle's parameter tables and codec (CPU only)."""
import math

import numpy as np
import pytest

from conftest import golden
from oracle import clifford as C
from oracle import codec as K
from oracle import lloyd_max as L
from oracle import params as P
from oracle import theory as T
from kv_cache_vector_norm_amd import workloads as W

D = 128


# ------------------------------------------------------------ parameters ---
def test_rotor_table_unit_rotors():
    r = P.rotor_table(D, 0)
    assert r.shape == (43, 4)
    # fp32-rounded unit rotors: s^2 + |b|^2 = 1 to fp32 rounding
    assert np.abs((r ** 2).sum(1) - 1.0).max() < 4e-7
    assert np.array_equal(r, r.astype(np.float32).astype(np.float64))


def test_pi_is_the_sign_fixed_qr_factor():
    from oracle import prng
    g = np.array(prng.normals(0, prng.TAG_PI, D * D)).reshape(D, D)
    q = P.gram_schmidt_q(g)
    assert np.abs(q.T @ q - np.eye(D)).max() < 1e-13
    r = q.T @ g
    assert np.abs(np.tril(r, -1)).max() < 1e-11
    assert np.all(np.diag(r) > 0)
    # same factor as a Householder QR with the sign of R's diagonal fixed
    qn, rn = np.linalg.qr(g)
    qn = qn * np.sign(np.diag(rn))
    assert np.abs(qn - q).max() < 1e-12


def test_s_is_half_rounded_gaussian():
    s = P.s_matrix(D, 0)
    assert np.array_equal(s, s.astype(np.float16).astype(np.float64))
    assert abs(s.mean()) < 0.02 and abs(s.var() - 1) < 0.03


def test_params_modes():
    p = P.Params(D, 3, 0, P.QJL)
    assert p.b_m == 2 and p.s is not None and p.rotors is not None and p.n_coords == 129
    p = P.Params(D, 3, 0, P.DENSE)
    assert p.b_m == 3 and p.pi is not None and p.rotors is None and p.n_coords == 128
    with pytest.raises(ValueError):
        P.Params(D, 5, 0, P.MSE)


# --------------------------------------------------------------- packing ---
def test_pack_hand_example():
    # codes 1, 2, 3 at 2 bits: 0b11_10_01 = 57
    assert K.pack_codes(np.array([[1, 2, 3]]), 2)[0, 0] == 57
    # 3-bit code index 10 straddles words: bits 30, 31 | 32
    codes = np.zeros((1, 12), dtype=np.int64)
    codes[0, 10] = 0b101
    w = K.pack_codes(codes, 3)
    assert w.shape == (1, 2)
    assert w[0, 0] == 1 << 30 and w[0, 1] == 1


@pytest.mark.parametrize("b,n", [(1, 129), (2, 129), (3, 129), (4, 129), (3, 128), (1, 128)])
def test_pack_roundtrip_and_width(b, n):
    rng = np.random.default_rng(b)
    codes = rng.integers(0, 1 << b, size=(50, n))
    w = K.pack_codes(codes, b)
    assert w.shape[1] == -(-(n * b) // 32)
    assert np.array_equal(K.unpack_codes(w, b, n), codes)


def test_half_rounding_is_nearest_even():
    one = 1.0
    assert K.half_bits(one + 2.0 ** -11)[()] == K.half_bits(1.0)[()]       # tie -> even
    assert K.half_bits(one + 3 * 2.0 ** -11)[()] == K.half_bits(1.0 + 2.0 ** -9)[()]  # tie -> even (up)
    assert K.half_bits(one + 2.0 ** -11 + 2.0 ** -30)[()] == K.half_bits(1.0 + 2.0 ** -10)[()]


# ----------------------------------------------------------- transforms ---
@pytest.mark.parametrize("d", [3, 6, 128])
def test_exact_inverse_without_quantisation(d):
    p = P.Params(d, 3, 11, P.MSE)
    p.rotors = P.rotor_table(d, 11, round_f32=False)   # exactly unit rotors
    rng = np.random.default_rng(d)
    x = rng.normal(size=(20, d))
    y = K.forward(p, x)
    assert np.allclose(K.inverse(p, y), x, atol=1e-14)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_rotor_forward_matches_quaternion_matrices():
    p = P.Params(D, 3, 2, P.MSE)
    p.rotors = P.rotor_table(D, 2, round_f32=False)    # exactly unit rotors
    rng = np.random.default_rng(2)
    x = rng.normal(size=(7, D))
    y, full = K.rotor_forward(p, x)
    v = np.zeros((7, 129))
    v[:, :D] = x
    for g in range(43):
        m = C.quaternion_matrix(C.rotor(*p.rotors[g]))
        assert np.allclose(y[:, 3 * g:3 * g + 3], v[:, 3 * g:3 * g + 3] @ m.T, atol=1e-14)
    # the trivector (and scalar, bivector) parts of every group vanish
    assert np.abs(full[:, :, [0, 4, 5, 6, 7]]).max() < 1e-14
    # the forward map is not the identity (non-commutativity fix)
    assert np.abs(y[:, :D] - x).max() > 1e-2


def test_tq_exact_inverse_with_float64_pi():
    p = P.Params(D, 3, 0, P.DENSE)
    p.pi = P.pi_matrix(D, 0, round_f32=False)
    x = np.random.default_rng(0).normal(size=(5, D))
    assert np.allclose(K.inverse(p, K.forward(p, x)), x, atol=1e-13)


def test_nearest_centroid_bruteforce():
    for b in (1, 2, 3, 4):
        p = P.Params(D, b, 0, P.MSE)
        y = np.random.default_rng(b).normal(scale=0.15, size=5000)
        nearest = np.abs(y[:, None] - p.centroids[None, :]).argmin(1)
        assert np.array_equal(K.scalar_quantize(p, y), nearest)


def test_tie_goes_to_lower_index():
    p = P.Params(D, 2, 0, P.MSE)
    y = p.boundaries.copy()
    assert np.array_equal(K.scalar_quantize(p, y), np.arange(len(y)))


def test_zero_vector():
    for mode in (P.MSE, P.QJL, P.DENSE, P.DENSE | P.QJL):
        p = P.Params(D, 3, 0, mode)
        rec, diag = K.quantize(p, np.zeros((1, D)))
        assert K.half_value(rec.norms)[0] == 0.0
        assert np.all(K.dequantize(p, rec) == 0.0)


def test_blog_norm_separation():
    g = golden("blog_2d_example.json")
    p = P.Params(D, 4, 0, P.MSE)
    x = np.zeros((1, D))
    x[0, :2] = g["x"]
    rec, diag = K.quantize(p, x)
    assert diag.n[0] == g["norm"] and K.half_value(rec.norms)[0] == g["norm"]


# ------------------------------------------------------------ quality ---
def test_1024_unit_vectors_mse_and_cosine():
    x = W.unit_vectors_1024().astype(np.float64)
    g = golden("readme_mse_table.json")
    for row in g["rows"]:
        p = P.Params(D, row["bits"], 0, P.MSE)
        rec, xt, _ = K.roundtrip(p, x)
        err = ((x - xt) ** 2).sum(1)
        assert abs(err.mean() - row["mse"]) < max(4 * err.std() / math.sqrt(len(err)), 6e-4)
        cos = ((x * xt).sum(1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xt, axis=1)).mean()
        assert abs(cos - row["cosine"]) < 2e-3


@pytest.mark.parametrize("mode", [P.MSE, P.DENSE])
def test_rq_and_tq_match_the_integral(mode):
    x = W.unit_gaussian(8000, seed=5).astype(np.float64)
    for b in (2, 3):
        p = P.Params(D, b, 0, mode)
        rec, xt, _ = K.roundtrip(p, x)
        err = ((x - xt) ** 2).sum(1)
        assert abs(err.mean() - L.beta_unit_mse(p.centroids, D)) < 4 * err.std() / math.sqrt(len(err)) + 2e-4


def test_score_equals_dot_with_dequantised_key():
    p = P.Params(D, 3, 0, P.QJL)
    x = W.gaussian(300, seed=3).astype(np.float64)
    q = W.queries(5, seed=4).astype(np.float64)
    rec, _ = K.quantize(p, x)
    assert np.allclose(K.score(p, q, rec), q @ K.dequantize(p, rec).T, rtol=1e-12, atol=1e-10)


def test_gqa_mapping():
    p = P.Params(D, 3, 0, P.QJL)
    x = W.gaussian(2 * 50, seed=3).astype(np.float64)
    q = W.queries(4, seed=4).astype(np.float64)
    rec, _ = K.quantize(p, x)
    s = K.score_gqa(p, q, rec, group=2, t=50)
    full = K.score(p, q, rec)
    assert np.allclose(s[:2], full[:2, :50]) and np.allclose(s[2:], full[2:, 50:])


# ----------------------------------------------------- QJL statistics ---
def _with_s(p, s):
    p.s = s
    return p


def test_qjl_unbiased_and_variance_over_gaussian_s():
    """Lemma 4: E_S <y, x~_qjl> = <y, r>; the variance is
    ((pi/2)|r|^2|y|^2 - <y,r>^2)/m and below pi/(2d) |r|^2 |y|^2."""
    p = P.Params(D, 3, 0, P.QJL)
    rng = np.random.default_rng(9)
    x = rng.normal(size=(1, D))
    y = rng.normal(size=D)
    rec0, _ = K.quantize(p, x)
    nhat, xmse, _, _ = K.decode(p, rec0)
    xu = x[0] / np.linalg.norm(x[0])
    r = xu - xmse[0]
    est = []
    for _ in range(3000):
        _with_s(p, rng.normal(size=(D, D)))
        rec, diag = K.quantize(p, x)
        s = K.score(p, y[None, :], rec)[0, 0] / nhat[0] - y @ xmse[0]
        est.append(s * diag.gamma[0] / K.half_value(rec.rnorms)[0])   # undo gamma's half rounding
    est = np.array(est)
    target = y @ r
    assert abs(est.mean() - target) < 4 * est.std() / math.sqrt(len(est))
    var_exact = T.qjl_variance_exact(D, r, y)
    assert abs(est.var() / var_exact - 1) < 0.1
    assert var_exact <= T.lemma4_var_bound(D, r @ r, y @ y)


def test_half_rounded_s_shows_no_detectable_bias():
    p = P.Params(D, 3, 0, P.QJL)
    rng = np.random.default_rng(10)
    x = rng.normal(size=(1, D))
    y = rng.normal(size=D)
    exact = []
    for _ in range(1500):
        _with_s(p, rng.normal(size=(D, D)).astype(np.float16).astype(np.float64))
        rec, _ = K.quantize(p, x)
        exact.append(K.score(p, y[None], rec)[0, 0])
    exact = np.array(exact)
    rec, _ = K.quantize(p, x)
    nhat, xmse, _, _ = K.decode(p, rec)
    # unbiased for <y, x> up to the stored norms' half rounding
    xu = x[0] / np.linalg.norm(x[0])
    assert abs(exact.mean() - nhat[0] * (y @ xu)) < 4 * exact.std() / math.sqrt(len(exact)) + 1e-3 * abs(nhat[0] * (y @ xu))


def test_theorem2_prod_distortion_bound():
    rng = np.random.default_rng(11)
    for b in (2, 3):
        p = P.Params(D, b, 0, P.QJL)
        x = W.unit_gaussian(400, seed=12 + b).astype(np.float64)
        y = rng.normal(size=D)
        y /= np.linalg.norm(y)
        errs = []
        for _ in range(20):
            _with_s(p, rng.normal(size=(D, D)))
            rec, _ = K.quantize(p, x)
            errs.append((K.score(p, y[None], rec)[0] - x @ y) ** 2)
        assert np.mean(errs) <= T.thm2_upper(b, D)


def test_one_bit_shrinkage_over_haar_rotations():
    """1-bit TurboQuant: E_Pi <q, x~> = kappa <q, x>, kappa = d (E|X|)^2."""
    d = 32
    rng = np.random.default_rng(13)
    p = P.Params(d, 1, 0, P.DENSE)
    x = rng.normal(size=(1, d))
    x /= np.linalg.norm(x)
    q = x[0] + 0.5 * rng.normal(size=d)
    ratios = []
    for _ in range(3000):
        qq, rr = np.linalg.qr(rng.normal(size=(d, d)))
        p.pi = qq * np.sign(np.diag(rr))
        rec, _ = K.quantize(p, x)
        nhat, xmse, _, _ = K.decode(p, rec)
        ratios.append((q @ xmse[0]) / (q @ x[0]))
    ratios = np.array(ratios)
    kappa = T.one_bit_shrinkage(d)
    assert abs(ratios.mean() - kappa) < 4 * ratios.std() / math.sqrt(len(ratios))


# --------------------------------------------------------------- needle ---
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("t", [512, 2048, 8192])
def test_synthetic_needle(bits, t):
    p = P.Params(D, bits, 0, P.QJL)
    keys, q, idx = W.needle_keys(t, seed=bits * 100 + t)
    rec, _ = K.quantize(p, keys.astype(np.float64))
    s = K.score(p, q[None].astype(np.float64), rec)[0]
    assert int(np.argmax(s)) == idx


# --------------------------------------------------------------- counts ---
def test_page_counts():
    g = golden("counts.json")
    assert T.tq_param_count(128, 3) == g["tq_params"]
    lo, hi = g["rq_params_range"]
    assert lo <= T.rq_param_count(128, 3) <= hi
    assert abs(T.rq_param_count(4096, 3) - g["rq_params_d4096_approx"]) / g["rq_params_d4096_approx"] < 0.01
    assert abs(T.tq_param_count(4096, 3) - g["tq_params_d4096_approx"]) / g["tq_params_d4096_approx"] < 0.01
    assert T.sandwich_fma_per_group() == g["fma_per_group"]
    assert T.sandwich_fma_per_vector(128) == g["fma_sandwich_per_vector"]
    assert T.dense_rotation_fma(128) == g["tq_rotation_fma"]
    assert P.n_groups(128) == g["groups"] and T.rq_param_count_compact(128) == g["stored_indices_rq"]
    assert round(T.compression_ratio(128, g["stored_indices_tq"], 3), 1) == g["compression_3bit_tq"]
    assert round(T.compression_ratio(128, g["stored_indices_rq"], 3), 1) == g["compression_3bit_rq"]


def test_sparse_product_structure_counts():
    """README 'FMA Count': R * v (grade-1 v, 3 non-zero) has 4 non-zero
    outputs; (R v) * R~ has 4 non-zero inputs.  Count from the Cayley table."""
    r_support = [0, 4, 5, 6]
    v_support = [1, 2, 3]
    outs = {int(np.nonzero(C.CAYLEY[i, j])[0][0]) for i in r_support for j in v_support}
    assert sorted(outs) == [1, 2, 3, 7]


# ------------------------------------------------ QJL only (one bit) ---
def test_qjl_only_record_is_the_sign_sketch_of_the_unit_vector():
    """With zero MSE bits the residual is the whole unit vector: no codes,
    gamma = 1 (the blog's QJL demo sets exactly this), and the record is
    the norm plus sign(S x_u)."""
    p = P.Params(D, 1, 0, P.QJL)
    assert p.b_m == 0 and K.code_words(p.n_coords, p.b_m) == 0
    x = W.gaussian(50, seed=30).astype(np.float64)
    x[7] = 0.0
    rec, diag = K.quantize(p, x)
    assert rec.codes.shape == (50, 0)
    g = K.half_value(rec.rnorms)
    assert np.all(np.delete(g, 7) == 1.0) and g[7] == 0.0
    nhat, xmse, ghat, sigma = K.decode(p, rec)
    assert np.all(xmse == 0.0)
    # the sign of every projection agrees with S applied to the unit vector
    xu = x / np.where(np.linalg.norm(x, axis=1) > 0, np.linalg.norm(x, axis=1), 1.0)[:, None]
    z = xu @ p.s.T
    ok = np.abs(z) > 1e-12
    assert np.array_equal((sigma > 0)[ok], (z >= 0)[ok])


def test_qjl_only_estimator_and_reconstruction_are_unbiased():
    """E_S of the one-bit inner-product estimate is <q, x> (Lemma 4 with
    r = x_u), its variance is the closed form of Lemma 4, and E_S of the
    dequantised vector is x itself (sqrt(pi/2)/m undoes E|s^T x_u| shrinkage)."""
    p = P.Params(D, 1, 0, P.QJL)
    rng = np.random.default_rng(31)
    x = rng.normal(size=(1, D))
    q = rng.normal(size=D)
    xu = x[0] / np.linalg.norm(x[0])
    est, rec_sum = [], np.zeros(D)
    for _ in range(3000):
        _with_s(p, rng.normal(size=(D, D)))
        rec, _ = K.quantize(p, x)
        nhat = K.half_value(rec.norms)[0]
        est.append(K.score(p, q[None], rec)[0, 0] / nhat)
        rec_sum += K.dequantize(p, rec)[0] / nhat
    est = np.array(est)
    assert abs(est.mean() - q @ xu) < 4 * est.std() / math.sqrt(len(est))
    assert abs(est.var() / T.qjl_variance_exact(D, xu, q) - 1) < 0.1
    mean_rec = rec_sum / 3000
    # per coordinate, kappa S^T sigma has variance about pi / (2 m)
    assert np.abs(mean_rec - xu).max() < 5 * math.sqrt(math.pi / (2 * D) / 3000)
