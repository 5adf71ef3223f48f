"""Pins for the oracle's generator and Cl(3,0) algebra (CPU only)."""
import math

import numpy as np
import pytest
from scipy import stats

from conftest import golden
from oracle import clifford as C
from oracle import prng


# ------------------------------------------------------------------ PRNG ---
def test_splitmix64_reference_sequence():
    g = golden("splitmix64_seed0.json")
    s = prng.SplitMix64(g["seed"])
    assert [s.next_u64() for _ in range(5)] == [int(v, 16) for v in g["outputs"]]


def test_stream_zero_tag_is_plain_splitmix():
    a = prng.stream(12345, 0)
    b = prng.SplitMix64(12345)
    assert [a.next_u64() for _ in range(4)] == [b.next_u64() for _ in range(4)]


def test_uniform_open_interval_and_resolution():
    g = prng.SplitMix64(0)
    u = [g.uniform() for _ in range(20000)]
    assert 0.0 < min(u) and max(u) < 1.0
    # u = ((w >> 11) + 1/2) 2^-53: below 1/2 the half-step is representable,
    # so u * 2^53 sits exactly half-way between integers.
    low = [x for x in u if x < 0.5]
    assert len(low) > 9000
    assert all(((x * 2.0 ** 53) % 1.0) == 0.5 for x in low)


def test_box_muller_pair_structure():
    # z0^2 + z1^2 = -2 ln u1 and atan2(z1, z0) = 2 pi u2 (mod 2 pi).
    g = prng.stream(5, 1)
    u1, u2 = g.uniform(), g.uniform()
    z0, z1 = prng.normals(5, 1, 2)
    assert math.isclose(z0 * z0 + z1 * z1, -2.0 * math.log(u1), rel_tol=1e-14)
    ang = math.atan2(z1, z0) % (2 * math.pi)
    assert math.isclose(ang, (2 * math.pi * u2) % (2 * math.pi), rel_tol=1e-12, abs_tol=1e-12)


def test_normal_moments_and_ks():
    z = np.array(prng.normals(0, 3, 200000))
    assert abs(z.mean()) < 0.01            # 4.5 SE
    assert abs(z.var() - 1.0) < 0.015      # 4.7 SE
    assert stats.kstest(z, "norm").pvalue > 1e-3


def test_streams_differ_by_tag_and_seed():
    a = prng.normals(0, 1, 8)
    b = prng.normals(0, 2, 8)
    c = prng.normals(1, 1, 8)
    assert a != b and a != c


# ------------------------------------------------------------- Cl(3,0) ---
def _basis(name):
    v = np.zeros(8)
    v[C.BASIS_NAMES.index(name)] = 1.0
    return v


def test_cayley_table_against_hand_derived_products():
    for left, right, sign, res in golden("cl3_products.json")["products"]:
        out = C.gp(_basis(left), _basis(right))
        assert np.array_equal(out, sign * _basis(res)), (left, right, out)


def test_geometric_product_associative_and_distributive():
    rng = np.random.default_rng(0)
    a, b, c = rng.normal(size=(3, 8))
    assert np.allclose(C.gp(C.gp(a, b), c), C.gp(a, C.gp(b, c)), atol=1e-13)
    assert np.allclose(C.gp(a, b + c), C.gp(a, b) + C.gp(a, c), atol=1e-13)


def test_vector_square_is_norm_squared():
    v = np.array([0.3, -1.2, 2.0])
    sq = C.gp(C.embed_vector(v), C.embed_vector(v))
    assert np.allclose(sq, np.r_[v @ v, np.zeros(7)], atol=1e-15)


@pytest.fixture
def rotors():
    rng = np.random.default_rng(3)
    return [C.rotor_from_bivector(*rng.normal(size=3)) for _ in range(20)]


def test_rotor_unit_and_sparse(rotors):
    for r in rotors:
        assert np.allclose(C.gp(r, C.reverse(r)), np.r_[1.0, np.zeros(7)], atol=1e-14)
        assert r[1] == r[2] == r[3] == r[7] == 0.0


def test_sandwich_properties(rotors):
    rng = np.random.default_rng(4)
    for r in rotors:
        v = rng.normal(size=3)
        out = C.sandwich(r, v)
        # pure grade 1: scalar, bivector and trivector parts vanish
        assert np.allclose(out[[0, 4, 5, 6, 7]], 0.0, atol=1e-14)
        assert math.isclose(np.linalg.norm(out[1:4]), np.linalg.norm(v), rel_tol=1e-14)
        back = C.inverse_sandwich(r, out[1:4])
        assert np.allclose(back[1:4], v, atol=1e-14)
        m = C.rotation_matrix_bruteforce(r)
        assert np.allclose(m @ m.T, np.eye(3), atol=1e-14)
        assert math.isclose(np.linalg.det(m), 1.0, rel_tol=1e-13)
        assert np.allclose(C.quaternion_matrix(r), m, atol=1e-14)
        assert np.allclose(m @ v, out[1:4], atol=1e-14)


def test_rotation_angle_is_twice_bivector_norm():
    b = np.array([0.3, -0.4, 0.5])
    th = np.linalg.norm(b)
    m = C.rotation_matrix_bruteforce(C.rotor_from_bivector(*b))
    # trace of a rotation by phi is 1 + 2 cos(phi); the sandwich turns by 2|b|
    assert math.isclose(np.trace(m), 1 + 2 * math.cos(2 * th), rel_tol=1e-13)


def test_left_product_used_twice_is_the_identity_bug():
    """README 'Non-Commutative Algebra Bug Fix': computing R~ (R x) instead
    of (R x) R~ gives back x; the real sandwich is not the identity."""
    rng = np.random.default_rng(5)
    for _ in range(5):
        r = C.rotor_from_bivector(*rng.normal(size=3))
        v = rng.normal(size=3)
        bug = C.gp(C.reverse(r), C.gp(r, C.embed_vector(v)))
        assert np.allclose(bug[1:4], v, atol=1e-14)
        assert np.abs(C.sandwich(r, v)[1:4] - v).max() > 1e-3


def test_rotor_times_vector_has_vector_and_trivector_only(rotors):
    # README "The Fused CUDA Kernel": grade-1 input gives vector + trivector.
    v = np.array([0.2, 0.7, -0.4])
    for r in rotors:
        rv = C.gp(r, C.embed_vector(v))
        assert np.allclose(rv[[0, 4, 5, 6]], 0.0, atol=1e-15)


def test_blog_2d_example():
    g = golden("blog_2d_example.json")
    x = np.array(g["x"])
    assert np.linalg.norm(x) == g["norm"]
    u = x / np.linalg.norm(x)
    assert np.allclose(u, g["unit"], atol=1e-15)
    y = np.array(g["rot90_ccw"]) @ u
    assert np.allclose(y, g["rotated"], atol=1e-15)
    assert math.isclose(np.linalg.norm(y), 1.0, rel_tol=1e-15)
    # the same turn as a Cl(3,0) rotor in the e1-e2 plane: angle 2|b12| = -90 deg
    r = C.rotor_from_bivector(-math.pi / 4, 0.0, 0.0)
    assert np.allclose(C.sandwich(r, np.r_[u, 0.0])[1:3], g["rotated"], atol=1e-15)
