"""Cl(3,0) geometric algebra, written out plainly (test infrastructure only).

Sources: RotorQuant README, "How RotorQuant Works" (multivector basis
[1, e1, e2, e3, e12, e13, e23, e123]; a rotor has the four non-zero
components [s, 0, 0, 0, b12, b13, b23, 0]) and "Non-Commutative Algebra Bug
Fix" (the sandwich is (R * x) * R~: R on the left first, then R~ on the
right).  The algebra has e_i e_i = +1 and e_i e_j = -e_j e_i for i != j.

Everything here is float64 and uses the full 8x8 product; nothing exploits
sparsity.  The sparse, matrix or quaternion forms are checked against this
module by the tests, never the other way round.
"""
import math

import numpy as np

# Basis order of the pages, as bitmasks over (e1, e2, e3).
BASIS_NAMES = ("1", "e1", "e2", "e3", "e12", "e13", "e23", "e123")
BASIS_MASKS = (0b000, 0b001, 0b010, 0b100, 0b011, 0b101, 0b110, 0b111)
_INDEX_OF_MASK = {m: i for i, m in enumerate(BASIS_MASKS)}
GRADE = np.array([bin(m).count("1") for m in BASIS_MASKS])


def _blade_product(ma, mb):
    """(sign, mask) of the product of two basis blades.

    Each blade is the ordered product of its generators.  Moving every
    generator of the right blade leftwards past the generators of the left
    blade with a larger index costs one sign flip per transposition; equal
    generators then cancel because e_i e_i = +1 in Cl(3,0).
    """
    swaps = 0
    for j in range(3):
        if mb >> j & 1:
            for i in range(j + 1, 3):
                if ma >> i & 1:
                    swaps += 1
    return (-1.0 if swaps % 2 else 1.0), ma ^ mb


def cayley_tensor():
    """T[i, j, k] such that (a b)_k = sum_ij a_i b_j T[i, j, k]."""
    t = np.zeros((8, 8, 8))
    for i, ma in enumerate(BASIS_MASKS):
        for j, mb in enumerate(BASIS_MASKS):
            s, m = _blade_product(ma, mb)
            t[i, j, _INDEX_OF_MASK[m]] = s
    return t


CAYLEY = cayley_tensor()


def gp(a, b):
    """Full geometric product of multivectors a and b (last axis 8)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.einsum("...i,...j,ijk->...k", a, b, CAYLEY)


def reverse(a):
    """Reversion: grade k picks up (-1)^(k(k-1)/2), i.e. grades 2, 3 flip."""
    a = np.array(a, dtype=np.float64, copy=True)
    a[..., GRADE >= 2] *= -1.0
    return a


def grade_part(a, k):
    a = np.asarray(a, dtype=np.float64)
    return a * (GRADE == k)


def embed_vector(v):
    """Grade-1 embedding of 3-vectors (last axis 3) into multivectors."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape[:-1] + (8,))
    out[..., 1:4] = v
    return out


def rotor(s, b12, b13, b23):
    """Rotor multivector [s, 0, 0, 0, b12, b13, b23, 0]."""
    return np.array([s, 0.0, 0.0, 0.0, b12, b13, b23, 0.0])


def rotor_from_bivector(b12, b13, b23):
    """exp of the bivector B = b12 e12 + b13 e13 + b23 e23, normalised.

    B squares to -|b|^2, so exp(B) = cos|b| + (sin|b| / |b|) B.  The result
    is then divided by sqrt(<R R~>_0) so that R R~ = 1 holds to rounding.
    This is the reading of "normalized random bivector exponentials" used
    for the rotor tables.  Scalar libm functions are used (``math``), so the
    float64 values are those of the C library.
    """
    b12, b13, b23 = float(b12), float(b13), float(b23)
    th = math.sqrt(b12 * b12 + b13 * b13 + b23 * b23)
    k = math.sin(th) / th if th > 0.0 else 1.0
    r = rotor(math.cos(th), k * b12, k * b13, k * b23)
    n2 = gp(r, reverse(r))[0]
    return r / math.sqrt(n2)


def sandwich(r, v):
    """(R V) R~ with V the grade-1 embedding of v; returns all 8 parts."""
    return gp(gp(r, embed_vector(v)), reverse(r))


def inverse_sandwich(r, v):
    """(R~ V) R, the inverse map used on dequantisation."""
    return gp(gp(reverse(r), embed_vector(v)), r)


def rotation_matrix_bruteforce(r):
    """3x3 M with grade-1 of (R v) R~ == M v, column j = image of e_j."""
    m = np.zeros((3, 3))
    for j in range(3):
        e = np.zeros(3)
        e[j] = 1.0
        m[:, j] = sandwich(r, e)[1:4]
    return m


def quaternion_matrix(r):
    """Rotation matrix of the quaternion that corresponds to rotor r.

    With e12, e13, e23 identified with quaternion units, the rotor
    [s, b12, b13, b23] acts as the unit quaternion (w, x, y, z) =
    (s, -b23, b13, -b12); the usual quaternion rotation matrix then equals
    the sandwich map.  Used only as an independent cross-check.
    """
    s, b12, b13, b23 = r[0], r[4], r[5], r[6]
    w, x, y, z = s, -b23, b13, -b12
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
        [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
        [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)],
    ])
