"""Parameter tables of a codec session, from (d, bits, seed, mode).

Test infrastructure only.  Each table is computed in float64 and rounded
once to the precision the codec stores it in; the oracle then does all its
arithmetic in float64 on those rounded values.

Sources:
* RotorQuant README, "How RotorQuant Works": one rotor
  [s, 0, 0, 0, b12, b13, b23, 0] per group of three coordinates,
  ceil(d/3) = 43 groups at d = 128 (section "Why Rotors?").
* RotorQuant README, "Codebook Calibration Fix": one codebook, built for the
  coordinate law of a unit vector with d_eff = d.
* RotorQuant README, "How TurboQuant Works", Stage 1: Pi is the orthogonal
  factor of the QR decomposition of a Gaussian matrix; PolarQuant article,
  "Шаг 1": the random matrix is orthogonalised by Gram-Schmidt.
* Same README, Stage 2 and its estimator formula: S is a Gaussian m x d
  projection; here m = d = 128.
* Blog, QJL section, and hyper.ai "方法" (Algorithm 2): with QJL, b total
  bits per coordinate are b - 1 bits of MSE codes plus 1 sign bit.

Readings where the pages are silent:
* Rotor draw: three N(0,1) bivector coefficients per group, in group order,
  exponentiated and normalised (see clifford.rotor_from_bivector).
* Pi: modified Gram-Schmidt with one re-orthogonalisation pass on the
  columns of a row-major filled Gaussian matrix G, so that G = Q R with
  diag(R) > 0; Pi = Q, and the rotation is y = Pi x.
* S: row-major N(0,1) draws, each rounded to the nearest IEEE half; that
  rounded matrix *is* S (the pages fix only that S is Gaussian).
* Every table is rounded to fp32 except S (fp16 values).
"""
import math

import numpy as np

from . import clifford, lloyd_max, prng

MSE = 0
QJL = 1
DENSE = 2


def n_groups(d):
    return -(-d // 3)


def mse_bits(bits, mode):
    return bits - 1 if mode & QJL else bits


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rotor_table(d, seed, round_f32=True):
    """[G, 4] rotors (s, b12, b13, b23), fp32-rounded, as float64."""
    g = n_groups(d)
    z = prng.normals(seed, prng.TAG_ROTORS, 3 * g)
    out = np.zeros((g, 4))
    for i in range(g):
        r = clifford.rotor_from_bivector(z[3 * i], z[3 * i + 1], z[3 * i + 2])
        out[i] = (r[0], r[4], r[5], r[6])
    return f32(out) if round_f32 else out


def rotor_matrices(rotors):
    """[G, 3, 3] float64 matrices of the fp32 rotors, by brute force."""
    return np.stack([clifford.rotation_matrix_bruteforce(clifford.rotor(*r)) for r in rotors])


def codebook(bits, d):
    """(centroids, boundaries), fp32-rounded, as float64.

    Boundaries are the float64 midpoints of the float64 centroids, each
    rounded once to fp32.
    """
    c, t = lloyd_max.beta_codebook(bits, d)
    return f32(c), f32(t)


def gram_schmidt_q(g):
    """Q of G = Q R with diag(R) > 0: modified Gram-Schmidt, re-orthogonalised."""
    n = g.shape[1]
    q = np.zeros_like(g)
    for j in range(n):
        v = g[:, j].copy()
        for _ in range(2):
            for i in range(j):
                v -= np.dot(q[:, i], v) * q[:, i]
        q[:, j] = v / np.linalg.norm(v)
    return q


def pi_matrix(d, seed, round_f32=True):
    g = np.array(prng.normals(seed, prng.TAG_PI, d * d)).reshape(d, d)
    q = gram_schmidt_q(g)
    return f32(q) if round_f32 else q


def s_matrix(d, seed):
    z = np.array(prng.normals(seed, prng.TAG_S, d * d)).reshape(d, d)
    return z.astype(np.float16).astype(np.float64)


class Params:
    """All tables of one session, as the oracle uses them."""

    def __init__(self, d=128, bits=3, seed=0, mode=MSE):
        if d <= 0:
            raise ValueError("d must be positive")
        self.d = d
        self.bits = bits
        self.seed = seed
        self.mode = mode
        self.dense = bool(mode & DENSE)
        self.qjl = bool(mode & QJL)
        self.b_m = mse_bits(bits, mode)
        if self.b_m == 0 and self.qjl:
            # QJL only (one bit in total): no MSE stage, the residual is the
            # whole unit vector (blog's QJL demo with zero MSE bits: r = x,
            # gamma = 1).  One level of value 0 and no boundaries say that.
            self.centroids, self.boundaries = np.zeros(1), np.zeros(0)
        elif not 1 <= self.b_m <= 4:
            raise ValueError("MSE bits must be 1..4 (0 only with QJL)")
        else:
            self.centroids, self.boundaries = codebook(self.b_m, d)
        if self.dense:
            self.pi = pi_matrix(d, seed)
            self.rotors = None
            self.n_coords = d
        else:
            self.rotors = rotor_table(d, seed)
            self.pi = None
            self.n_coords = 3 * n_groups(d)
        self.s = s_matrix(d, seed) if self.qjl else None
        self.m = d

    @property
    def qjl_scale(self):
        """sqrt(pi/2) / m, the estimator's constant (README formula)."""
        return math.sqrt(math.pi / 2.0) / self.m
