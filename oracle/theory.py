"""Closed forms and counts the pages state (test infrastructure only).

Sources and readings:
* Theorem 1 (blog, "MSE 标量量化 (Theorem 1)" and "与理论上界的比较"):
  D_mse <= C * 4^-b for a unit vector.  The printed constant sqrt(3 pi)/2
  (~1.53) contradicts the same page's own derivation, which multiplies
  pi * sqrt(3) pi * 4 (so the Theorem-1 constant is sqrt(3) pi / 2), its
  remark that the constant is about 2.7 for large b, and the README's
  measured MSEs (0.116 at b = 2 is above 1.53/16).  The reading taken here
  is C = sqrt(3) * pi / 2 ~= 2.721; both candidates are exposed.
* Theorem 3 (blog, lower bound): D_mse >= 4^-b.
* Lemma 4 / Theorem 2 (blog, QJL section): E_S <y, x~_qjl> = <y, r>;
  Var <= pi / (2d) * |r|^2 |y|^2; D_prod <= sqrt(3) pi^2 |y|^2 / d * 4^-b.
* 1-bit shrinkage (blog, Theorem 2 preamble): about 2/pi.
* Parameter counts (README "Parameter Efficiency", "Why Rotors?"; podcast
  page): TurboQuant d^2 + codebook = 16,399 at d = 128, b = 3; RotorQuant
  "43 rotors x 8 + 4 grade codebooks", printed as ~380 (README) and 372
  (podcast).
* FMA counts (README "FMA Count"): 20 + 28 = 48 per group, 2,064 per vector;
  TurboQuant 16,384 per rotation.
* Compression (README table "Stored indices" / "3-bit compression").
"""
import math

from scipy import special

THM1_CONSTANT_DERIVED = math.sqrt(3.0) * math.pi / 2.0
THM1_CONSTANT_PRINTED = math.sqrt(3.0 * math.pi) / 2.0


def thm1_upper(b, constant=THM1_CONSTANT_DERIVED):
    return constant * 4.0 ** (-b)


def thm3_lower(b):
    return 4.0 ** (-b)


def thm2_upper(b, d, ynorm2=1.0):
    return math.sqrt(3.0) * math.pi ** 2 * ynorm2 / d * 4.0 ** (-b)


def lemma4_var_bound(d, rnorm2, ynorm2):
    return math.pi / (2.0 * d) * rnorm2 * ynorm2


def qjl_variance_exact(m, r, y):
    """Var_S <y, sqrt(pi/2)/m |r| S^T sign(S r)> for i.i.d. N(0,1) S.

    Each of the m rows s contributes sqrt(pi/2) |r| <s, y> sign(<s, r>)/m;
    with u = r/|r|, E[<s,y> sign(<s,u>)] = sqrt(2/pi) <y,u> and
    E[<s,y>^2] = |y|^2, so the per-row variance is
    (pi/2)|r|^2|y|^2 - <y,r>^2 and the mean of m rows divides it by m.
    """
    import numpy as np
    r = np.asarray(r, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    rn2 = float(r @ r)
    yn2 = float(y @ y)
    return ((math.pi / 2.0) * rn2 * yn2 - float(y @ r) ** 2) / m


def mean_abs_coord(d):
    """E|X| for one coordinate of a uniform unit vector in R^d."""
    return math.exp(special.gammaln(d / 2.0) - special.gammaln((d + 1) / 2.0)) / math.sqrt(math.pi)


def one_bit_distortion(d):
    """Unit-vector MSE of the 1-bit Lloyd-Max code: 1 - d (E|X|)^2."""
    return 1.0 - d * mean_abs_coord(d) ** 2


def one_bit_shrinkage(d):
    """kappa with E_Pi <q, x~> = kappa <q, x> for the 1-bit code over Haar
    Pi: kappa = d (E|X|)^2, which tends to 2/pi as d grows."""
    return d * mean_abs_coord(d) ** 2


def tq_param_count(d, bits):
    """d x d rotation + 2^b centroids + (2^b - 1) boundaries."""
    return d * d + (1 << bits) + (1 << bits) - 1


def rq_param_count(d, bits):
    """8 multivector slots per rotor + four grade codebooks of 2^b."""
    return 8 * (-(-d // 3)) + 4 * (1 << bits)


def rq_param_count_compact(d):
    """4 non-zero rotor components per group (README "Why Rotors?")."""
    return 4 * (-(-d // 3))


def sandwich_fma_per_group():
    """Rotor-left product: 4 non-zero outputs x 5 FMAs; right product:
    4 outputs x 7 FMAs (README "FMA Count")."""
    return 4 * 5 + 4 * 7


def sandwich_fma_per_vector(d):
    return sandwich_fma_per_group() * (-(-d // 3))


def dense_rotation_fma(d):
    return d * d


def compression_ratio(d, index_count, bits, side_bits=32):
    """fp16 bits over stored index bits plus side information."""
    return (16 * d) / (index_count * bits + side_bits)
