"""The codec, stated plainly in float64 (test infrastructure only).

Quantize (RotorQuant, README "The Fused CUDA Kernel" and "RotorQuant Fused
Kernels": normalize -> embed -> rotor sandwich -> quantize; dequantize runs
inverse sandwich -> extract -> rescale):
  1. n = ||x||_2, x_u = x / n (x_u = 0 when n = 0); the norm is stored
     separately as an IEEE half (README "Codebook Calibration Fix", item 2).
  2. v = (x_u, 0): groups of three coordinates, zero padded to 3*ceil(d/3).
  3. y_g = grade-1 part of (R_g V_g) R_g~ (two explicit geometric products,
     README "Non-Commutative Algebra Bug Fix").
  4. code_i = #{k : y_i > t_k}: nearest centroid with midpoint boundaries;
     an exact tie goes to the lower index, as an argmin over distances
     returns the first minimiser (blog demo's argmin).
  5. Codes are packed as one little-endian bit stream: code i occupies bits
     [b*i, b*i + b) of the 32-bit word array (layout is this codec's own; the
     pages do not give one).
  With QJL (README Stage 2 and estimator; blog QJL section; hyper.ai
  Algorithm 2), using b - 1 MSE bits:
  6. x~_u = dequantised MSE part (steps 1-3 of dequantize below, unit scale);
     r = x_u - x~_u; gamma = ||r|| (stored as half); z = S r;
     sign bit j = [z_j >= 0] (a stored bit cannot hold sign 0), packed
     LSB-first into 4 words.

Dequantize:
  1. y^_i = c[code_i]; 2. x~_g = grade-1 part of (R_g~ Y^_g) R_g, pad dropped;
  3. with QJL: x~ += sqrt(pi/2)/m * gamma^ * S^T (2 bit - 1);
  4. out = n^ x~, with n^ and gamma^ the stored halves.

Score (README estimator formula): for a query q and a stored key,
  s = n^ * ( <q, x~_mse,u> + gamma^ * sqrt(pi/2)/m * <S q, 2 bit - 1> ),
computed here from the plain definition (dequantise, then dot products);
no 1/sqrt(d) and no softmax.

TurboQuant (hyper.ai Algorithms 1 and 2; README Stage 1): the same with
y = Pi x_u on d coordinates and x~_u = Pi^T y^.
"""
import math

import numpy as np

from . import clifford
from .params import Params


def code_words(n_coords, b):
    return -(-(n_coords * b) // 32)


def sign_words(m):
    return -(-m // 32)


# ----------------------------------------------------------------- packing --
def pack_codes(codes, b):
    """[N, n] integer codes -> [N, W] uint32, dense LSB-first bit stream."""
    codes = np.asarray(codes, dtype=np.uint64)
    nvec, n = codes.shape
    w = code_words(n, b)
    bits = np.zeros((nvec, 32 * w), dtype=np.uint64)
    for i in range(n):
        for k in range(b):
            bits[:, b * i + k] = (codes[:, i] >> np.uint64(k)) & np.uint64(1)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    words = (bits.reshape(nvec, w, 32) * weights).sum(axis=2)
    return words.astype(np.uint32)


def unpack_codes(words, b, n):
    words = np.asarray(words, dtype=np.uint64)
    nvec, w = words.shape
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    bits = bits.reshape(nvec, 32 * w)
    codes = np.zeros((nvec, n), dtype=np.int64)
    for k in range(b):
        codes += (bits[:, b * np.arange(n) + k] << np.uint64(k)).astype(np.int64)
    return codes


def pack_signs(bits):
    return pack_codes(bits, 1)


def unpack_signs(words, m):
    return unpack_codes(words, 1, m)


def half_bits(x):
    """IEEE half, round to nearest even, of float64 values -> uint16 bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def half_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------- rotations --
def _group_view(v, g):
    return v.reshape(v.shape[0], g, 3)


def rotor_forward(p, xu):
    """y = grade-1 parts of (R_g V_g) R_g~ over the zero-padded groups."""
    nvec = xu.shape[0]
    g = p.rotors.shape[0]
    v = np.zeros((nvec, 3 * g))
    v[:, : p.d] = xu
    mv = clifford.embed_vector(_group_view(v, g))            # [N, G, 8]
    r = np.zeros((g, 8))
    r[:, 0], r[:, 4], r[:, 5], r[:, 6] = p.rotors.T
    rr = clifford.reverse(r)
    left = np.einsum("gi,ngj,ijk->ngk", r, mv, clifford.CAYLEY, optimize=True)
    out = np.einsum("ngi,gj,ijk->ngk", left, rr, clifford.CAYLEY, optimize=True)
    return out[:, :, 1:4].reshape(nvec, 3 * g), out


def rotor_inverse(p, yhat):
    """x~ = grade-1 parts of (R_g~ Y_g) R_g; returns all 3G coordinates."""
    nvec = yhat.shape[0]
    g = p.rotors.shape[0]
    mv = clifford.embed_vector(_group_view(yhat, g))
    r = np.zeros((g, 8))
    r[:, 0], r[:, 4], r[:, 5], r[:, 6] = p.rotors.T
    rr = clifford.reverse(r)
    left = np.einsum("gi,ngj,ijk->ngk", rr, mv, clifford.CAYLEY, optimize=True)
    out = np.einsum("ngi,gj,ijk->ngk", left, r, clifford.CAYLEY, optimize=True)
    return out[:, :, 1:4].reshape(nvec, 3 * g)


def forward(p, xu):
    if p.dense:
        return xu @ p.pi.T
    return rotor_forward(p, xu)[0]


def inverse(p, yhat):
    if p.dense:
        return yhat @ p.pi
    return rotor_inverse(p, yhat)[:, : p.d]


# ------------------------------------------------------------------- codec --
def scalar_quantize(p, y):
    """code = #{k : y > t_k} per coordinate."""
    return (y[..., None] > p.boundaries).sum(axis=-1)


class Record:
    """A batch of compressed vectors (structure of arrays)."""

    def __init__(self, codes, norms, signs=None, rnorms=None):
        self.codes = codes      # [N, W] uint32
        self.norms = norms      # [N] uint16 (half bits)
        self.signs = signs      # [N, 4] uint32 or None
        self.rnorms = rnorms    # [N] uint16 or None


class Diagnostics:
    """Float64 intermediates the parity protocol needs (decision margins)."""

    def __init__(self, n, y, z=None, gamma=None):
        self.n = n
        self.y = y
        self.z = z
        self.gamma = gamma


def _mse_unit_recon(p, codes):
    yhat = p.centroids[codes]
    return inverse(p, yhat)


def quantize(p: Params, x):
    """Quantize rows of x (exact input values, any float dtype)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(n > 0.0, n, 1.0)
    xu = np.where(n[:, None] > 0.0, x / safe[:, None], 0.0)
    y = forward(p, xu)
    codes = scalar_quantize(p, y)
    rec = Record(pack_codes(codes, p.b_m), half_bits(n))
    diag = Diagnostics(n, y)
    if p.qjl:
        r = xu - _mse_unit_recon(p, codes)
        gamma = np.sqrt(np.sum(r * r, axis=1))
        z = r @ p.s.T
        rec.signs = pack_signs((z >= 0.0).astype(np.int64))
        rec.rnorms = half_bits(gamma)
        diag.z = z
        diag.gamma = gamma
    return rec, diag


def decode(p: Params, rec: Record):
    """(n^, x~_mse_u, gamma^, sigma) read back from a record."""
    codes = unpack_codes(rec.codes, p.b_m, p.n_coords)
    xmse = _mse_unit_recon(p, codes)
    nhat = half_value(rec.norms)
    if not p.qjl:
        return nhat, xmse, None, None
    ghat = half_value(rec.rnorms)
    sigma = 2.0 * unpack_signs(rec.signs, p.m).astype(np.float64) - 1.0
    return nhat, xmse, ghat, sigma


def dequantize(p: Params, rec: Record):
    nhat, xt, ghat, sigma = decode(p, rec)
    if p.qjl:
        xt = xt + p.qjl_scale * ghat[:, None] * (sigma @ p.s)
    return nhat[:, None] * xt


def score(p: Params, q, rec: Record):
    """[H, T] estimates of <q_h, k_t> for every query row and stored key."""
    q = np.asarray(q, dtype=np.float64)
    nhat, xt, ghat, sigma = decode(p, rec)
    s = q @ xt.T
    if p.qjl:
        sq = q @ p.s.T                                   # rows: S q_h
        s = s + p.qjl_scale * ghat[None, :] * (sq @ sigma.T)
    return s * nhat[None, :]


def score_gqa(p: Params, q, rec: Record, group, t, kv_stride=None):
    """Grouped-query scoring: query head h reads KV head h // group.

    `rec` holds the keys of all KV heads, head j's t keys starting at
    vector j * kv_stride.  Returns [H, t].
    """
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], t))
    for h in range(q.shape[0]):
        j = h // group
        sl = slice(j * kv_stride, j * kv_stride + t)
        out[h] = score(p, q[h : h + 1], _rows(rec, sl))[0]
    return out


def _rows(rec: Record, sl):
    return Record(rec.codes[sl], rec.norms[sl],
                  None if rec.signs is None else rec.signs[sl],
                  None if rec.rnorms is None else rec.rnorms[sl])


def attend(pk: Params, pv: Params, q, krec: Record, vrec: Record, group, t, scale, kv_stride=None):
    """Decode attention read straight from a compressed cache.

    Attention is softmax(q K^T / sqrt(d)) V, a softmax-weighted sum of the
    values (PolarQuant article, "Проблема KV-кэша в трансформерах"); the
    README's note under "Triton Kernels" asks for the q.k scores to be taken
    from the compressed keys.  For query head h, reading KV head j = h // group
    (keys and values of head j start at vector j * kv_stride):
      s_t = scale * score(q_h, k_t)        the estimator above, over t keys
      p   = softmax(s)                     (max subtracted first; same value)
      out_h = sum_t p_t * dequantize(v_t)  values decoded with their own session
    Returns [H, d].
    """
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    s = scale * score_gqa(pk, q, krec, group, t, kv_stride)
    out = np.zeros((q.shape[0], pv.d))
    for h in range(q.shape[0]):
        j = h // group
        e = np.exp(s[h] - s[h].max())
        pr = e / e.sum()
        xv = dequantize(pv, _rows(vrec, slice(j * kv_stride, j * kv_stride + t)))
        out[h] = pr @ xv
    return out


def attend_with_current(pk: Params, pv: Params, q, krec: Record, vrec: Record, group, t, scale, k_cur, v_cur,
                        kv_stride=None):
    """Decode attention of one step where the current token's own key and
    value enter at full precision and the t earlier tokens come from the
    compressed cache (README "Post-Prefill Quantization": each decode step
    stores the new key compressed but the current token's attention uses
    the full-precision key).  For query head h of KV head j = h // group,
    one softmax over [scale * score(q_h, k_t) for cached t] + [scale <q_h, k_cur_j>]
    weighs [dequantize(v_t)] + [v_cur_j].  Returns [H, d]."""
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    k_cur = np.asarray(k_cur, dtype=np.float64)
    v_cur = np.asarray(v_cur, dtype=np.float64)
    s = scale * score_gqa(pk, q, krec, group, t, kv_stride) if t > 0 else np.zeros((q.shape[0], 0))
    out = np.zeros((q.shape[0], pv.d))
    for h in range(q.shape[0]):
        j = h // group
        z = np.concatenate([s[h], [scale * (q[h] @ k_cur[j])]])
        e = np.exp(z - z.max())
        pr = e / e.sum()
        vals = v_cur[j][None, :]
        if t > 0:
            vals = np.concatenate([dequantize(pv, _rows(vrec, slice(j * kv_stride, j * kv_stride + t))), vals])
        out[h] = pr @ vals
    return out


def roundtrip(p: Params, x):
    rec, diag = quantize(p, x)
    return rec, dequantize(p, rec), diag


# ----------------------------------------------------------- diagnostics --
def boundary_distance(p: Params, y):
    """Distance of each y_i to its nearest decision boundary."""
    return np.min(np.abs(y[..., None] - p.boundaries), axis=-1)


def qjl_scale(m):
    return math.sqrt(math.pi / 2.0) / m
