"""Outlier-channel separation for QJL-only (one-bit) keys, stated plainly in
float64.  Test infrastructure only: imported by tests/, the smoke check and
the bench's CPU baseline, never by the library.

What the pages say: the README's list of QJL kernels (section "CUDA
Kernels", "QJL Kernels") describes the one-bit quantiser as random
projection + sign quantisation + outlier separation, with score kernels for
plain and grouped-query attention; the blog's random-rotation section
(Lemma 1) and the podcast page say LLM feature vectors carry very large
outliers that make direct quantisation inaccurate, and the blog's demo
plants one such channel.  The pages give no rule for choosing, storing or
scoring the separated channels, so this module takes the plainest reading
(each point is also listed among the readings of the design notes):

* Channels.  The outlier channels of a head are the k channels with the
  largest mean |x_j| over that head's keys at bulk quantisation (a tie goes
  to the lower channel index), kept in increasing order and then fixed for
  the head; k = 0 is the plain QJL-only codec.
* Storage.  A key's values on those channels are stored as IEEE halves
  (round to nearest even; an fp16 input keeps its exact value).
* QJL stage.  It sees only the inlier part x_in (outlier channels set to
  0): n = ||x_in||, x_u = x_in / n, sign bits of S x_u, gamma = ||x_u||,
  as in the QJL-only codec (r = x_u, no MSE stage).
* Dequantisation.  x~ = the inlier channels of n^ sqrt(pi/2)/m gamma^
  S^T sigma, plus the stored values on the outlier channels, so the outlier
  channels come back exactly.
* Score.  <q, x~>, the plain definition (no 1/sqrt(d), no softmax); with
  q_in = q with the outlier channels set to 0 this is
  n^ sqrt(pi/2)/m gamma^ <S q_in, sigma> + sum_{j in O} q_j o^_j.
"""
import numpy as np

from . import codec as OC
from .params import Params


def select_channels(x, k):
    """The k channels of largest mean |x_j| over the rows of x (one head's
    keys), ties to the lower index, returned in increasing order."""
    x = np.asarray(x, dtype=np.float64)
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    mean_abs = np.mean(np.abs(x), axis=0)
    order = sorted(range(x.shape[1]), key=lambda j: (-mean_abs[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def select_channels_heads(x, head_rows, k):
    """select_channels for each block of head_rows consecutive rows."""
    x = np.asarray(x, dtype=np.float64)
    heads = x.shape[0] // head_rows
    return np.stack([select_channels(x[h * head_rows:(h + 1) * head_rows], k) for h in range(heads)]) \
        if k else np.zeros((heads, 0), dtype=np.int64)


def _inlier(x, chans):
    xin = np.array(x, dtype=np.float64, copy=True)
    if len(chans):
        xin[:, chans] = 0.0
    return xin


def quantize(p: Params, x, chans):
    """QJL-only record of the inlier part of each row of x, and the rows'
    values on `chans` as half bits [n, k].  Returns (record, outliers, diag)."""
    if not (p.qjl and p.b_m == 0):
        raise ValueError("outlier separation is defined for QJL-only sessions (1 bit with QJL)")
    x = np.asarray(x, dtype=np.float64)
    chans = np.asarray(chans, dtype=np.int64)
    outliers = OC.half_bits(x[:, chans]) if len(chans) else np.zeros((x.shape[0], 0), np.uint16)
    rec, diag = OC.quantize(p, _inlier(x, chans))
    return rec, outliers, diag


def quantize_heads(p: Params, x, head_rows, chans):
    """quantize() over blocks of head_rows rows, block h with chans[h]."""
    x = np.asarray(x, dtype=np.float64)
    recs, outs, zs = [], [], []
    for h in range(chans.shape[0]):
        rec, o, d = quantize(p, x[h * head_rows:(h + 1) * head_rows], chans[h])
        recs.append(rec)
        outs.append(o)
        zs.append(d.z)
    rec = OC.Record(np.concatenate([r.codes for r in recs]), np.concatenate([r.norms for r in recs]),
                    np.concatenate([r.signs for r in recs]), np.concatenate([r.rnorms for r in recs]))
    return rec, np.concatenate(outs), np.concatenate(zs)


def dequantize(p: Params, rec, outliers, chans):
    """x~: the QJL-only reconstruction with its outlier channels replaced by
    the stored values."""
    chans = np.asarray(chans, dtype=np.int64)
    xt = OC.dequantize(p, rec)
    if len(chans):
        xt[:, chans] = OC.half_value(outliers)
    return xt


def dequantize_heads(p: Params, rec, outliers, head_rows, chans):
    out = []
    for h in range(chans.shape[0]):
        sl = slice(h * head_rows, (h + 1) * head_rows)
        out.append(dequantize(p, OC._rows(rec, sl), outliers[sl], chans[h]))
    return np.concatenate(out)


def score(p: Params, q, rec, outliers, chans):
    """[H, T]: <q_h, x~_t> for every query row and stored key."""
    q = np.asarray(q, dtype=np.float64)
    return q @ dequantize(p, rec, outliers, chans).T


def score_gqa(p: Params, q, rec, outliers, chans, group, t, kv_stride=None):
    """Query row h reads KV head j = h // group: its t keys start at record
    row j * kv_stride and its channel set is chans[j].  Returns [H, t]."""
    kv_stride = t if kv_stride is None else kv_stride
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], t))
    for h in range(q.shape[0]):
        j = h // group
        sl = slice(j * kv_stride, j * kv_stride + t)
        out[h] = score(p, q[h:h + 1], OC._rows(rec, sl), outliers[sl], chans[j])[0]
    return out
