"""Pins for the oracle's outlier-channel separation of QJL-only keys (CPU
only): the reduction to the plain QJL-only codec at k = 0, exact outlier
channels, unbiasedness over S draws, the variance the separation removes,
and the channel choice on hand-made and generated keys."""
import math

import numpy as np
import pytest

from oracle import codec as K
from oracle import outlier as O
from oracle import params as P
from oracle import theory as T
from kv_cache_vector_norm_amd import workloads as W

D = 128


def _keys(n, seed, chans=(3, 40, 77, 120), scale=10.0):
    x = W.gaussian(n, seed=seed).astype(np.float64)
    x[:, list(chans)] *= scale
    return x.astype(np.float16).astype(np.float64)


def test_zero_channels_is_the_plain_qjl_only_codec():
    p = P.Params(D, 1, 0, P.QJL)
    x = _keys(200, 1)
    rec, out, _ = O.quantize(p, x, np.zeros(0, np.int64))
    ref, _ = K.quantize(p, x)
    assert out.shape == (200, 0)
    for a, b in ((rec.norms, ref.norms), (rec.signs, ref.signs), (rec.rnorms, ref.rnorms)):
        assert np.array_equal(a, b)
    assert np.array_equal(O.dequantize(p, rec, out, []), K.dequantize(p, ref))
    q = W.queries(3, seed=2).astype(np.float64)
    assert np.array_equal(O.score(p, q, rec, out, []), q @ K.dequantize(p, ref).T)


def test_outlier_channels_come_back_exactly_and_the_rest_is_the_inlier_sketch():
    p = P.Params(D, 1, 0, P.QJL)
    chans = np.array([3, 40, 77, 120])
    x = _keys(300, 3)
    rec, out, _ = O.quantize(p, x, chans)
    xt = O.dequantize(p, rec, out, chans)
    assert np.array_equal(xt[:, chans], x[:, chans])          # fp16 inputs: exact
    # the record is the QJL-only record of x with the outlier channels zeroed
    xin = x.copy()
    xin[:, chans] = 0.0
    ref, _ = K.quantize(p, xin)
    assert np.array_equal(rec.norms, ref.norms) and np.array_equal(rec.signs, ref.signs)
    assert np.array_equal(K.half_value(rec.norms), np.linalg.norm(xin, axis=1).astype(np.float16).astype(np.float64))
    rest = np.setdiff1d(np.arange(D), chans)
    assert np.array_equal(xt[:, rest], K.dequantize(p, ref)[:, rest])


def test_score_is_the_split_estimator():
    """<q, x~> equals n^ sqrt(pi/2)/m gamma^ <S q_in, sigma> + sum_O q_j o^_j,
    q_in = q with the outlier channels set to 0: the dequantised key's zero
    inlier part on the outlier channels is what lets a scorer use S q_in."""
    p = P.Params(D, 1, 0, P.QJL)
    chans = np.array([0, 5, 64, 127])
    x = _keys(120, 4, chans=chans)
    q = W.queries(6, seed=5).astype(np.float64)
    rec, out, _ = O.quantize(p, x, chans)
    s = O.score(p, q, rec, out, chans)
    nhat, _, ghat, sigma = K.decode(p, rec)
    qin = q.copy()
    qin[:, chans] = 0.0
    est = p.qjl_scale * (qin @ p.s.T) @ sigma.T * (nhat * ghat)[None, :] + q[:, chans] @ K.half_value(out).T
    assert np.allclose(s, est, rtol=1e-12, atol=1e-9)


def _with_s(p, s):
    p.s = s
    return p


def test_unbiased_over_s_and_the_variance_it_removes():
    """Over Gaussian S draws the estimate is unbiased for <q, x> (the outlier
    values are fp16 inputs, so exact), with the QJL-only variance of the
    inlier part alone (Lemma 4 with r = x_in / |x_in|, y = q_in, times
    |x_in|^2); without separation it is the closed form for the whole
    vector, several times larger with four x10 channels in q and x."""
    p = P.Params(D, 1, 0, P.QJL)
    rng = np.random.default_rng(41)
    chans = np.array([3, 40, 77, 120])
    x = _keys(1, 6)
    q = rng.normal(size=D)
    q[chans] *= 10.0
    xin = x[0].copy()
    xin[chans] = 0.0
    qin = q.copy()
    qin[chans] = 0.0
    sep, plain = [], []
    for _ in range(2500):
        _with_s(p, rng.normal(size=(D, D)))
        rec, out, _ = O.quantize(p, x, chans)
        nh = K.half_value(rec.norms)[0]
        # undo the fp16 rounding of the stored inlier norm (not a property of S)
        sep.append((O.score(p, q[None], rec, out, chans)[0, 0] - q[chans] @ x[0, chans]) * np.linalg.norm(xin) / nh
                   + q[chans] @ x[0, chans])
        rec0, _ = K.quantize(p, x)
        plain.append(K.score(p, q[None], rec0)[0, 0] * np.linalg.norm(x[0]) / K.half_value(rec0.norms)[0])
    sep, plain = np.array(sep), np.array(plain)
    exact = q @ x[0]
    assert abs(sep.mean() - exact) < 4 * sep.std() / math.sqrt(len(sep))
    var_sep = T.qjl_variance_exact(D, xin / np.linalg.norm(xin), qin) * (xin @ xin)
    assert abs(sep.var() / var_sep - 1) < 0.1
    var_plain = T.qjl_variance_exact(D, x[0] / np.linalg.norm(x[0]), q) * (x[0] @ x[0])
    assert abs(plain.var() / var_plain - 1) < 0.1
    assert var_plain > 3 * var_sep


def test_channel_choice_hand_example_and_ties():
    x = np.zeros((3, D))
    x[:, 10] = [1.0, -1.0, 1.0]        # mean |x| 1
    x[:, 2] = [0.0, 3.0, 0.0]          # 1
    x[:, 99] = [-2.0, -2.0, -2.0]      # 2
    x[:, 50] = [0.5, 0.5, 0.5]         # 0.5
    assert list(O.select_channels(x, 1)) == [99]
    assert list(O.select_channels(x, 2)) == [2, 99]           # 2 and 10 tie: the lower index
    assert list(O.select_channels(x, 3)) == [2, 10, 99]
    assert list(O.select_channels(x, 4)) == [2, 10, 50, 99]
    assert list(O.select_channels(x, 5)) == [0, 2, 10, 50, 99]   # zero channels tie: lowest first
    assert len(O.select_channels(x, 0)) == 0


def test_channel_choice_finds_the_planted_channels_of_the_cache_generator():
    torch = pytest.importorskip("torch")
    for seed in (1, 2, 3):
        g = torch.Generator()
        g.manual_seed(W.cache_seed(seed, 0, 0))
        planted = sorted(torch.randperm(D, generator=g)[:W.N_OUTLIERS].tolist())
        k, _, _ = W.lowrank_head(4096, W.cache_seed(seed, 0, 0), torch=torch)
        got = O.select_channels(k.numpy().astype(np.float64), W.N_OUTLIERS)
        assert list(got) == planted


def test_heads_use_their_own_channels():
    p = P.Params(D, 1, 0, P.QJL)
    a, b = _keys(64, 7, chans=(1, 2, 3, 4)), _keys(64, 8, chans=(100, 101, 102, 103))
    x = np.concatenate([a, b])
    chans = O.select_channels_heads(x, 64, 4)
    assert chans.tolist() == [[1, 2, 3, 4], [100, 101, 102, 103]]
    rec, out, _ = O.quantize_heads(p, x, 64, chans)
    xt = O.dequantize_heads(p, rec, out, 64, chans)
    assert np.array_equal(xt[:64, 1:5], a[:, 1:5]) and np.array_equal(xt[64:, 100:104], b[:, 100:104])
    q = W.queries(4, seed=9).astype(np.float64)
    s = O.score_gqa(p, q, rec, out, chans, group=2, t=64)
    assert np.allclose(s[2:], q[2:] @ xt[64:].T, rtol=0, atol=1e-9)
