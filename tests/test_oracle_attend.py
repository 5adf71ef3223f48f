"""Pins for the oracle's decode attention over a compressed cache (CPU only).

The oracle states softmax(scale * q.k) . V with the keys read through the
estimator and the values through dequantisation.  These checks tie it to
what the definition forces, each chosen so a plausible slip fails one:
a single key returns its value exactly (nothing else can come out of a
one-element softmax); scale 0 gives the plain mean of the values (a missing
normalisation or a transposed weight matrix fails it); a dominant key at a
large scale returns that key's value (keys and values misaligned, or the
scale ignored, fails it); per-head constant values come back per head (a
wrong GQA head mapping fails it); permuting keys and values together
changes nothing; every output coordinate lies inside its head's values'
range; and the weights equal scipy's softmax of the scaled estimates.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import codec as OC
from oracle import params as OP
from kv_cache_vector_norm_amd import workloads as W

D = 128
PK = OP.Params(D, 3, 0, OP.QJL)
PV = OP.Params(D, 2, 0, OP.MSE)


def _cache(t, kv_heads, seed, pk=PK, pv=PV):
    k = W.gaussian(t * kv_heads, seed=seed).astype(np.float64)
    v = W.gaussian(t * kv_heads, seed=seed + 1).astype(np.float64)
    krec, _ = OC.quantize(pk, k)
    vrec, _ = OC.quantize(pv, v)
    return krec, vrec


def _head_values(pv, vrec, j, t, stride):
    return OC.dequantize(pv, OC._rows(vrec, slice(j * stride, j * stride + t)))


def test_single_key_returns_its_value():
    krec, vrec = _cache(1, 2, 10)
    q = W.queries(4, seed=11)
    out = OC.attend(PK, PV, q, krec, vrec, 2, 1, 1 / np.sqrt(D))
    for h in range(4):
        assert np.array_equal(out[h], _head_values(PV, vrec, h // 2, 1, 1)[0])


def test_zero_scale_is_the_mean_of_the_values():
    t = 37
    krec, vrec = _cache(t, 2, 12)
    q = W.queries(4, seed=13)
    out = OC.attend(PK, PV, q, krec, vrec, 2, t, 0.0)
    for h in range(4):
        assert np.abs(out[h] - _head_values(PV, vrec, h // 2, t, t).mean(0)).max() < 1e-14


def test_dominant_key_at_large_scale():
    t = 24
    k = W.gaussian(t, seed=14).astype(np.float64)
    q = W.queries(1, seed=15).astype(np.float64)
    k[17] = 3.0 * q[0]                          # by far the largest q.k
    krec, _ = OC.quantize(PK, k)
    v = W.gaussian(t, seed=16).astype(np.float64)
    vrec, _ = OC.quantize(PV, v)
    est = OC.score(PK, q, krec)[0]
    gap = est[17] - np.max(np.delete(est, 17))
    assert gap > 50.0
    out = OC.attend(PK, PV, q, krec, vrec, 1, t, 1.0)
    xv = OC.dequantize(PV, vrec)
    assert np.abs(out[0] - xv[17]).max() < 1e-12 * np.abs(xv).max() + t * np.exp(-gap) * np.abs(xv).max()
    # with a small scale the other keys weigh in again
    assert np.abs(OC.attend(PK, PV, q, krec, vrec, 1, t, 1e-3)[0] - xv[17]).max() > 1e-3


def test_gqa_head_mapping():
    t, kv_heads, group = 9, 3, 4
    krec, _ = _cache(t, kv_heads, 18)
    base = W.gaussian(kv_heads, seed=19).astype(np.float64)
    vrec, _ = OC.quantize(PV, np.repeat(base, t, axis=0))        # head j's values all equal
    q = W.queries(kv_heads * group, seed=20)
    out = OC.attend(PK, PV, q, krec, vrec, group, t, 0.3)
    const = OC.dequantize(PV, vrec)[::t]
    for h in range(kv_heads * group):
        assert np.abs(out[h] - const[h // group]).max() < 1e-14
    # the strided layout reads head j's block at j * kv_stride
    stride = 13
    kpad = np.zeros((stride * kv_heads, D))
    vpad = np.zeros((stride * kv_heads, D))
    k = W.gaussian(t * kv_heads, seed=18).astype(np.float64)
    for j in range(kv_heads):
        kpad[j * stride:j * stride + t] = k[j * t:(j + 1) * t]
        vpad[j * stride:j * stride + t] = base[j]
    kr2, _ = OC.quantize(PK, kpad)
    vr2, _ = OC.quantize(PV, vpad)
    out2 = OC.attend(PK, PV, q, kr2, vr2, group, t, 0.3, kv_stride=stride)
    assert np.abs(out2 - out).max() < 1e-14


def test_joint_permutation_and_convex_hull():
    t = 31
    krec, vrec = _cache(t, 1, 21)
    q = W.queries(3, seed=22)
    out = OC.attend(PK, PV, q, krec, vrec, 3, t, 1 / np.sqrt(D))
    perm = np.random.Generator(np.random.PCG64(23)).permutation(t)
    out_p = OC.attend(PK, PV, q, OC._rows(krec, perm), OC._rows(vrec, perm), 3, t, 1 / np.sqrt(D))
    assert np.abs(out - out_p).max() < 1e-13
    xv = OC.dequantize(PV, vrec)
    assert np.all(out >= xv.min(0) - 1e-13) and np.all(out <= xv.max(0) + 1e-13)


@pytest.mark.parametrize("pk,pv", [(PK, PV), (OP.Params(D, 4, 0, OP.DENSE | OP.QJL), OP.Params(D, 3, 0, OP.QJL))])
def test_weights_are_the_softmax_of_scaled_estimates(pk, pv):
    t, group = 40, 2
    krec, vrec = _cache(t, 2, 24, pk, pv)
    q = W.queries(4, seed=25)
    scale = 1 / np.sqrt(D)
    out = OC.attend(pk, pv, q, krec, vrec, group, t, scale)
    for h in range(4):
        j = h // group
        est = OC.score(pk, q[h:h + 1], OC._rows(krec, slice(j * t, (j + 1) * t)))[0]
        ref = softmax(scale * est) @ _head_values(pv, vrec, j, t, t)
        assert np.abs(out[h] - ref).max() < 1e-13


# ------------------------------------------- the current token, exact ---
def test_current_token_alone_and_uniform():
    q = W.queries(4, seed=30)
    kc = W.gaussian(2, seed=31).astype(np.float64)
    vc = W.gaussian(2, seed=32).astype(np.float64)
    krec, vrec = _cache(1, 2, 33)
    # nothing cached: the output is the current value
    out0 = OC.attend_with_current(PK, PV, q, krec, vrec, 2, 0, 0.1, kc, vc)
    for h in range(4):
        assert np.array_equal(out0[h], vc[h // 2])
    # scale 0: the plain mean over the cached values and the current one
    t = 20
    krec, vrec = _cache(t, 2, 34)
    out = OC.attend_with_current(PK, PV, q, krec, vrec, 2, t, 0.0, kc, vc)
    for h in range(4):
        j = h // 2
        vals = np.concatenate([_head_values(PV, vrec, j, t, t), vc[j][None]])
        assert np.abs(out[h] - vals.mean(0)).max() < 1e-14


def test_current_token_dominant_or_negligible():
    t = 16
    krec, vrec = _cache(t, 1, 35)
    q = W.queries(2, seed=36).astype(np.float64)
    vc = W.gaussian(1, seed=37).astype(np.float64)
    # the current key along q dominates: its value comes back
    kc = 50.0 * q[:1] / np.linalg.norm(q[0])
    out = OC.attend_with_current(PK, PV, q[:1], krec, vrec, 1, t, 1.0, kc, vc)
    assert np.abs(out[0] - vc[0]).max() < 1e-9
    # against q it is negligible: the cached attention comes back
    kn = -50.0 * q[:1] / np.linalg.norm(q[0])
    out = OC.attend_with_current(PK, PV, q[:1], krec, vrec, 1, t, 1.0, kn, vc)
    ref = OC.attend(PK, PV, q[:1], krec, vrec, 1, t, 1.0)
    assert np.abs(out - ref).max() < 1e-9 * np.abs(ref).max()
