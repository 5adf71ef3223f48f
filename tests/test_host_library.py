"""CPU checks of the C ABI library: it loads, exports every declared symbol,
reports layouts, builds the same parameter tables as the oracle, and rejects
bad arguments without touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import params as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    import kv_cache_vector_norm_amd as K
    return K


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:rq|tq|pq)_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(K):
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K.EXPORTS)


def test_layouts(K):
    widths = {(b, m): K.rq_layout(128, b, m) for b in (1, 2, 3, 4) for m in (K.RQ_MSE, K.RQ_DENSE)}
    assert [widths[(b, K.RQ_MSE)]["code_words"] for b in (1, 2, 3, 4)] == [5, 9, 13, 17]
    assert [widths[(b, K.RQ_DENSE)]["code_words"] for b in (1, 2, 3, 4)] == [4, 8, 12, 16]
    q = K.rq_layout(128, 3, K.RQ_QJL)
    assert q["mse_bits"] == 2 and q["sign_words"] == 4 and q["record_bytes"] == 9 * 4 + 2 + 16 + 2
    assert K.rq_layout(128, 3, K.RQ_MSE)["record_bytes"] == 54
    assert K.rq_layout(128, 3, K.RQ_MSE)["n_groups"] == 43
    # QJL only: no code words, norm + 4 sign words + gamma
    for m in (K.RQ_QJL, K.RQ_QJL | K.RQ_DENSE):
        q1 = K.rq_layout(128, 1, m)
        assert q1["mse_bits"] == 0 and q1["code_words"] == 0 and q1["record_bytes"] == 2 + 16 + 2


@pytest.mark.parametrize("bits,mode", [(b, OP.MSE) for b in (1, 2, 3, 4)] + [(b, OP.QJL) for b in (1, 2, 3, 4, 5)]
                         + [(b, OP.DENSE) for b in (2, 3, 4)] + [(3, OP.DENSE | OP.QJL), (1, OP.DENSE | OP.QJL)])
def test_host_params_match_oracle(K, bits, mode):
    p = K.rq_host_params(128, bits, 0, mode)
    o = OP.Params(128, bits, 0, mode)

    def ulps(a, b):
        a = np.asarray(a, np.float32)
        b = np.asarray(b, np.float32)
        assert a.shape == b.shape
        if a.size == 0:
            return 0
        return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64)).max()

    assert ulps(p["centroids"], o.centroids) <= 1
    assert ulps(p["boundaries"], o.boundaries) <= 1
    if mode & OP.DENSE:
        assert ulps(p["pi"], o.pi) <= 1
        pf = p["pi"].astype(np.float64)
        assert np.abs(pf @ pf.T - np.eye(128)).max() < 1e-6
    else:
        assert ulps(p["rotors"], o.rotors) <= 1
        assert np.abs(p["rotmats"].astype(np.float64) - OP.rotor_matrices(o.rotors)).max() < 2e-7
    if mode & OP.QJL:
        assert np.array_equal(p["s"], o.s.astype(np.float16).view(np.uint16))


def test_polar_layout_and_tables_match_oracle(K):
    """PolarQuant sessions: a 64-byte record of 16 words, the four Lloyd
    codebooks of the article's angle laws and the dense sessions' Pi, all
    equal to the oracle's fp32 values."""
    from oracle import polar as PQ
    lay = K.rq_layout(128, 4, K.RQ_POLAR)
    assert lay["code_words"] == 16 and lay["record_bytes"] == 64 and lay["sign_words"] == 0
    assert lay["n_coords"] == 128 and lay["n_groups"] == 0
    p = K.rq_host_params(128, 4, 0, K.RQ_POLAR)
    books = PQ.codebooks()
    assert np.array_equal(p["centroids"], np.concatenate([b[0] for b in books]).astype(np.float32))
    assert np.array_equal(p["boundaries"], np.concatenate([b[1] for b in books]).astype(np.float32))
    assert np.array_equal(p["pi"], PQ.PolarParams(128, 0).pi.astype(np.float32))
    assert np.array_equal(p["pi"], K.rq_host_params(128, 4, 0, K.RQ_DENSE)["pi"])
    # the kernels fold first-level points into the first octant (turns by pi
    # and pi/2, a reflection in the diagonal) and test only t_1: the
    # boundaries must repeat under those moves
    t = np.concatenate([[0.0], p["boundaries"][:15].astype(np.float64)])
    k = np.arange(16)
    assert np.abs(t[1:] - k[1:] * np.pi / 8).max() < 3e-7
    assert np.abs(t[5:] - t[1:12] - np.pi / 2).max() < 5e-7
    assert abs(t[3] - (np.pi / 2 - t[1])) < 2e-7 and abs(t[2] - np.pi / 4) < 1e-7
    with pytest.raises(K.RQError):
        K.rq_host_quantizer(128, 4, K.RQ_POLAR)


@pytest.mark.parametrize("d,bits,mode,status", [(128, 3, 4, 1), (128, 4, 5, 1), (128, 4, 6, 1), (64, 4, 4, 2)])
def test_polar_bad_settings(K, d, bits, mode, status):
    with pytest.raises(K.RQError) as e:
        K.rq_layout(d, bits, mode)
    assert e.value.status == status


def test_different_seeds_give_different_tables(K):
    a = K.rq_host_params(128, 3, 0, K.RQ_QJL)
    b = K.rq_host_params(128, 3, 1, K.RQ_QJL)
    assert not np.array_equal(a["rotors"], b["rotors"]) and not np.array_equal(a["s"], b["s"])
    assert np.array_equal(a["centroids"], b["centroids"])


@pytest.mark.parametrize("d,bits,mode,status", [
    (128, 0, 0, 1), (128, 5, 0, 1), (128, 0, 1, 1), (128, 6, 1, 1), (128, 3, 8, 1), (-1, 3, 0, 1),
    (64, 3, 0, 2), (256, 3, 1, 2)])
def test_bad_settings(K, d, bits, mode, status):
    with pytest.raises(K.RQError) as e:
        K.rq_layout(d, bits, mode)
    assert e.value.status == status
    with pytest.raises(K.RQError) as e:
        K.rq_host_params(d, bits, 0, mode)
    assert e.value.status == status
    assert K.rq_last_error() != ""


def test_null_arguments_rejected_before_any_device_work(K):
    lib = K.lib()
    assert lib.rq_quantize(None, None, 1, 10, 128, None, None, None, None, None) == K.RQ_EINVAL
    assert "ctx" in K.rq_last_error()
    assert lib.rq_dequantize(None, None, None, None, None, 10, None, 1, 128, None) == K.RQ_EINVAL
    assert lib.rq_roundtrip(None, None, 1, 10, 128, None, None, None, None, None, 1, 128, None) == K.RQ_EINVAL
    assert lib.rq_score(None, None, 1, 1, None, None, None, None, 10, 10, None, 10, None) == K.RQ_EINVAL
    assert lib.tq_quantize(None, None, 1, 10, 128, None, None, None, None, None) == K.RQ_EINVAL
    assert lib.pq_quantize(None, None, 1, 10, 128, None, None) == K.RQ_EINVAL
    assert lib.pq_dequantize(None, None, 10, None, 1, 128, None) == K.RQ_EINVAL
    assert lib.pq_roundtrip(None, None, 1, 10, 128, None, None, 1, 128, None) == K.RQ_EINVAL
    assert lib.pq_score(None, None, 1, 1, None, 10, 10, None, 10, None) == K.RQ_EINVAL
    assert lib.rq_get_layout(None, None) == K.RQ_EINVAL
    assert lib.rq_layout(128, 3, 0, None) == K.RQ_EINVAL
    lib.rq_free(None)


def test_init_without_device_fails_cleanly(K):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p(12345)
    rc = K.lib().rq_init(128, 3, 0, 0, ctypes.byref(h))
    assert rc in (K.RQ_EHIP, K.RQ_ENOMEM) and h.value is None
    rc = K.lib().rq_init(64, 3, 0, 0, ctypes.byref(h))
    assert rc == K.RQ_EUNSUPPORTED and h.value is None


def test_version(K):
    assert "gfx950" in K.rq_version()


def test_single_hip_runtime_in_process():
    """librq.so and torch must share one HIP runtime (torch owns the memory
    and streams the library is handed)."""
    import subprocess
    import sys
    code = ("import kv_cache_vector_norm_amd, torch, re; "
            "m = open('/proc/self/maps').read(); "
            "print(len(set(re.findall(r'/\\S*libamdhip64\\S*', m))))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def _slot(y, bias):
    """The kernels' slot of fp32 y: fp32 fma(y, 2032, bias), mantissa bits
    4..11.  y * 2032 is exact in float64 and so is the sum whenever a
    double rounding could matter, so float64 then float32 is the single
    fp32 rounding of the fma."""
    t = (y.astype(np.float64) * 2032.0 + np.float64(bias)).astype(np.float32)
    return (t.view(np.uint32) & 0xFF0) >> 4


def _edge_and_boundary_probes(boundaries, bias, ulps):
    """fp32 values within `ulps` ulps of every boundary and every slot edge."""
    pts = [boundaries.astype(np.float32)]
    for k in range(257):
        pts.append(np.float32(((16 * k - 0.5) - (bias - 12582912.0)) / 2032.0))
    pts = np.concatenate([np.atleast_1d(p) for p in pts]).astype(np.float32)
    out = [pts]
    up, dn = pts.copy(), pts.copy()
    for _ in range(ulps):
        up = np.nextafter(up, np.float32(2.0))
        dn = np.nextafter(dn, np.float32(-2.0))
        out += [up, dn]
    v = np.concatenate(out)
    return v[np.abs(v) <= np.float32(1.001)]


@pytest.mark.parametrize("bits,mode", [(b, OP.MSE) for b in (1, 2, 3, 4)] + [(b, OP.QJL) for b in (2, 3, 4, 5)]
                         + [(b, OP.DENSE) for b in (1, 2, 3, 4)] + [(b, OP.DENSE | OP.QJL) for b in (2, 3, 4, 5)])
def test_slot_table_is_exact_nearest_centroid(K, bits, mode):
    """The kernels' 256-slot lookup gives #{k : y > t_k} and c[code] for every
    fp32 y in [-1.001, 1.001]: random draws, both sides of every boundary and
    every slot edge within 60 ulps, and the end points."""
    p = K.rq_host_params(128, bits, 0, mode)
    c, t = p["centroids"], p["boundaries"]
    bias, table = K.rq_host_quantizer(128, bits, mode)
    rng = np.random.default_rng(bits * 10 + mode)
    y = np.concatenate([
        rng.normal(0.0, 0.09, 400_000).astype(np.float32),
        rng.uniform(-1.001, 1.001, 200_000).astype(np.float32),
        _edge_and_boundary_probes(t, bias, 60),
        np.array([-1.001, -1.0, -0.0, 0.0, 1.0, 1.001], np.float32),
    ])
    ref = (y[:, None] > t[None, :]).sum(axis=1)
    e = table[_slot(y, bias)]
    thr = e[:, 1].view(np.float32)
    gt = y > thr
    code = e[:, 0] + gt
    val = np.where(gt, e[:, 3], e[:, 2]).view(np.float32)
    assert np.array_equal(code, ref)
    assert np.array_equal(val, c[ref])
    # slots are monotone in y and no slot holds two boundaries
    s = _slot(np.sort(y), bias)
    assert np.all(np.diff(s.astype(np.int64)) >= 0)
    assert len(set(_slot(t, bias).tolist())) == len(t)


def test_workloads_and_package_import_touch_no_hip():
    """The input generators (shared by the oracle's tests) and the package
    itself import without loading librq.so or the HIP runtime; the library
    is loaded on the first call."""
    import subprocess
    import sys
    code = ("import kv_cache_vector_norm_amd as K, kv_cache_vector_norm_amd.workloads as W; "
            "W.gaussian(4, seed=0); "
            "m = open('/proc/self/maps').read(); "
            "print(int('librq' in m), int('libamdhip64' in m))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["0", "0"]


def test_library_stamp_matches_sources(K):
    """librq.so carries the digest of the sources it was built from, and the
    loader accepts it only when that equals the digest of csrc/ and include/."""
    from kv_cache_vector_norm_amd import build as B
    with open(B.stamp_path()) as f:
        assert f.read().strip() == B.source_digest()
    K.lib()
