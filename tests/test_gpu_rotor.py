"""GPU parity of the rotor codec (rq_quantize / rq_dequantize / rq_roundtrip)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import parity as PR
from oracle import codec as OC
from oracle import params as OP
from kv_cache_vector_norm_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _oracle_params(bits, mode, seed=0):
    return OP.Params(D, bits, seed, mode)


def _inputs(n, dtype, seed=3, unit=False):
    if unit:
        return W.unit_gaussian(n, seed=seed, dtype=dtype)
    return W.gaussian(n, seed=seed, dtype=dtype)


def _run_quant(K, codec, x_host, ld=None):
    n = x_host.shape[0]
    if ld is None:
        x = torch.from_numpy(x_host).cuda()
    else:
        buf = torch.zeros((n, ld), dtype=torch.from_numpy(x_host).dtype, device="cuda")
        buf[:, :D] = torch.from_numpy(x_host).cuda()
        x = buf
    rec = codec.quantize(x)
    torch.cuda.synchronize()
    return rec, x


MODES = [(b, OP.MSE) for b in (1, 2, 3, 4)] + [(b, OP.QJL) for b in (2, 3, 4, 5)]


@pytest.mark.parametrize("bits,mode", MODES)
def test_session_params_match_oracle(K, bits, mode):
    c = K.Codec(bits=bits, seed=0, mode=mode)
    p = c.params()
    o = _oracle_params(bits, mode)
    assert np.array_equal(p["rotors"].astype(np.float64), o.rotors)
    assert np.array_equal(p["centroids"].astype(np.float64), o.centroids)
    assert np.array_equal(p["boundaries"].astype(np.float64), o.boundaries)
    m = OP.rotor_matrices(o.rotors)
    assert np.abs(p["rotmats"] - m).max() < 2e-7
    if mode & OP.QJL:
        assert np.array_equal(p["s"], o.s.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("bits,mode", MODES)
@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000, 4097])
def test_quantize_parity(K, bits, mode, n):
    x = _inputs(n, np.float16, seed=n + bits)
    c = K.Codec(bits=bits, seed=0, mode=mode)
    rec, _ = _run_quant(K, c, x)
    codes, norms, signs, rnorms = rec.host()
    p = _oracle_params(bits, mode)
    orec, diag = OC.quantize(p, x.astype(np.float64))
    excl, rep = PR.compare_codes(p, codes, diag)
    PR.compare_halves(norms, diag.n, "norms")
    if mode & OP.QJL:
        PR.compare_signs(p, signs, diag, excl)
        keep = ~excl
        PR.compare_halves(rnorms[keep], diag.gamma[keep], "rnorms")


@pytest.mark.parametrize("bits,mode", [(3, OP.MSE), (1, OP.MSE), (4, OP.MSE), (3, OP.QJL), (2, OP.QJL), (5, OP.QJL)])
@pytest.mark.parametrize("in_dtype", [np.float16, np.float32])
def test_dequant_and_roundtrip(K, bits, mode, in_dtype):
    n = 777
    x = _inputs(n, in_dtype, seed=11)
    c = K.Codec(bits=bits, seed=0, mode=mode)
    xt = torch.from_numpy(x).cuda()
    rec, y32 = c.roundtrip(xt, dtype=torch.float32)
    y16 = c.roundtrip(xt, dtype=torch.float16)[1]
    d32 = c.dequantize(rec, dtype=torch.float32)
    d16 = c.dequantize(rec, dtype=torch.float16)
    torch.cuda.synchronize()
    # roundtrip output is exactly the dequantisation of the record it wrote
    assert torch.equal(y32, d32)
    assert torch.equal(y16, d16)
    assert torch.equal(y16, d32.to(torch.float16))
    p = _oracle_params(bits, mode)
    hrec = PR.record_from_host(*rec.host())
    ody = OC.dequantize(p, hrec)
    nhat = OC.half_value(hrec.norms)
    PR.compare_recon(d32.cpu().numpy(), ody, nhat, "dequantize fp32")
    # end to end from the raw input, on vectors with no band coordinate
    orec, diag = OC.quantize(p, x.astype(np.float64))
    excl, _ = PR.compare_codes(p, hrec.codes, diag)
    oy = OC.dequantize(p, orec)
    PR.compare_recon(y32.cpu().numpy(), oy, nhat, "roundtrip end to end", rows=~excl)


def test_strided_rows_and_fp32(K):
    n = 130
    c = K.Codec(bits=3, seed=5, mode=OP.QJL)
    x = _inputs(n, np.float16, seed=2)
    rec_a, _ = _run_quant(K, c, x)
    rec_b, _ = _run_quant(K, c, x, ld=136)
    for a, b in zip(rec_a.host(), rec_b.host()):
        assert np.array_equal(a, b)
    # fp32 input with a padded pitch
    x32 = x.astype(np.float32)
    rec_c, _ = _run_quant(K, c, x32, ld=132)
    p = _oracle_params(3, OP.QJL, seed=5)
    _, diag = OC.quantize(p, x32.astype(np.float64))
    codes, norms, signs, rnorms = rec_c.host()
    excl, _ = PR.compare_codes(p, codes, diag)
    PR.compare_signs(p, signs, diag, excl)


@pytest.mark.parametrize("mode", [OP.MSE, OP.QJL])
def test_zero_and_tiny_vectors(K, mode):
    x = np.zeros((70, D), np.float16)
    x[5, 3] = np.float16(1e-3)
    x[6, :] = np.float16(6e-5)
    c = K.Codec(bits=3, seed=0, mode=mode)
    xt = torch.from_numpy(x).cuda()
    rec, y = c.roundtrip(xt, dtype=torch.float32)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    zero = np.all(x == 0, axis=1)
    assert np.all(y[zero] == 0.0)
    assert np.all(np.isfinite(y))
    assert np.all(rec.host()[1][zero] == 0)


def test_deterministic(K):
    x = torch.from_numpy(_inputs(5000, np.float16, seed=9)).cuda()
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)
    a = [t.clone() for t in c.roundtrip(x, dtype=torch.float16)[0].__dict__.values()]
    b = [t.clone() for t in c.roundtrip(x, dtype=torch.float16)[0].__dict__.values()]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_1024_unit_vectors_mse_and_cosine(K):
    """1,024 fp32 unit vectors, 3-bit MSE-only roundtrip (README MSE table:
    MSE 0.034, cosine 0.983)."""
    x = W.unit_vectors_1024()
    c = K.Codec(bits=3, seed=0, mode=OP.MSE)
    rec, y = c.roundtrip(torch.from_numpy(x).cuda(), dtype=torch.float32)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    x64 = x.astype(np.float64)
    mse = ((x64 - y) ** 2).sum(1).mean()
    cos = ((x64 * y).sum(1) / np.linalg.norm(x64, axis=1) / np.linalg.norm(y, axis=1)).mean()
    assert abs(mse - 0.034) < 1.5e-3 and abs(cos - 0.983) < 2e-3
    p = _oracle_params(3, OP.MSE)
    orec, diag = OC.quantize(p, x64)
    excl, rep = PR.compare_codes(p, rec.host()[0], diag)
    PR.compare_recon(y, OC.dequantize(p, orec), OC.half_value(orec.norms), rows=~excl)


def test_65536_keys_full_parity(K):
    """65,536 fp16 N(0,1) keys, 2-bit MSE + 1-bit QJL (3 bits total)."""
    x = W.keys_65536()
    c = K.Codec(bits=3, seed=0, mode=OP.QJL)
    rec, y = c.roundtrip(torch.from_numpy(x).cuda(), dtype=torch.float32)
    torch.cuda.synchronize()
    codes, norms, signs, rnorms = rec.host()
    p = _oracle_params(3, OP.QJL)
    orec, diag = OC.quantize(p, x.astype(np.float64))
    excl, rep = PR.compare_codes(p, codes, diag)
    assert rep["band_fraction"] <= PR.BAND_FRACTION
    PR.compare_halves(norms, diag.n, "norms")
    PR.compare_signs(p, signs, diag, excl)
    PR.compare_recon(y.cpu().numpy(), OC.dequantize(p, PR.record_from_host(codes, norms, signs, rnorms)),
                     OC.half_value(norms), "dequantize")


@pytest.mark.parametrize("bits,mode,n", [(3, OP.MSE, 600_000), (3, OP.QJL, 300_000), (4, OP.DENSE, 300_000)])
def test_roundtrip_with_several_tiles_per_wave(K, bits, mode, n):
    """Batches large enough that each wave of the roundtrip handles more than
    one 64-vector tile (the whole-row output path): the record equals
    rq_quantize's and the output equals rq_dequantize of it, bit for bit."""
    c = K.Codec(bits=bits, seed=0, mode=mode)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((n, D), generator=g, device="cuda").to(torch.float16)
    rec, y = c.roundtrip(x, dtype=torch.float16)
    rec2 = c.quantize(x)
    d = c.dequantize(rec, dtype=torch.float16)
    torch.cuda.synchronize()
    for a, b in zip((rec.codes, rec.norms, rec.signs, rec.rnorms), (rec2.codes, rec2.norms, rec2.signs, rec2.rnorms)):
        assert (a is None and b is None) or torch.equal(a, b)
    assert torch.equal(y, d)
    # oracle sample: rows of the last 65,536 (for the MSE-only launch these are
    # all second tiles of their waves, fetched during the first) and of the first
    rows = np.concatenate([W.sample_rows(65536, 1 / 32, seed=n), n - 65536 + W.sample_rows(65536, 1 / 32, seed=n + 1)])
    idx = torch.from_numpy(rows).cuda()
    xs = x[idx].float().cpu().numpy()
    codes, norms, signs, rnorms = (None if a is None else a[idx].cpu().numpy()
                                   for a in (rec.codes, rec.norms, rec.signs, rec.rnorms))
    codes, norms = codes.view(np.uint32), norms.view(np.uint16)
    signs = None if signs is None else signs.view(np.uint32)
    rnorms = None if rnorms is None else rnorms.view(np.uint16)
    p = _oracle_params(bits, mode)
    PR.check_records(p, xs, codes, norms, signs, rnorms)
    PR.compare_recon(y[idx].float().cpu().numpy(), OC.dequantize(p, PR.record_from_host(codes, norms, signs, rnorms)),
                     OC.half_value(norms), "roundtrip sample", tol=PR.RECON_TOL + 2.0 ** -11)
