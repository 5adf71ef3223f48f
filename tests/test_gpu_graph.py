"""HIP graph capture of the decode-step kernels: a captured roundtrip +
scoring sequence over two buffer sets is replayed several times, with eager
work and synchronisation between replays, and every replay's records,
reconstructions and scores equal the eager results bit for bit (the bench
times these sequences as graph replays)."""
import numpy as np
import pytest

from kv_cache_vector_norm_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_norm_amd as K
    return K


def _host(rec):
    return [None if t is None else t.cpu().numpy().copy() for t in (rec.codes, rec.norms, rec.signs, rec.rnorms)]


@pytest.mark.parametrize("mode,bits", [("qjl", 3), ("mse", 3)])
def test_graph_replays_equal_eager(K, mode, bits):
    dev = torch.device("cuda:0")
    c = K.Codec(bits=bits, seed=0, mode=K.RQ_QJL if mode == "qjl" else K.RQ_MSE)
    n, nq = 4160, 64       # several tiles and a ragged tail
    xs = [torch.from_numpy(W.gaussian(n, seed=s, dtype=np.float16)).to(dev) for s in (11, 12)]
    q = torch.from_numpy(W.queries(nq, seed=13)).to(dev)
    recs = [c.alloc_record(n, dev) for _ in xs]
    ys = [torch.empty_like(x) for x in xs]
    scs = [torch.empty((nq, n), dtype=torch.float32, device=dev) for _ in xs]

    def step(k):
        c.roundtrip(xs[k], rec=recs[k], out=ys[k])
        c.score(q, recs[k], nq, n, out=scs[k])

    for k in range(2):
        step(k)
    torch.cuda.synchronize()
    ref = [(_host(recs[k]), ys[k].cpu().clone(), scs[k].cpu().clone()) for k in range(2)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(2):
            step(k)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(2):
            step(k)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in range(2):              # clobber the outputs between replays
            ys[k].zero_()
            scs[k].fill_(-1.0)
            recs[k].norms.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(2):
            got = _host(recs[k])
            for a, b in zip(got, ref[k][0]):
                assert (a is None and b is None) or np.array_equal(a, b), (rep, k)
            assert torch.equal(ys[k].cpu(), ref[k][1]), (rep, k)
            assert torch.equal(scs[k].cpu(), ref[k][2]), (rep, k)
        _ = (xs[0].float() * 2).sum().item()   # eager work between replays
