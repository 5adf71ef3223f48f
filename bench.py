#!/usr/bin/env python3
"""Throughput of the KV-vector codec hot path on one MI355X.

One step = one pass of the whole path over one batch: the fused rotor
quantize -> dequantize roundtrip of 65,536 fp16 keys (d = 128, 2-bit Lloyd-Max
codes + 1-bit QJL signs = 3 bits, fp16 norms, S = 128 x 128 Gaussian) writing
the record and the fp16 reconstruction, then q.k estimates of 64 fp32 queries
against all 65,536 compressed keys.  Inputs are seeded synthetic data
resident in HBM; the timed steps rotate over enough buffer sets (>= 1 GiB)
that every step reads cold data from HBM rather than from the 256 MB
last-level cache.

Prints one JSON line.  `value` is quant+dequant vectors per second of whole
steps; per-kernel times come from HIP events on the launch stream around
the launches of every eighth timed step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N_VEC = 65536
N_Q = 64
EVENT_EVERY = 8
BITS = 3
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(lay, in_bytes=256, out_bytes=256):
    """Bytes one roundtrip moves per vector: input, record, output."""
    return in_bytes + lay["record_bytes"] + out_bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="also time the MSE-only and the 2-bit + QJL roundtrips over an N sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 262,144-key dense sweep and the model-shaped cache measurements")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many bytes (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench with "
                         "--copy-bytes into profiles/traffic.json, then exit")
    return ap.parse_args()


MAGIC_BUNDLE = b"__CLANG_OFFLOAD_BUNDLE__"


def _elf_sections(data):
    """{name: (offset, size, link, entsize)} of a little-endian ELF64 image."""
    import struct
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = hdrs[shstrndx][4]
    out = {}
    for h in hdrs:
        name = data[names + h[0]:data.index(b"\0", names + h[0])].decode()
        out[name] = (h[4], h[5], h[6], h[9], h[3])
    return out, hdrs


def kernel_code_digest(kernel_symbol=None):
    """First 16 hex digits of a sha256 over built gfx950 machine code in
    librq.so: of one kernel's instructions when `kernel_symbol` (its mangled
    name) is given, else of the whole offload section.  It changes exactly
    when that code does, not for edits that leave it alone."""
    import struct
    with open(os.path.join(ROOT, "kv_cache_vector_norm_amd", "librq.so"), "rb") as f:
        data = f.read()
    secs, _ = _elf_sections(data)
    off, size = secs[".hip_fatbin"][0], secs[".hip_fatbin"][1]
    fatbin = data[off:off + size]
    if kernel_symbol is None:
        return hashlib.sha256(fatbin).hexdigest()[:16]
    start = fatbin.find(MAGIC_BUNDLE)
    while start >= 0:
        n = struct.unpack_from("<Q", fatbin, start + len(MAGIC_BUNDLE))[0]
        pos = start + len(MAGIC_BUNDLE) + 8
        for _ in range(n):
            o, sz, tl = struct.unpack_from("<QQQ", fatbin, pos)
            pos += 24
            triple = fatbin[pos:pos + tl].decode()
            pos += tl
            if "gfx950" not in triple or not sz:
                continue
            co = fatbin[start + o:start + o + sz]
            csecs, hdrs = _elf_sections(co)
            if ".symtab" not in csecs:
                continue
            so, ss, link, ent, _ = csecs[".symtab"]
            stro = hdrs[link][4]
            for k in range(ss // ent):
                st_name, st_info, st_other, st_shndx, st_value, st_size = struct.unpack_from(
                    "<IBBHQQ", co, so + k * ent)
                name = co[stro + st_name:co.index(b"\0", stro + st_name)].decode()
                if name == kernel_symbol and st_size:
                    sh = hdrs[st_shndx]
                    foff = sh[4] + (st_value - sh[3])
                    return hashlib.sha256(co[foff:foff + st_size]).hexdigest()[:16]
        start = fatbin.find(MAGIC_BUNDLE, start + 1)
    raise RuntimeError(f"kernel {kernel_symbol} not found in librq.so")


def measured_traffic(kernel, digest):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel code; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("code") != digest:
        return None
    return e.get("bytes_per_launch")


ROUNDTRIP_KERNEL = "rq_quant_kernel<2, true, true, true, true>"
ROUNDTRIP_SYMBOL = "_ZN3rqk15rq_quant_kernelILi2ELb1ELb1ELb1ELb1EEEvNS_8RotorDevEPKcllPjPtS4_S5_Pcl"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_dispatches(path, counter):
    """{kernel name: [counter value (KiB) per dispatch, in dispatch order]}
    from a rocprofv3 CSV."""
    import csv
    sums, names = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            sums[d] = sums.get(d, 0.0) + float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    out = {}
    for d in sorted(sums, key=int):
        out.setdefault(names[d], []).append(sums[d])
    return out


def ingest_counters(fetch_csv, write_csv, copy_bytes):
    """HBM bytes per roundtrip launch, scaled by a plain copy of known size.

    The calibration copy is the last copyBuffer dispatch of the run (the
    --copy-bytes copies close the process); each counter is divided by what
    it reads for that copy per byte moved."""
    fetch = _counter_dispatches(fetch_csv, "FETCH_SIZE")
    write = _counter_dispatches(write_csv, "WRITE_SIZE")

    def values(d, name):
        hits = [v for k, vs in d.items() if name in k for v in vs]
        if not hits:
            raise SystemExit(f"no dispatch of {name} in the counter CSV")
        return hits

    f_copy = values(fetch, COPY_KERNEL)[-1] * 1024.0
    w_copy = values(write, COPY_KERNEL)[-1] * 1024.0
    fr, wr = values(fetch, ROUNDTRIP_KERNEL), values(write, ROUNDTRIP_KERNEL)
    f_rt = sum(fr) / len(fr) * 1024.0
    w_rt = sum(wr) / len(wr) * 1024.0
    cf, cw = f_copy / copy_bytes, w_copy / copy_bytes
    entry = {
        "code": kernel_code_digest(ROUNDTRIP_SYMBOL),
        "kernel": ROUNDTRIP_KERNEL,
        "dispatches": len(fr),
        "fetch_kib_raw": round(f_rt / 1024.0, 1), "write_kib_raw": round(w_rt / 1024.0, 1),
        "copy_bytes": copy_bytes, "copy_fetch_factor": round(cf, 4), "copy_write_factor": round(cw, 4),
        "fetch_bytes_per_launch": round(f_rt / cf), "write_bytes_per_launch": round(w_rt / cw),
        "bytes_per_launch": round(f_rt / cf + w_rt / cw),
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t["rq_roundtrip_qjl3_f16"] = entry
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(entry))


def cpu_baseline(x_host, q_host):
    """The float64 oracle on a bounded sample, single thread."""
    from threadpoolctl import threadpool_limits
    from oracle import codec as OC
    from oracle import params as OP
    n = 2048
    p = OP.Params(128, BITS, 0, OP.QJL)
    xs = x_host[:n].astype("float64")
    qs = q_host.astype("float64")
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            rec, _ = OC.quantize(p, xs)
            OC.dequantize(p, rec)
            OC.score(p, qs, rec)
            reps += 1
            el = time.perf_counter() - t0
            if el > 8.0 or reps >= 20:
                break
    return {"value": n * reps / el, "unit": "vectors/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of the {N_VEC} keys (roundtrip + {N_Q} queries scored against them), "
                      f"{reps} passes, float64 numpy, 1 thread",
            "scores_per_s": n * N_Q * reps / el}


def _timed(stream, fn, reps):
    """Average microseconds per call of fn(i) over reps back-to-back calls,
    from HIP events on the launch stream (after one untimed call)."""
    import torch
    fn(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        fn(i + 1)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def workload_extras(K, W, dev, stream):
    """Throughput at the other workload shapes (inputs resident in HBM):
    the TurboQuant dense path and the rotor path over 262,144 fp16 N(0,1)
    keys (rotating over 8 such batches, 0.5 GB of input, so launches read
    cold data), and the Qwen2.5-3B- and Llama-3.1-8B-shaped caches quantised
    in one call each plus one decode step of per-layer scoring."""
    import torch
    out = {}
    n = 262144
    sets = 8
    xs = torch.randn((sets * n, 128), device=dev).to(torch.float16)
    ys = torch.empty_like(xs)
    sweep = {}
    for name, mode, bits_list in (("dense", K.RQ_DENSE, (2, 3, 4)), ("dense+qjl", K.RQ_DENSE | K.RQ_QJL, (2, 3, 4, 5)),
                                  ("rotor", K.RQ_MSE, (2, 3, 4)), ("rotor+qjl", K.RQ_QJL, (2, 3, 4, 5))):
        for b in bits_list:
            c = K.Codec(bits=b, seed=0, mode=mode)
            recs = [c.alloc_record(n, dev) for _ in range(sets)]

            def rt(i, c=c, recs=recs):
                k = i % sets
                c.roundtrip(xs[k * n:(k + 1) * n], rec=recs[k], out=ys[k * n:(k + 1) * n])
            us = _timed(stream, rt, 24)
            alg = 256 + c.layout["record_bytes"] + 256
            e = {"us": round(us, 2), "vectors_per_s": round(n / (us * 1e-6), 1),
                 "gbs": round(n * alg / (us * 1e-6) / 1e9, 1)}
            if mode & K.RQ_DENSE:
                # useful MFMA work: Pi x and Pi^T y (and S r, S^T sigma with QJL), 2 flop per MAC
                flops = 2 * 128 * 128 * (4 if mode & K.RQ_QJL else 2)
                e["mfma_tflops"] = round(n * flops / (us * 1e-6) / 1e12, 2)
            sweep[f"{name}{b}"] = e
            del recs, c
    out["keys262144_roundtrip"] = sweep
    del xs, ys

    # paged cache, Qwen2.5-3B shape, one sequence: bulk prefill of 32,768
    # tokens per layer, then decode steps (per layer: append the new token,
    # attend with the current token's key and value at full precision)
    spec = W.QWEN25_3B
    L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
    kcod, vcod = K.Codec(bits=3, seed=0, mode=K.RQ_QJL), K.Codec(bits=3, seed=0, mode=K.RQ_MSE)
    cache = K.Cache(kcod, vcod, layers=L, kv_heads=H, page_tokens=256, max_pages=L * H * (T // 256 + 8))
    seq = cache.open(T + 1024)
    kvl = torch.randn((2, H, T, 128), device=dev).to(torch.float16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for layer in range(L):
        cache.append(seq, layer, kvl[0], kvl[1])
    e1.record(stream)
    torch.cuda.synchronize()
    prefill_us = e0.elapsed_time(e1) * 1e3
    qd = torch.randn((HQ, 128), device=dev)
    kn = torch.randn((H, 1, 128), device=dev).to(torch.float16)
    kcur = kn[:, 0].float().contiguous()
    need = K.lib().rq_cache_attend_workspace(cache.h, HQ, T + 64)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    att = torch.empty((HQ, 128), dtype=torch.float32, device=dev)

    def step(i):
        for layer in range(L):
            cache.attend(seq, layer, qd, k_cur=kcur, v_cur=kcur, out=att, workspace=ws)
            cache.append(seq, layer, kn, kn)
    dec_us = _timed(stream, step, 5)
    out["qwen2.5-3b_paged_cache"] = {"prefill_tokens": T, "prefill_quantize_us": round(prefill_us, 1),
                                     "decode_step_us": round(dec_us, 1), "layers": L, "page_tokens": 256}
    cache.close(seq)
    del cache, kvl, ws, att

    for spec in (W.QWEN25_3B, W.LLAMA31_8B):
        L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
        g = HQ // H
        kv, q = W.kv_cache(spec, device=dev, base_seed=1, torch=torch)
        flat = kv.view(-1, 128)
        c = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
        rec = c.alloc_record(flat.shape[0], dev)
        qus = _timed(stream, lambda i: c.quantize(flat, rec=rec), 3 if flat.shape[0] > 10_000_000 else 10)
        scores = torch.empty((L, HQ, T), dtype=torch.float32, device=dev)
        per = H * T
        subs = [K.Record(rec.codes[l * per:(l + 1) * per], rec.norms[l * per:(l + 1) * per],
                         rec.signs[l * per:(l + 1) * per], rec.rnorms[l * per:(l + 1) * per]) for l in range(L)]

        def decode_layers(i):
            for l in range(L):
                c.score(q[l], subs[l], g, T, T, out=scores[l])

        def decode(i):
            # all layers in one call: query row l * HQ + h reads KV head
            # (l * HQ + h) / g = l * H + h / g, i.e. record rows of layer l
            c.score(q.view(L * HQ, 128), rec, g, T, T, out=scores.view(L * HQ, T))
        lus = _timed(stream, decode_layers, 3)
        dus = _timed(stream, decode, 5)
        # decode attention over the compressed keys and values in one call
        n_k = L * H * T
        krec = K.Record(rec.codes[:n_k], rec.norms[:n_k], rec.signs[:n_k], rec.rnorms[:n_k])
        vrec = K.Record(rec.codes[n_k:], rec.norms[n_k:], rec.signs[n_k:], rec.rnorms[n_k:])
        ws = torch.empty(K.rq_attend_workspace(L * HQ, g, T) + 256, dtype=torch.uint8, device=dev)
        att = torch.empty((L * HQ, 128), dtype=torch.float32, device=dev)
        aus = _timed(stream, lambda i: K.attend(c, c, q.view(L * HQ, 128), krec, vrec, g, T, T, out=att,
                                                workspace=ws), 5)
        # PolarQuant keys of the same cache: bulk quantise, one decode step of
        # scoring (all layers, one call), and attention with those keys
        pc = K.PolarCodec(seed=0)
        pw = pc.alloc_words(n_k, dev)
        pqus = _timed(stream, lambda i: pc.quantize(flat[:n_k], words=pw), 3)
        pdus = _timed(stream, lambda i: pc.score(q.view(L * HQ, 128), pw, g, T, T, out=scores.view(L * HQ, T)), 5)
        paus = _timed(stream, lambda i: K.attend(pc, c, q.view(L * HQ, 128), pw, vrec, g, T, T, out=att,
                                                 workspace=ws), 3)
        # PolarQuant values of the same cache: attention with the rotor keys,
        # and with PolarQuant keys and values
        pv = K.PolarCodec(seed=3)
        pvw = pv.alloc_words(n_k, dev)
        pv.quantize(flat[n_k:], words=pvw)
        pvus = _timed(stream, lambda i: K.attend(c, pv, q.view(L * HQ, 128), krec, pvw, g, T, T, out=att,
                                                 workspace=ws), 3)
        ppus = _timed(stream, lambda i: K.attend(pc, pv, q.view(L * HQ, 128), pw, pvw, g, T, T, out=att,
                                                 workspace=ws), 3)
        del pw, pc, pvw, pv
        nv = flat.shape[0]
        ns = L * HQ * T
        out[spec["name"]] = {
            "vectors": nv, "bulk_quantize_us": round(qus, 1),
            "quantize_vectors_per_s": round(nv / (qus * 1e-6), 1),
            "quantize_gbs": round(nv * (256 + c.layout["record_bytes"]) / (qus * 1e-6) / 1e9, 1),
            "decode_step_us": round(dus, 1), "decode_scores": ns,
            "decode_scores_per_s": round(ns / (dus * 1e-6), 1),
            "decode_step_per_layer_calls_us": round(lus, 1),
            "decode_attention_us": round(aus, 1),
            "decode_attention_keys_per_s": round(n_k / (aus * 1e-6), 1),
            "polar_keys_quantize_us": round(pqus, 1),
            "polar_keys_quantize_gbs": round(n_k * (256 + 64) / (pqus * 1e-6) / 1e9, 1),
            "polar_decode_step_us": round(pdus, 1),
            "polar_decode_scores_per_s": round(ns / (pdus * 1e-6), 1),
            "polar_keys_decode_attention_us": round(paus, 1),
            "polar_values_decode_attention_us": round(pvus, 1),
            "polar_keys_and_values_decode_attention_us": round(ppus, 1)}
        del kv, q, flat, rec, scores, subs, c, krec, vrec, ws, att
        torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.ingest_counters:
        ingest_counters(a.ingest_counters[0], a.ingest_counters[1], a.copy_bytes or (256 << 20))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the codec library runs on a single MI355X and has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import kv_cache_vector_norm_amd as K
    from kv_cache_vector_norm_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    codec = K.Codec(bits=BITS, seed=0, mode=K.RQ_QJL)
    lay = codec.layout
    x_host = W.keys_65536()
    q_host = W.queries_64()
    x0 = torch.from_numpy(x_host).to(dev)
    q = torch.from_numpy(q_host).to(dev)

    set_bytes = N_VEC * (256 + 256 + lay["record_bytes"] + 4 * N_Q)
    nsets = max(2, int(np.ceil((1 << 30) / set_bytes)))
    xs, ys, recs, scs = [], [], [], []
    for i in range(nsets):
        xs.append(x0.clone())
        ys.append(torch.empty((N_VEC, 128), dtype=torch.float16, device=dev))
        recs.append(codec.alloc_record(N_VEC, dev))
        scs.append(torch.empty((N_Q, N_VEC), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        k = i % nsets
        if ev is not None:
            ev[0].record(stream)
        codec.roundtrip(xs[k], rec=recs[k], out=ys[k])
        if ev is not None:
            ev[1].record(stream)
        codec.score(q, recs[k], N_Q, N_VEC, out=scs[k])
        if ev is not None:
            ev[2].record(stream)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    # Per-kernel durations come from HIP events around the two launches of
    # every EVENT_EVERY-th timed step: an event record is a GPU-side marker
    # costing a few microseconds, so bracketing every step would slow the
    # very steps being timed.
    sampled = list(range(0, a.steps, EVENT_EVERY))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rt_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in sampled]))
    sc_ms = float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in sampled]))
    ms_per_step = elapsed * 1e3 / a.steps

    bytes_vec = algorithmic_bytes(lay)
    rt_gbs = N_VEC * bytes_vec / (rt_ms * 1e-3) / 1e9
    digest = kernel_code_digest(ROUNDTRIP_SYMBOL)
    traffic = measured_traffic("rq_roundtrip_qjl3_f16", digest)
    roof = {"bound": "hbm", "achieved": round(rt_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(rt_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "rq_roundtrip (2-bit codes + QJL, fp16 in/out)",
            "algorithmic_bytes_per_vector": bytes_vec, "vectors_per_launch": N_VEC,
            "avg_launch_us": round(rt_ms * 1e3, 2), "launches_timed": len(sampled)}
    score_bytes = N_VEC * lay["record_bytes"] + 4 * N_Q * N_VEC
    extras = {
        "scores_per_s": round(N_Q * N_VEC * a.steps / elapsed, 1),
        "roundtrip_vectors_per_s": round(N_VEC / (rt_ms * 1e-3), 1),
        "score_us": round(sc_ms * 1e3, 2),
        "score_scores_per_s": round(N_Q * N_VEC / (sc_ms * 1e-3), 1),
        "score_gbs": round(score_bytes / (sc_ms * 1e-3) / 1e9, 1),
        "buffer_sets": nsets,
    }

    # MSE-only 3-bit roundtrip (the HBM-bandwidth codec) on the same keys
    mse = K.Codec(bits=3, seed=0, mode=K.RQ_MSE)
    mrec = [mse.alloc_record(N_VEC, dev) for _ in range(nsets)]
    for i in range(a.warmup):
        mse.roundtrip(xs[i % nsets], rec=mrec[i % nsets], out=ys[i % nsets])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        mse.roundtrip(xs[i % nsets], rec=mrec[i % nsets], out=ys[i % nsets])
    e1.record(stream)
    torch.cuda.synchronize()
    mse_us = e0.elapsed_time(e1) * 1e3 / a.steps
    mb = algorithmic_bytes(mse.layout)
    extras["mse3_roundtrip_us"] = round(mse_us, 2)
    extras["mse3_roundtrip_gbs"] = round(N_VEC * mb / (mse_us * 1e-6) / 1e9, 1)
    extras["mse3_roundtrip_vectors_per_s"] = round(N_VEC / (mse_us * 1e-6), 1)

    # QJL-only keys (1 bit in total) on the same keys: roundtrip and scoring
    q1 = K.Codec(bits=1, seed=0, mode=K.RQ_QJL)
    q1rec = [q1.alloc_record(N_VEC, dev) for _ in range(nsets)]
    us1 = _timed(stream, lambda i: q1.roundtrip(xs[i % nsets], rec=q1rec[i % nsets], out=ys[i % nsets]), a.steps)
    sus1 = _timed(stream, lambda i: q1.score(q, q1rec[i % nsets], N_Q, N_VEC, out=scs[i % nsets]), a.steps)
    extras["qjl1_roundtrip_us"] = round(us1, 2)
    extras["qjl1_roundtrip_gbs"] = round(N_VEC * algorithmic_bytes(q1.layout) / (us1 * 1e-6) / 1e9, 1)
    extras["qjl1_score_us"] = round(sus1, 2)
    del q1rec, q1

    # PolarQuant (16-word records, 496 bits of content) on the same keys:
    # fused roundtrip, and the 64 queries scored against all keys
    pc = K.PolarCodec(seed=0)
    pw = [pc.alloc_words(N_VEC, dev) for _ in range(nsets)]
    pus = _timed(stream, lambda i: pc.roundtrip(xs[i % nsets], words=pw[i % nsets], out=ys[i % nsets]), a.steps)
    psus = _timed(stream, lambda i: pc.score(q, pw[i % nsets], N_Q, N_VEC, out=scs[i % nsets]), a.steps)
    extras["polar_roundtrip_us"] = round(pus, 2)
    extras["polar_roundtrip_gbs"] = round(N_VEC * (256 + 64 + 256) / (pus * 1e-6) / 1e9, 1)
    extras["polar_roundtrip_vectors_per_s"] = round(N_VEC / (pus * 1e-6), 1)
    extras["polar_score_us"] = round(psus, 2)
    extras["polar_scores_per_s"] = round(N_VEC * N_Q / (psus * 1e-6), 1)
    del pw, pc

    if a.sweep:
        # the MSE-only 3-bit roundtrip and the headline 2-bit + QJL one over N
        sweeps = {"mse3_sweep": (mse, mb), "qjl3_sweep": (codec, algorithmic_bytes(lay))}
        for key, (cdc, nb) in sweeps.items():
            sweep = {}
            for n in (65536, 262144, 1048576, 4194304, 16777216):
                xb = torch.randn((n, 128), device=dev).to(torch.float16)
                yb = torch.empty_like(xb)
                rb = cdc.alloc_record(n, dev)
                for _ in range(3):
                    cdc.roundtrip(xb, rec=rb, out=yb)
                reps = max(3, min(50, int(4e8 // (n * 566))))
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    cdc.roundtrip(xb, rec=rb, out=yb)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                sweep[str(n)] = {"us": round(us, 2), "gbs": round(n * nb / (us * 1e-6) / 1e9, 1)}
                del xb, yb, rb
            extras[key] = sweep

    # achievable-HBM reference: a plain device copy of 1 GiB (read + write)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cus = _timed(stream, lambda i: dst.copy_(src), 5)
    extras["copy_1gib_gbs"] = round(2 * (1 << 30) / (cus * 1e-6) / 1e9, 1)
    del src, dst

    if not a.no_workloads:
        extras["workloads"] = workload_extras(K, W, dev, stream)

    if a.copy_bytes:
        src = torch.empty(a.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "quant+dequant vectors/s (d=128, 3-bit) + % HBM roofline; q·k scores/s",
        "value": round(N_VEC * a.steps / elapsed, 1),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "65,536 fp16 N(0,1) keys d=128, RotorQuant 2-bit MSE + 1-bit QJL (3 bits), "
                               "fused roundtrip + q.k estimates of 64 fp32 queries",
                   "vectors": N_VEC, "queries": N_Q, "bits": BITS, "mode": "rotor+qjl", "seed": 0},
        "roofline": roof,
        "kernel_code": digest,
        **extras,
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x_host, q_host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
