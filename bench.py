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
steps (host clock around the K steps).  Kernel times come from HIP events on
the launch stream around back-to-back launches over the rotating buffer sets
(median of several trials), so they hold only the kernels and the gaps
between them.  The line also carries the reference copy of the same bytes
(the practical HBM ceiling), the 1,024-vector fp32 quality row, the
roundtrips over an N sweep, the other codecs and workload shapes, and the
float64 CPU oracle timed on one core and on all host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
                    [--no-workloads] [--no-cpu]
    python bench.py --profile-set        # the kernels the profiles/ summaries cover
    python bench.py --summarize DIR      # rocprofv3 CSVs of --profile-set -> profiles/
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N_VEC = 65536
N_Q = 64
BITS = 3
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
CPU_SHARE = 16          # host threads one GPU's share of the box may use
ORACLE_SECONDS = 8.0    # wall time of each CPU oracle leg


def algorithmic_bytes(lay, in_bytes=256, out_bytes=256):
    """Bytes one roundtrip moves per vector: input, record, output."""
    return in_bytes + lay["record_bytes"] + out_bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=10, help="trials of back-to-back launches per kernel time")
    ap.add_argument("--no-sweep", action="store_true", help="skip the roundtrips over the N sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 262,144-key dense sweep and the model-shaped cache measurements")
    ap.add_argument("--profile-set", action="store_true",
                    help="run each profiled kernel a few times (for rocprofv3) and exit")
    ap.add_argument("--summarize", metavar="DIR",
                    help="turn rocprofv3 runs of --profile-set under DIR into profiles/ summaries, then exit")
    ap.add_argument("--trace-command", default=None,
                    help="with --trace-summary: the command that made the trace, written as the summary's header")
    ap.add_argument("--trace-title", default=None, help="with --trace-summary: the header's title")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_CSV", "OUT_MD"),
                    help="group a rocprofv3 kernel trace by kernel and grid size into a markdown table, then exit")
    return ap.parse_args()


# ------------------------------------------------- machine-code digests --
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


def kernel_digests():
    """{mangled kernel symbol: first 16 hex digits of a sha256 over its
    gfx950 machine code} for every kernel in librq.so (built here from this
    repository's sources).  A digest changes exactly when that code does."""
    import struct
    with open(os.path.join(ROOT, "kv_cache_vector_norm_amd", "librq.so"), "rb") as f:
        data = f.read()
    secs, _ = _elf_sections(data)
    off, size = secs[".hip_fatbin"][0], secs[".hip_fatbin"][1]
    fatbin = data[off:off + size]
    out = {"": hashlib.sha256(fatbin).hexdigest()[:16]}
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
                if st_size and (st_info & 0xF) == 2 and not name.endswith(".kd"):
                    sh = hdrs[st_shndx]
                    foff = sh[4] + (st_value - sh[3])
                    out[name] = hashlib.sha256(co[foff:foff + st_size]).hexdigest()[:16]
        start = fatbin.find(MAGIC_BUNDLE, start + 1)
    return out


def kernel_code_digest(kernel_symbol=None, _cache={}):
    """Digest of one kernel's machine code (its mangled name), or of the
    whole offload section when kernel_symbol is None."""
    if "d" not in _cache:
        _cache["d"] = kernel_digests()
    d = _cache["d"]
    key = kernel_symbol or ""
    if key not in d:
        raise RuntimeError(f"kernel {kernel_symbol} not found in librq.so")
    return d[key]


def digest_of(mangled_part):
    """Digest of the one kernel whose mangled name contains `mangled_part`."""
    hits = [s for s in kernel_digests() if s and mangled_part in s]
    if len(hits) != 1:
        raise RuntimeError(f"{len(hits)} kernels match {mangled_part}")
    return kernel_code_digest(hits[0])


ROUNDTRIP_KERNEL = "rq_quant_kernel<2, true, true, true, true, 8>"
ROUNDTRIP_SYMBOL = "_ZN3rqk15rq_quant_kernelILi2ELb1ELb1ELb1ELb1ELi8EEEvNS_8RotorDevEPKcllPjPtS4_S5_Pcl"


# -------------------------------------------------- profiled kernel set --
# Each case of --profile-set: (label, kernel name prefix in rocprofv3 output,
# mangled-name part for the code digest, launches (one warm-up + timed),
# algorithmic bytes per launch, useful MFMA flops per launch, what it is).
def profile_cases():
    n1, nm, nd = N_VEC, 1 << 20, 262144
    fl = 2 * 128 * 128      # flops of one 128 x 128 matrix-vector product
    # Qwen2.5-3B-shaped decode step: keys (or values) of every layer and the
    # estimates of every query row
    from kv_cache_vector_norm_amd import workloads as W
    qs = W.QWEN25_3B
    qk, qr, qt = qs["layers"] * qs["kv_heads"] * qs["tokens"], qs["layers"] * qs["q_heads"], qs["tokens"]
    return [
        ("copy_65536_same_bytes", "rqk::copy_kernel", "11copy_kernel", 4, n1 * 568, 0,
         "reference copy of 65,536 x 568 B (read 284 B, write 284 B per vector)"),
        ("rq_roundtrip_qjl3_65536", "rqk::rq_quant_kernel<2, true, true, true, true, 8>",
         "15rq_quant_kernelILi2ELb1ELb1ELb1ELb1ELi8EE", 4, n1 * 568, 0,
         "rotor roundtrip, 2-bit codes + QJL, fp16 in/out, 65,536 keys (the step's codec kernel)"),
        ("rq_score_64x65536", "rqk::score_kernel<2, true, true, 2, false>", "12score_kernelILi2ELb1ELb1ELi2ELb0EE", 4,
         n1 * 56 + 4 * N_Q * n1, 0, "q.k estimates of 64 queries against 65,536 compressed keys"),
        ("rq_roundtrip_mse3_65536", "rqk::rq_quant_kernel<3, false, true, true, true, 4>",
         "15rq_quant_kernelILi3ELb0ELb1ELb1ELb1ELi4EE", 4, n1 * 566, 0,
         "rotor roundtrip, 3-bit MSE only, fp16 in/out, 65,536 keys"),
        ("pq_roundtrip_65536", "rqk::pq_quant_kernel<true, true, true, 8>",
         "15pq_quant_kernelILb1ELb1ELb1ELi8EE", 4, n1 * (256 + 64 + 256), n1 * 2 * fl * 3,
         "PolarQuant roundtrip, fp16 in/out, 65,536 keys (flops: Pi x, Pi^T y~, 3 fp16 MFMAs each)"),
        ("rq_roundtrip_mse3_1048576", "rqk::rq_quant_kernel<3, false, true, true, true, 4>",
         "15rq_quant_kernelILi3ELb0ELb1ELb1ELb1ELi4EE", 4, nm * 566, 0,
         "rotor roundtrip, 3-bit MSE only, fp16 in/out, 1,048,576 keys"),
        ("copy_1048576_same_bytes", "rqk::copy_kernel", "11copy_kernel", 4, nm * 566, 0,
         "reference copy of 1,048,576 x 566 B"),
        ("tq_roundtrip_dense3_262144", "rqk::tq_quant_kernel<3, false, true, true, true,",
         "15tq_quant_kernelILi3ELb0ELb1ELb1ELb1ELi", 4, nd * (256 + 50 + 256), nd * 2 * fl * 3,
         "TurboQuant roundtrip, 3-bit MSE, fp16 in/out, 262,144 keys (flops: Pi x, Pi^T y, 3 fp16 MFMAs each)"),
        ("tq_roundtrip_dense_qjl3_262144", "rqk::tq_quant_kernel<2, true, true, true, true,",
         "15tq_quant_kernelILi2ELb1ELb1ELb1ELb1ELi", 4, nd * (256 + 52 + 256), nd * fl * (3 + 3 + 2 + 2 + 1),
         "TurboQuant roundtrip, 2-bit + QJL, fp16 in/out, 262,144 keys"),
        ("rq_attend_scores_qwen", "rqk::score_kernel<2, true, true, 0, false>",
         "12score_kernelILi2ELb1ELb1ELi0ELb0EE", 4, qk * 56 + 4 * qr * qt, 0,
         "decode attention pass 1 (estimates and per-workgroup row maxima), Qwen2.5-3B-shaped cache, all layers"),
        ("rq_attend_values_qwen", "rqk::attend_values16_kernel<2, true, true>",
         "22attend_values16_kernelILi2ELb1ELb1EE", 4, qk * 56 + 4 * qr * qt, 0,
         "decode attention value pass (centroid and sign sums), Qwen2.5-3B-shaped cache, all layers"),
        ("copy_calibration_256mib", "rqk::copy_kernel", "11copy_kernel", 1, 2 * (256 << 20), 0,
         "counter calibration: reference copy of 256 MiB"),
    ]


def profile_set(K, W, dev):
    """Launch every case of profile_cases() in order: one warm-up and three
    timed launches each (one launch for the calibration copy), nothing else
    from this library in between."""
    import torch
    stream = torch.cuda.current_stream()

    def note(label):
        torch.cuda.synchronize()
        print(f"profile-set: {label}", flush=True)

    x = torch.from_numpy(W.keys_65536()).to(dev)
    q = torch.from_numpy(W.queries_64()).to(dev)
    big = torch.empty((1 << 20, 128), dtype=torch.float16, device=dev)
    big.normal_()
    ybig = torch.empty_like(big)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.random_(0, 255)

    def copy(nbytes, times):
        for _ in range(times):
            K.rq_bench_copy(src, dst, nbytes, stream)

    note("copy_65536_same_bytes")
    copy(N_VEC * 284, 4)
    # the 65,536-vector cases rotate over buffer sets as the bench's own
    # timing does: the warm-up runs on the last set made, the timed launches
    # on the first ones, which later sets have pushed out of the caches
    sets = 9
    order = [sets - 1, 0, 1, 2]
    xs = [x.clone() for _ in range(sets)]
    ys = [torch.empty_like(x) for _ in range(sets)]
    c = K.Codec(bits=3, seed=0, mode=K.RQ_QJL)
    recs = [c.alloc_record(N_VEC, dev) for _ in range(sets)]
    scs = [torch.empty((N_Q, N_VEC), dtype=torch.float32, device=dev) for _ in range(sets)]
    for i in range(sets):
        c.quantize(xs[i], rec=recs[i])    # (the quantiser alone: another kernel)
    note("rq_roundtrip_qjl3_65536")
    for i in order:
        c.roundtrip(xs[i], rec=recs[i], out=ys[i])
    note("rq_score_64x65536")
    for i in order:
        c.score(q, recs[i], N_Q, N_VEC, out=scs[i])
    m = K.Codec(bits=3, seed=0, mode=K.RQ_MSE)
    mrecs = [m.alloc_record(N_VEC, dev) for _ in range(sets)]
    note("rq_roundtrip_mse3_65536")
    for i in order:
        m.roundtrip(xs[i], rec=mrecs[i], out=ys[i])
    pc = K.PolarCodec(seed=0)
    pws = [pc.alloc_words(N_VEC, dev) for _ in range(sets)]
    note("pq_roundtrip_65536")
    for i in order:
        pc.roundtrip(xs[i], words=pws[i], out=ys[i])
    del xs, ys, recs, scs, mrecs, pws, pc
    mrec = m.alloc_record(1 << 20, dev)
    note("rq_roundtrip_mse3_1048576")
    for _ in range(4):
        m.roundtrip(big, rec=mrec, out=ybig)
    note("copy_1048576_same_bytes")
    copy((1 << 20) * 283, 4)
    xd = big[:262144]
    yd = ybig[:262144]
    for label, bits, mode in (("tq_roundtrip_dense3_262144", 3, K.RQ_DENSE),
                              ("tq_roundtrip_dense_qjl3_262144", 3, K.RQ_DENSE | K.RQ_QJL)):
        dc = K.Codec(bits=bits, seed=0, mode=mode)
        drec = dc.alloc_record(262144, dev)
        note(label)
        for _ in range(4):
            dc.roundtrip(xd, rec=drec, out=yd)
        del dc, drec
    del big, ybig, mrec
    spec = W.QWEN25_3B
    L, H, T, HQ = spec["layers"], spec["kv_heads"], spec["tokens"], spec["q_heads"]
    kv, qq = W.kv_cache(spec, device=dev, base_seed=1, torch=torch)
    flat = kv.view(-1, 128)
    crec = c.alloc_record(flat.shape[0], dev)
    c.quantize(flat, rec=crec)
    n_k = L * H * T
    krec = K.Record(crec.codes[:n_k], crec.norms[:n_k], crec.signs[:n_k], crec.rnorms[:n_k])
    vrec = K.Record(crec.codes[n_k:], crec.norms[n_k:], crec.signs[n_k:], crec.rnorms[n_k:])
    g = HQ // H
    ws = torch.empty(K.rq_attend_workspace(L * HQ, g, T) + 256, dtype=torch.uint8, device=dev)
    att = torch.empty((L * HQ, 128), dtype=torch.float32, device=dev)
    note("rq_attend_qwen (rq_attend_scores_qwen, rq_attend_values_qwen)")
    for _ in range(4):
        K.attend(c, c, qq.view(L * HQ, 128), krec, vrec, g, T, T, out=att, workspace=ws)
    del kv, crec, ws
    note("copy_calibration_256mib")
    copy(256 << 20, 1)
    torch.cuda.synchronize()
    print("profile-set: done", flush=True)


# --------------------------------------------- rocprofv3 CSV summaries --
PMC_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "busy": ["VALUBusy", "MfmaUtil", "OccupancyPercent", "LDSBankConflict"],
    "insts": ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS"],
    "insts2": ["SQ_INSTS_SALU", "SQ_INSTS_SMEM", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR"],
}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for base, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(base, fn)
    return None


def _col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return None


def _assign(names_in_order, cases):
    """Dispatch indices (in order) of each case: the k-th group of `launches`
    dispatches whose kernel name (without a leading "void ") starts with the
    case's prefix."""
    names_in_order = [nm[5:] if nm.startswith("void ") else nm for nm in names_in_order]
    taken = {}
    out = {}
    for label, prefix, _, launches, *_ in cases:
        idx = [i for i, nm in enumerate(names_in_order) if nm.startswith(prefix)]
        start = taken.get(prefix, 0)
        out[label] = idx[start:start + launches]
        taken[prefix] = start + launches
    return out


def summarize(d):
    """profiles/ summaries from rocprofv3 runs of `bench.py --profile-set`
    kept under d: kt/ (kernel trace) and one directory per PMC pass."""
    cases = profile_cases()
    trace = _read_csv(_find(os.path.join(d, "kt"), "kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in trace]
    where = _assign(names, cases)
    res = {}
    for label, prefix, mpart, launches, alg, flops, what in cases:
        rows = [trace[i] for i in where[label]]
        timed = rows[1:] if len(rows) > 1 else rows
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        r0 = rows[0] if rows else {}
        res[label] = {
            "what": what, "kernel": prefix, "code": digest_of(mpart), "launches": len(rows),
            "avg_us": round(sum(durs) / len(durs), 2) if durs else None,
            "vgpr": _col(r0, "Arch_VGPR_Count", "VGPR_Count", "arch_vgpr_count"),
            "agpr": _col(r0, "Accum_VGPR_Count", "accum_vgpr_count"),
            "sgpr": _col(r0, "SGPR_Count", "sgpr_count"),
            "lds_bytes": _col(r0, "LDS_Block_Size", "Group_Segment_Size", "lds_block_size"),
            "scratch_bytes": _col(r0, "Scratch_Size", "Private_Segment_Size", "scratch_size"),
            "grid": _col(r0, "Grid_Size", "Grid_Size_X", "grid_size"),
            "workgroup": _col(r0, "Workgroup_Size", "Workgroup_Size_X", "workgroup_size"),
            "alg_bytes": alg, "flops": flops,
        }
        if durs and alg:
            res[label]["alg_gbs"] = round(alg / (res[label]["avg_us"] * 1e-6) / 1e9, 1)
            res[label]["frac_hbm"] = round(res[label]["alg_gbs"] / HBM_PEAK_GBS, 4)
        if durs and flops:
            res[label]["mfma_tflops"] = round(flops / (res[label]["avg_us"] * 1e-6) / 1e12, 2)
    # counter passes: per dispatch, in dispatch order
    counters = {}
    for pas in PMC_PASSES:
        path = _find(os.path.join(d, pas), "counter_collection.csv")
        if not path:
            continue
        rows = _read_csv(path)
        per = {}
        for r in rows:
            did = int(r["Dispatch_Id"])
            e = per.setdefault(did, {"name": r["Kernel_Name"], "vals": {}})
            cn = r["Counter_Name"]
            e["vals"][cn] = e["vals"].get(cn, 0.0) + float(r["Counter_Value"])
        order = sorted(per)
        nm = [per[i]["name"] for i in order]
        w = _assign(nm, cases)
        for label in w:
            ds = [per[order[i]]["vals"] for i in w[label]]
            ds = ds[1:] if len(ds) > 1 else ds
            if not ds:
                continue
            for cn in ds[0]:
                counters.setdefault(label, {})[cn] = sum(v.get(cn, 0.0) for v in ds) / len(ds)
    # HBM bytes: counters scaled by what they read for the calibration copy
    cal = counters.get("copy_calibration_256mib", {})
    cal_bytes = 256 << 20
    cf = cal.get("FETCH_SIZE", 0.0) * 1024.0 / cal_bytes
    cw = cal.get("WRITE_SIZE", 0.0) * 1024.0 / cal_bytes
    traffic = {}
    for label, c in counters.items():
        e = res[label]
        e["counters"] = {k: round(v, 3) for k, v in sorted(c.items())}
        if cf > 0 and cw > 0 and "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            fb = c["FETCH_SIZE"] * 1024.0 / cf
            wb = c["WRITE_SIZE"] * 1024.0 / cw
            e["hbm_read_bytes"], e["hbm_write_bytes"] = round(fb), round(wb)
            if e["alg_bytes"]:
                e["traffic_over_alg"] = round((fb + wb) / e["alg_bytes"], 3)
            traffic[label] = {"code": e["code"], "kernel": e["kernel"], "fetch_bytes_per_launch": round(fb),
                              "write_bytes_per_launch": round(wb), "bytes_per_launch": round(fb + wb),
                              "copy_fetch_factor": round(cf, 4), "copy_write_factor": round(cw, 4)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(ROOT, "profiles", "kernels.json"), "w") as f:
        json.dump(res, f, indent=1)
    with open(os.path.join(ROOT, "profiles", "profile_set_counters.md"), "w") as f:
        f.write(profile_markdown(res, cf, cw))
    print(json.dumps(res, indent=1))


PROFILE_COMMANDS = """    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/kt -o kt -- python3 $R/bench.py --profile-set
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/fetch -o p -- python3 $R/bench.py --profile-set
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/write -o p -- python3 $R/bench.py --profile-set
    rocprofv3 --pmc VALUBusy MfmaUtil OccupancyPercent LDSBankConflict --output-format csv -d $R/gpurun_out/prof/busy -o p -- python3 $R/bench.py --profile-set
    rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS --output-format csv -d $R/gpurun_out/prof/insts -o p -- python3 $R/bench.py --profile-set
    rocprofv3 --pmc SQ_INSTS_SALU SQ_INSTS_SMEM SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR --output-format csv -d $R/gpurun_out/prof/insts2 -o p -- python3 $R/bench.py --profile-set
    python3 bench.py --summarize gpurun_out/prof          # (R = the repository root)
"""


def profile_markdown(res, cf, cw):
    """One table per measured quantity over the profiled kernels."""
    def g(e, k):
        return e.get("counters", {}).get(k)

    def fmt(v, nd=1):
        if v is None:
            return "-"
        if isinstance(v, str):
            return v
        return f"{v:,.{nd}f}" if isinstance(v, float) else f"{v:,}"
    out = ["# rocprofv3 counters of the profiled kernels (`bench.py --profile-set`)", "",
           "Commands (MI355X; one counter set per run, each over the same launch sequence):", "",
           PROFILE_COMMANDS, "",
           "Each kernel runs one warm-up and three measured launches (the 256 MiB calibration copy",
           "once); figures are means over the measured launches.  Machine-code digests tie each",
           "row to the kernel as built (`kernel_code` / `profiles/kernels.json`).  HBM bytes are",
           f"FETCH_SIZE and WRITE_SIZE scaled by what they read for the 256 MiB copy_kernel (fetch factor "
           f"{cf:.4f}, write factor {cw:.4f} per byte moved).", "",
           "| kernel (workload) | code | avg us (trace) | alg. bytes | alg. GB/s | of 8 TB/s | HBM bytes read + written "
           "| HBM / alg. | VGPR | LDS B | scratch B/lane |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, e in res.items():
        hbm = (e["hbm_read_bytes"] + e["hbm_write_bytes"]) if "hbm_read_bytes" in e else None
        out.append(f"| {label} | {e['code']} | {fmt(e['avg_us'], 2)} | {fmt(e['alg_bytes'] or None)} | "
                   f"{fmt(e.get('alg_gbs'))} | {fmt(e.get('frac_hbm'), 3)} | {fmt(hbm)} | "
                   f"{fmt(e.get('traffic_over_alg'), 3)} | {e['vgpr']} | {e['lds_bytes']} | {e['scratch_bytes']} |")
    out += ["", "Busy and occupancy (rocprofv3 derived counters; percent of the GPU's time over the dispatch):", "",
            "| kernel | VALUBusy % | MfmaUtil % | OccupancyPercent | LDSBankConflict % | useful MFMA TFLOP/s |",
            "|---|---|---|---|---|---|"]
    for label, e in res.items():
        out.append(f"| {label} | {fmt(g(e, 'VALUBusy'))} | {fmt(g(e, 'MfmaUtil'))} | {fmt(g(e, 'OccupancyPercent'))} | "
                   f"{fmt(g(e, 'LDSBankConflict'))} | {fmt(e.get('mfma_tflops'), 2)} |")
    out += ["", "Instruction counts per dispatch (all waves; per wave = count / SQ_WAVES):", "",
            "| kernel | SQ_WAVES | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | SMEM / wave | VMEM rd / wave "
            "| VMEM wr / wave |", "|---|---|---|---|---|---|---|---|---|"]
    for label, e in res.items():
        w = g(e, "SQ_WAVES")

        def pw(k):
            v = g(e, k)
            return fmt(v / w) if v is not None and w else "-"
        out.append(f"| {label} | {fmt(w, 0)} | {pw('SQ_INSTS_VALU')} | {pw('SQ_INSTS_MFMA')} | {pw('SQ_INSTS_LDS')} | "
                   f"{pw('SQ_INSTS_SALU')} | {pw('SQ_INSTS_SMEM')} | {pw('SQ_INSTS_VMEM_RD')} | "
                   f"{pw('SQ_INSTS_VMEM_WR')} |")
    out += ["", "Workloads:", ""]
    out += [f"- {label}: {e['what']}" for label, e in res.items()]
    return "\n".join(out) + "\n"


def trace_summary(path):
    """Markdown table of a rocprofv3 kernel trace grouped by kernel and grid
    size (this library's kernels): calls, average / minimum / maximum
    duration in microseconds."""
    rows = _read_csv(path)
    groups = {}
    for r in rows:
        nm = r["Kernel_Name"]
        nm = nm[5:] if nm.startswith("void ") else nm
        if not nm.startswith("rqk::"):
            continue                # the library's kernels only (not torch's set-up kernels)
        nm = nm.split("(")[0]
        key = (nm, int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | grid (threads) | calls | avg us | min us | max us | total us |", "|---|---|---|---|---|---|---|"]
    for (nm, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {nm} | {grid:,} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                     f"{sum(d):,.1f} |")
    return "\n".join(lines) + "\n"


def measured_traffic(label, digest):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel code; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(label)
    if not e or e.get("code") != digest:
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------- CPU oracle baseline --
def _oracle_leg(args):
    """One worker of the CPU baseline: the float64 oracle's roundtrip and
    64-query scoring (or bulk quantisation only) of rows [lo, hi), repeated
    for `seconds`, on one BLAS thread (pinned to `cpu` when given)."""
    lo, hi, seconds, cpu, kind = args
    if cpu is not None:
        os.sched_setaffinity(0, {cpu})
    import numpy as np
    from threadpoolctl import threadpool_limits
    from kv_cache_vector_norm_amd import workloads as W
    from oracle import codec as OC
    from oracle import params as OP
    p = OP.Params(128, BITS, 0, OP.QJL)
    if kind == "lowrank":
        import torch
        k, _, _ = W.lowrank_head(hi - lo, W.cache_seed(1, 0, 0), torch=torch)
        xs = k.numpy().astype(np.float64)
    else:
        xs = W.keys_65536()[lo:hi].astype(np.float64)
    qs = W.queries_64().astype(np.float64)
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            rec, _ = OC.quantize(p, xs)
            if kind != "lowrank":
                OC.dequantize(p, rec)
                OC.score(p, qs, rec)
            reps += 1
            el = time.perf_counter() - t0
            if el > seconds:
                break
    return (hi - lo) * reps, el


def cpu_baseline():
    """The float64 oracle (as it stands) on the host cores: one pinned core,
    then all cores of this GPU's share, each worker on its own contiguous
    2,048-key slice of the 65,536 keys, plus the bulk-quantisation rate on
    low-rank keys of the model-shaped caches (one core), extrapolated to the
    Qwen2.5-3B- and Llama-3.1-8B-shaped caches.  Workers are spawned before
    anything touches the GPU."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    cpus = sorted(os.sched_getaffinity(0))
    ncores = min(CPU_SHARE, len(cpus))
    slice_n = 2048
    with ctx.Pool(1) as pool:
        v1, e1 = pool.map(_oracle_leg, [(0, slice_n, ORACLE_SECONDS, cpus[0], "step")])[0]
        vq, eq = pool.map(_oracle_leg, [(0, slice_n, ORACLE_SECONDS / 2, cpus[0], "lowrank")])[0]
    with ctx.Pool(ncores) as pool:
        legs = [(i * slice_n, (i + 1) * slice_n, ORACLE_SECONDS, cpus[i], "step") for i in range(ncores)]
        res = pool.map(_oracle_leg, legs)
    one = v1 / e1
    allc = sum(v / e for v, e in res)
    qrate = vq / eq
    qwen = 36 * 2 * 2 * 32768
    llama = 32 * 8 * 2 * 131072
    return {
        "value": round(allc, 1), "unit": "vectors/s", "cores": ncores, "kind": "oracle",
        "sample": (f"float64 numpy oracle, one BLAS thread per process: {ncores} processes, each on its own "
                   f"{slice_n}-key slice of the {N_VEC} keys (roundtrip + {N_Q} queries scored per key), "
                   f"{ORACLE_SECONDS:.0f} s each"),
        "scores_per_s": round(allc * N_Q, 1),
        "one_core": {"value": round(one, 1), "unit": "vectors/s", "cores": 1, "scores_per_s": round(one * N_Q, 1),
                     "sample": f"{slice_n} keys, {int(v1 // slice_n)} passes, pinned to cpu {cpus[0]}"},
        "bulk_quantize_one_core": {
            "vectors_per_s": round(qrate, 1),
            "sample": f"{slice_n} low-rank + outlier keys of one (layer, KV head), quantise only",
            "qwen2.5-3b_cache_s_extrapolated": round(qwen / qrate, 1),
            "llama3.1-8b_cache_s_extrapolated": round(llama / qrate, 1)},
    }


# -------------------------------------------------------------- timing --
def _b2b(stream, fn, reps, trials):
    """Median and minimum over `trials` of the average microseconds per call
    of fn(i) over `reps` back-to-back calls, from HIP events recorded on the
    launch stream (after one untimed call)."""
    import torch
    fn(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ts = []
    i = 1
    for _ in range(trials):
        e0.record(stream)
        for _ in range(reps):
            fn(i)
            i += 1
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    return statistics.median(ts), min(ts)


def _timed(stream, fn, reps):
    return _b2b(stream, fn, reps, 1)[0]


def quality_row(K, W, dev, stream):
    """1,024 fp32 unit vectors, rotor MSE-only 3 bits, roundtrip fp32 ->
    fp32: MSE and mean cosine of the GPU reconstruction and of the oracle's,
    and the launch time at this size (latency-bound)."""
    import numpy as np
    import torch
    from oracle import codec as OC
    from oracle import params as OP
    xh = W.unit_vectors_1024()
    x = torch.from_numpy(xh).to(dev)
    c = K.Codec(bits=3, seed=0, mode=K.RQ_MSE)
    rec, y = c.roundtrip(x)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().astype(np.float64)
    xd = xh.astype(np.float64)

    def mse_cos(r):
        mse = float(np.mean(np.sum((xd - r) ** 2, axis=1)))
        cos = float(np.mean(np.sum(xd * r, axis=1) / (np.linalg.norm(xd, axis=1) * np.linalg.norm(r, axis=1))))
        return mse, cos
    g_mse, g_cos = mse_cos(yh)
    p = OP.Params(128, 3, 0, OP.MSE)
    o_mse, o_cos = mse_cos(OC.roundtrip(p, xd)[1])
    us, us_min = _b2b(stream, lambda i: c.roundtrip(x, rec=rec, out=y), 50, 5)
    # one launch after an idle device: event pair around a single call
    lat = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(20):
        torch.cuda.synchronize()
        e0.record(stream)
        c.roundtrip(x, rec=rec, out=y)
        e1.record(stream)
        e1.synchronize()
        lat.append(e0.elapsed_time(e1) * 1e3)
    return {"workload": "1,024 fp32 unit vectors (N(0,1) normalised, seed 0), rotor 3-bit MSE, fp32 in/out",
            "mse": round(g_mse, 6), "cosine": round(g_cos, 6), "oracle_mse": round(o_mse, 6),
            "oracle_cosine": round(o_cos, 6), "pages_mse_cosine": [0.034, 0.983],
            "us_per_launch_back_to_back": round(us, 2), "single_launch_us": round(statistics.median(lat), 2)}


def sweeps(K, dev, stream, codecs):
    """Roundtrip rate over N (65,536 * 4^k up to 16,777,216) for each codec
    (rotor sessions and PolarQuant), beside the reference copy of the same
    bytes at each N.  Below 1 M
    vectors the launches rotate over enough buffer sets to read cold data."""
    import torch
    out = {}
    nmax = 16777216
    xb = torch.empty((nmax, 128), dtype=torch.float16, device=dev)
    xb.normal_()
    yb = torch.empty_like(xb)
    ccap = nmax * 288      # half of the largest record + fp16 in/out (PolarQuant: 576 B per vector)
    csrc = torch.empty(ccap, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    for key, cdc in codecs.items():
        nb = algorithmic_bytes(cdc.layout)
        polar = hasattr(cdc, "alloc_words")
        rb = cdc.alloc_words(nmax, dev) if polar else cdc.alloc_record(nmax, dev)
        sweep = {}
        for n in (65536, 262144, 1048576, 4194304, 16777216):
            sets = max(1, min(nmax // n, (1 << 30) // (n * nb)))
            half = n * nb // 2
            if sets * half > ccap or half % 16:
                raise RuntimeError("reference copy sizes outside its buffers")

            def rt(i, n=n, sets=sets):
                k = i % sets
                if polar:
                    cdc.roundtrip(xb[k * n:(k + 1) * n], words=rb[k * n:(k + 1) * n], out=yb[k * n:(k + 1) * n])
                    return
                r = K.Record(rb.codes[k * n:(k + 1) * n], rb.norms[k * n:(k + 1) * n],
                             None if rb.signs is None else rb.signs[k * n:(k + 1) * n],
                             None if rb.rnorms is None else rb.rnorms[k * n:(k + 1) * n])
                cdc.roundtrip(xb[k * n:(k + 1) * n], rec=r, out=yb[k * n:(k + 1) * n])

            def cp(i, n=n, sets=sets, half=half):
                k = i % sets
                K.rq_bench_copy(csrc[k * half:(k + 1) * half], cdst[k * half:(k + 1) * half], half, stream)
            reps = max(3, min(64, int(4e9 // (n * nb))))
            us, _ = _b2b(stream, rt, reps, 5)
            cus, _ = _b2b(stream, cp, reps, 5)
            gbs = n * nb / (us * 1e-6) / 1e9
            cgbs = 2 * half / (cus * 1e-6) / 1e9
            sweep[str(n)] = {"us": round(us, 2), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                             "copy_gbs": round(cgbs, 1), "frac_copy": round(gbs / cgbs, 4)}
        out[key] = sweep
        del rb
    del xb, yb, csrc, cdst
    torch.cuda.empty_cache()
    return out


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
            us, _ = _b2b(stream, rt, 8, 5)
            alg = 256 + c.layout["record_bytes"] + 256
            e = {"us": round(us, 2), "vectors_per_s": round(n / (us * 1e-6), 1),
                 "gbs": round(n * alg / (us * 1e-6) / 1e9, 1), "frac_hbm": round(n * alg / (us * 1e-6) / 8e12, 4)}
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
    # the same step over all layers in two calls (attend, then append)
    ql = qd.unsqueeze(0).expand(L, HQ, 128).contiguous()
    kl = kcur.unsqueeze(0).expand(L, H, 128).contiguous()
    knl = kn.unsqueeze(0).expand(L, H, 1, 128).contiguous()
    needl = K.lib().rq_cache_attend_layers_workspace(cache.h, L, HQ, T + 64)
    wsl = torch.empty(needl + 256, dtype=torch.uint8, device=dev)
    attl = torch.empty((L * HQ, 128), dtype=torch.float32, device=dev)

    def step_layers(i):
        cache.attend_layers(seq, 0, ql, k_cur=kl, v_cur=kl, out=attl, workspace=wsl)
        cache.append_layers(seq, 0, knl, knl)
    decl_us = _timed(stream, step_layers, 5)
    out["qwen2.5-3b_paged_cache"] = {"prefill_tokens": T, "prefill_quantize_us": round(prefill_us, 1),
                                     "decode_step_us": round(decl_us, 1), "decode_calls": 2,
                                     "decode_step_per_layer_calls_us": round(dec_us, 1), "layers": L,
                                     "page_tokens": 256}
    cache.close(seq)
    del cache, kvl, ws, att, wsl, attl

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
            "decode_attention_frac_hbm": round(2 * n_k * c.layout["record_bytes"] / (aus * 1e-6) / 8e12, 4),
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
    if a.summarize:
        summarize(a.summarize)
        return
    if a.trace_summary:
        with open(a.trace_summary[1], "w") as f:
            if a.trace_command:
                f.write(f"# {a.trace_title or 'rocprofv3 kernel trace'}, by kernel and grid size\n\n"
                        f"Command (MI355X):\n\n{a.trace_command}\n\n")
            f.write(trace_summary(a.trace_summary[0]))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the codec library runs on a single MI355X and has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline runs first, in spawned workers, before the GPU is used
    cpu = None if (a.no_cpu or a.profile_set) else cpu_baseline()

    import numpy as np
    import torch
    import kv_cache_vector_norm_amd as K
    from kv_cache_vector_norm_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.profile_set:
        profile_set(K, W, dev)
        return
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

    def roundtrip(i):
        k = i % nsets
        codec.roundtrip(xs[k], rec=recs[k], out=ys[k])

    def score(i):
        k = i % nsets
        codec.score(q, recs[k], N_Q, N_VEC, out=scs[k])

    for i in range(a.warmup):
        roundtrip(i)
        score(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        roundtrip(i)
        score(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / a.steps

    # per-kernel times: back-to-back launches over the rotating sets
    rt_us, rt_min = _b2b(stream, roundtrip, nsets, a.trials)
    sc_us, sc_min = _b2b(stream, score, nsets, a.trials)
    # the reference copy of the same bytes (568 B per vector: read 284, write 284)
    cbytes = N_VEC * algorithmic_bytes(lay) // 2
    csrc = torch.empty((nsets, cbytes), dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cp_us, _ = _b2b(stream, lambda i: K.rq_bench_copy(csrc[i % nsets], cdst[i % nsets], cbytes, stream), nsets,
                    a.trials)
    del csrc, cdst

    bytes_vec = algorithmic_bytes(lay)
    rt_gbs = N_VEC * bytes_vec / (rt_us * 1e-6) / 1e9
    cp_gbs = 2 * cbytes / (cp_us * 1e-6) / 1e9
    digest = kernel_code_digest(ROUNDTRIP_SYMBOL)
    traffic = measured_traffic("rq_roundtrip_qjl3_65536", digest)
    roof = {"bound": "hbm", "achieved": round(rt_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(rt_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "rq_roundtrip (2-bit codes + QJL, fp16 in/out): rqk::" + ROUNDTRIP_KERNEL,
            "algorithmic_bytes_per_vector": bytes_vec, "vectors_per_launch": N_VEC,
            "avg_launch_us": round(rt_us, 2), "min_trial_us": round(rt_min, 2),
            "timing": f"median over {a.trials} trials of {nsets} back-to-back launches over {nsets} rotating "
                      f"buffer sets, HIP events on the launch stream",
            "copy_same_bytes_gbs": round(cp_gbs, 1), "frac_of_copy": round(rt_gbs / cp_gbs, 4)}
    score_bytes = N_VEC * lay["record_bytes"] + 4 * N_Q * N_VEC
    extras = {
        "scores_per_s": round(N_Q * N_VEC * a.steps / elapsed, 1),
        "roundtrip_vectors_per_s": round(N_VEC / (rt_us * 1e-6), 1),
        "score_us": round(sc_us, 2),
        "score_scores_per_s": round(N_Q * N_VEC / (sc_us * 1e-6), 1),
        "score_gbs": round(score_bytes / (sc_us * 1e-6) / 1e9, 1),
        "score_frac_hbm": round(score_bytes / (sc_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_within_step": bool(rt_us + sc_us <= ms_per_step * 1e3 * 1.02),
        "buffer_sets": nsets,
    }
    extras["c0_quality"] = quality_row(K, W, dev, stream)

    # MSE-only 3-bit roundtrip (the HBM-bandwidth codec) on the same keys
    mse = K.Codec(bits=3, seed=0, mode=K.RQ_MSE)
    mrec = [mse.alloc_record(N_VEC, dev) for _ in range(nsets)]
    mse_us, _ = _b2b(stream, lambda i: mse.roundtrip(xs[i % nsets], rec=mrec[i % nsets], out=ys[i % nsets]), nsets,
                     a.trials)
    mb = algorithmic_bytes(mse.layout)
    extras["mse3_roundtrip_us"] = round(mse_us, 2)
    extras["mse3_roundtrip_gbs"] = round(N_VEC * mb / (mse_us * 1e-6) / 1e9, 1)
    extras["mse3_roundtrip_vectors_per_s"] = round(N_VEC / (mse_us * 1e-6), 1)
    del mrec

    # QJL-only keys (1 bit in total) on the same keys: roundtrip and scoring
    q1 = K.Codec(bits=1, seed=0, mode=K.RQ_QJL)
    q1rec = [q1.alloc_record(N_VEC, dev) for _ in range(nsets)]
    us1 = _timed(stream, lambda i: q1.roundtrip(xs[i % nsets], rec=q1rec[i % nsets], out=ys[i % nsets]), 4 * nsets)
    sus1 = _timed(stream, lambda i: q1.score(q, q1rec[i % nsets], N_Q, N_VEC, out=scs[i % nsets]), 4 * nsets)
    extras["qjl1_roundtrip_us"] = round(us1, 2)
    extras["qjl1_roundtrip_gbs"] = round(N_VEC * algorithmic_bytes(q1.layout) / (us1 * 1e-6) / 1e9, 1)
    extras["qjl1_score_us"] = round(sus1, 2)
    del q1rec, q1

    # PolarQuant (16-word records, 496 bits of content) on the same keys:
    # fused roundtrip, and the 64 queries scored against all keys
    pc = K.PolarCodec(seed=0)
    pw = [pc.alloc_words(N_VEC, dev) for _ in range(nsets)]
    pus = _timed(stream, lambda i: pc.roundtrip(xs[i % nsets], words=pw[i % nsets], out=ys[i % nsets]), 4 * nsets)
    psus = _timed(stream, lambda i: pc.score(q, pw[i % nsets], N_Q, N_VEC, out=scs[i % nsets]), 4 * nsets)
    extras["polar_roundtrip_us"] = round(pus, 2)
    extras["polar_roundtrip_gbs"] = round(N_VEC * (256 + 64 + 256) / (pus * 1e-6) / 1e9, 1)
    extras["polar_roundtrip_vectors_per_s"] = round(N_VEC / (pus * 1e-6), 1)
    extras["polar_score_us"] = round(psus, 2)
    extras["polar_scores_per_s"] = round(N_VEC * N_Q / (psus * 1e-6), 1)
    del pw, pc
    del xs, ys, recs, scs
    torch.cuda.empty_cache()

    if not a.no_sweep:
        extras["sweeps"] = sweeps(K, dev, stream, {"mse3": mse, "qjl3": codec, "polar": K.PolarCodec(seed=0)})

    # the runtime's own device copy of 1 GiB, for comparison with rq_bench_copy
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cus = _timed(stream, lambda i: dst.copy_(src), 5)
    extras["runtime_copy_1gib_gbs"] = round(2 * (1 << 30) / (cus * 1e-6) / 1e9, 1)
    del src, dst

    if not a.no_workloads:
        extras["workloads"] = workload_extras(K, W, dev, stream)

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
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
