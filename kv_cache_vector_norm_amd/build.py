"""Builds librq.so (the HIP library behind include/rq.h) in-tree for gfx950.

    python -m kv_cache_vector_norm_amd.build [--jobs N] [--verbose]

Every call compiles everything from scratch into _build/ at the repository
root and links kv_cache_vector_norm_amd/librq.so.  The host core is plain
C++ built with g++ (strict IEEE: no fast-math, no FP contraction, so the
parameter draws are the exact libm values); the kernels and the C ABI layer
are built with hipcc for gfx950 only.
"""
import argparse
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librq.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX_HOST", "g++")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing", "-ffp-contract=off",
    "-mcode-object-version=5",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def stamp_path():
    """File next to librq.so holding the source digest it was built from."""
    return LIB + ".srcdigest"


def source_digest():
    """sha256 over every file of csrc/ and include/ and this build script
    (names and contents, sorted): what librq.so is built from."""
    h = hashlib.sha256()
    paths = [os.path.abspath(__file__)]
    for d in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            p = os.path.join(d, name)
            if os.path.isfile(p):
                paths.append(p)
    for p in paths:
        h.update(os.path.relpath(p, ROOT).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:32]


def _units():
    units = [("rq_host.o", [CXX] + HOST_FLAGS + ["-c", os.path.join(CSRC, "rq_host.cpp")])]
    units.append(("rq_api.o", [HIPCC] + HIP_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, "rq_api.cpp")]))
    for f in ("rq_rotor_dispatch.hip", "rq_dense.hip", "rq_score.hip", "rq_attend.hip", "rq_qjl1.hip", "rq_cache.hip",
              "rq_polar.hip", "rq_copy.hip", "rq_outlier.hip"):
        units.append((f.replace(".hip", ".o"), [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, f)]))
    for kind in ("rotor", "dense"):
        for qjl in (0, 1):
            for b in (1, 2, 3, 4):
                name = f"rq_{kind}_b{b}_q{qjl}.o"
                units.append((name, [HIPCC] + HIP_FLAGS + [f"-DRQ_B={b}", f"-DRQ_QJL={'true' if qjl else 'false'}",
                                                           "-c", os.path.join(CSRC, f"rq_{kind}_inst.hip")]))
    return units


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(jobs=None, verbose=False):
    """Compile every unit and link librq.so; returns the library path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    units = _units()
    jobs = jobs or min(len(units), max(1, (os.cpu_count() or 4)))

    def compile_one(u):
        obj, cmd = u
        out = os.path.join(BUILD, obj)
        _run(cmd + ["-o", out], verbose)
        return out

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, units))
    tmp = LIB + ".tmp"
    # Link against the HIP runtime that PyTorch ships, so that a process using
    # torch for device memory and streams holds exactly one HIP runtime.
    hip_dir = hip_runtime_dir()
    _run(["g++", "-shared", "-fPIC", "-o", tmp] + objs +
         [f"-L{hip_dir}", "-l:libamdhip64.so", f"-Wl,-rpath,{hip_dir}", "-Wl,--no-undefined"], verbose)
    digest = source_digest()
    os.replace(tmp, LIB)
    with open(stamp_path(), "w") as f:
        f.write(digest + "\n")
    return LIB


def hip_runtime_dir():
    """Directory of the libamdhip64.so that torch loads (ROCm's as fallback)."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is not None and spec.submodule_search_locations:
        d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return "/opt/rocm/lib"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(a.jobs, a.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
