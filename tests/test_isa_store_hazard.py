"""The built kernels never rewrite the data registers of a pending 128-bit
(or 96-bit) vector-memory store within two wait states.

A buffer/global store of more than 64 bits reads its data registers after
it has issued; a VALU write to them in the next cycle can replace what gets
stored.  The compiler does not keep them apart on gfx950, so the kernels
close each group of wide stores with a scheduling barrier and an s_nop.
This test disassembles the gfx950 code objects inside librq.so (code built
here from this repository's sources) and checks every wide store.
"""
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_vector_norm_amd", "librq.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
WAIT_STATES = 2

WIDE_STORE = re.compile(r"^(buffer|global|flat)_store_(dwordx3|dwordx4|b96|b128)\b")
VREG = re.compile(r"^v(\d+)$|^v\[(\d+):(\d+)\]$")


def _regs(tok):
    m = VREG.match(tok.strip().rstrip(","))
    if not m:
        return range(0)
    if m.group(1) is not None:
        return range(int(m.group(1)), int(m.group(1)) + 1)
    return range(int(m.group(2)), int(m.group(3)) + 1)


def _code_objects(fatbin):
    """gfx950 ELF images of every offload bundle in a .hip_fatbin section."""
    out = []
    start = fatbin.find(MAGIC)
    while start >= 0:
        n = struct.unpack_from("<Q", fatbin, start + len(MAGIC))[0]
        off = start + len(MAGIC) + 8
        for _ in range(n):
            o, size, tl = struct.unpack_from("<QQQ", fatbin, off)
            off += 24
            triple = fatbin[off:off + tl].decode()
            off += tl
            if "gfx950" in triple and size:
                out.append(fatbin[start + o:start + o + size])
        start = fatbin.find(MAGIC, start + 1)
    return out


def scan(lines):
    """(wide stores seen, [(store, offending instruction)])."""
    insts = []
    for ln in lines:
        s = ln.split("//")[0].strip()
        if not s or s.endswith(":") or s.startswith(";") or s.startswith("."):
            continue
        insts.append(s)
    stores, hits = 0, []
    for i, s in enumerate(insts):
        op = s.split()[0]
        if not WIDE_STORE.match(op):
            continue
        stores += 1
        ops = s[len(op):].split(",")
        data = ops[0] if op.startswith("buffer") else (ops[1] if len(ops) > 1 else "")
        held = set(_regs(data))
        ws, j = 0, i + 1
        while ws < WAIT_STATES and j < len(insts):
            t = insts[j]
            j += 1
            top = t.split()[0]
            if top == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            if top.startswith("v_") and len(t.split()) > 1 and held & set(_regs(t.split()[1])):
                hits.append((s, t))
            ws += 1
    return stores, hits


def test_scan_finds_a_planted_hazard():
    code = ["buffer_store_dwordx4 v[10:13], v0, s[60:63], s97 offen nt",
            "v_bitop3_b32 v10, v9, 15, v67 bitop3:0x48",
            "buffer_store_dwordx4 v[20:23], v0, s[60:63], s98 offen nt",
            "s_nop 1",
            "v_mov_b32_e32 v20, 0"]
    stores, hits = scan(code)
    assert stores == 2 and len(hits) == 1 and hits[0][1].startswith("v_bitop3_b32 v10")


@pytest.mark.skipif(not os.path.exists(LIB), reason="librq.so is not built")
@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "llvm-objdump")), reason="no llvm-objdump")
def test_no_wide_store_data_hazard(tmp_path):
    fb = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fb}", LIB,
                    str(tmp_path / "copy.so")], check=True, capture_output=True)
    objs = _code_objects(fb.read_bytes())
    assert objs, "no gfx950 code object in librq.so"
    total, bad = 0, []
    for k, co in enumerate(objs):
        path = tmp_path / f"k{k}.co"
        path.write_bytes(co)
        dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", str(path)], check=True,
                             capture_output=True, text=True).stdout
        stores, hits = scan(dis.splitlines())
        total += stores
        bad += hits
    assert total > 100, f"only {total} wide stores found: the scan is not seeing the kernels"
    assert not bad, f"{len(bad)} wide stores with their data rewritten within {WAIT_STATES} wait states: {bad[:3]}"
