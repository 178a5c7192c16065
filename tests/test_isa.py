"""Checks of the compiler's gfx950 output for the kernels (CPU: hipcc cross-compiles).

Two properties: LDS reads do not wait for the next tile's copies (below), and
every kernel keeps the occupancy its tiling is built for (at the end).

Every tiled kernel issues buffer-to-LDS copies of its next tile while it reads the
current tile from the other LDS buffer.  When the compiler cannot tell those reads
from the copies' LDS writes, it puts a wait on the vector-memory counter right
before the read, so the read waits for the copy of the *next* tile and the copy
no longer overlaps the current one (dK/dV ran 6% slower that way).  The kernels
read each tile through restrict-qualified buffer pointers so that the compiler
can tell; this test keeps it that way for every kernel instantiation in the
library (all of them are reachable through the entry points).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_99_amd import build as fabuild

FUNC = re.compile(r"^(_Z\S+):\s*(?:;.*)?$", re.M)

# kernel families the entry points launch
CHECKED = ("fwd16v6_kernel", "fwd8_kernel", "fwd_split16_kernel",
           "dq16v3_kernel", "dkdv16v3_kernel")


def _asm(src: str, out: str) -> str:
    cmd = [fabuild.HIPCC, *fabuild.FLAGS, *fabuild.FILE_FLAGS.get(os.path.basename(src), []),
           "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _functions(asm: str):
    for m in FUNC.finditer(asm):
        end = asm.find(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end if end >= 0 else len(asm)]


def _instructions(body: str):
    for line in body.splitlines():
        t = line.strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            yield t


def lds_reads_after_vmem_waits(body: str):
    """LDS reads that directly follow a wait on the vector-memory counter."""
    found = []
    ins = list(_instructions(body))
    for i, t in enumerate(ins):
        if t.startswith("s_waitcnt") and "vmcnt(" in t:
            nxt = next((u for u in ins[i + 1:i + 6] if not u.startswith("s_waitcnt")), "")
            if nxt.startswith("ds_read"):
                found.append((t, nxt))
    return found


def test_detector_flags_a_wait_before_an_lds_read():
    body = "\n".join(["\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds",
                      "\ts_waitcnt vmcnt(0)",
                      "\tds_read_b64_tr_b16 v[2:3], v4 offset:64"])
    assert len(lds_reads_after_vmem_waits(body)) == 1
    assert lds_reads_after_vmem_waits(body.replace("vmcnt(0)", "lgkmcnt(0)")) == []


needs_hipcc = pytest.mark.skipif(not shutil.which(fabuild.HIPCC) and not os.path.exists(fabuild.HIPCC),
                                 reason="hipcc is not installed")


@pytest.fixture(scope="module")
def asms(tmp_path_factory):
    """gfx950 assembly of every library source, compiled once for this module."""
    d = tmp_path_factory.mktemp("isa")
    srcs = fabuild.sources()
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        return list(ex.map(lambda s: _asm(s, str(d / (os.path.basename(s) + ".s"))), srcs))


@needs_hipcc
def test_no_lds_read_waits_for_the_next_tiles_copies(asms):
    checked, bad = 0, []
    for asm in asms:
        for name, body in _functions(asm):
            if not any(k in name for k in CHECKED) or "offen lds" not in body:
                continue
            checked += 1
            hits = lds_reads_after_vmem_waits(body)
            if hits:
                bad.append((name, hits[:2]))
    assert checked >= 80, f"only {checked} checked kernels with buffer-to-LDS copies found"
    assert not bad, bad


# ----------------------------------------------------------------- occupancy

KDESC = re.compile(r"^\s*\.amdhsa_kernel (\S+)$(.*?)^\s*\.end_amdhsa_kernel", re.M | re.S)
LDS_BYTES = 160 * 1024      # per compute unit
REGS = 512                  # vector + accumulation registers per SIMD lane


def kernel_resources(asm: str):
    """(mangled name, registers, LDS bytes, scratch bytes) of every kernel."""
    for m in KDESC.finditer(asm):
        body = m.group(2)
        get = lambda k: int(re.search(r"\.amdhsa_" + k + r" (\d+)", body).group(1))
        yield m.group(1), get("next_free_vgpr"), get("group_segment_fixed_size"), \
            get("private_segment_fixed_size")


def waves_per_simd(regs: int) -> int:
    return REGS // (-(-regs // 8) * 8)


FWD = re.compile(r"fwd16v6_kernelINS_4(?:BF16|FP16)ELi(\d+)ELb(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELb(\d)ELi(\d+)E")
DQ = re.compile(r"dq16v3_kernelINS_4(?:BF16|FP16)ELi(\d+)ELb(\d)ELi(\d+)ELb(\d)ELb(\d)E")


def test_occupancy_rule():
    assert waves_per_simd(168) == 3 and waves_per_simd(169) == 2 and waves_per_simd(256) == 2


@needs_hipcc
def test_kernels_keep_the_occupancy_they_are_tiled_for(asms):
    """Each kernel's tiling assumes a number of waves per SIMD and of
    workgroups per compute unit; more registers or LDS than that allows would
    silently cost a wave (at d = 64 the forward once lost its third wave per
    SIMD this way).  Scratch (spilled registers) is checked too: the causal
    dense paths have none; the known exceptions are the dQ pass without the
    causal mask (masked-tile loop only) and with dropout at d = 128."""
    res = [r for asm in asms for r in kernel_resources(asm)]
    seen = set()
    for name, regs, lds, scratch in res:
        m = FWD.search(name)
        if m:
            d, _causal, nw, _bc, _pers, drop, _sparse, _gs = (int(x) for x in m.groups())
            seen.add("fwd")
            assert scratch == 0, (name, scratch)
            if d == 128:   # 2 waves per SIMD, NW / 4 waves per SIMD per workgroup
                assert waves_per_simd(regs) >= 2, (name, regs)
                assert (8 // nw) * lds <= LDS_BYTES, (name, lds)
            elif not drop:  # d = 64: 3 waves per SIMD (3 four-wave workgroups)
                assert waves_per_simd(regs) >= 3, (name, regs)
                assert 3 * lds <= LDS_BYTES, (name, lds)
            continue
        m = DQ.search(name)
        if m:
            d, causal, nw, drop, _sparse = (int(x) for x in m.groups())
            seen.add("dq")
            assert waves_per_simd(regs) >= 2, (name, regs)
            assert (8 // nw) * lds <= LDS_BYTES, (name, lds)
            if causal and not drop:
                assert scratch == 0, (name, scratch)
            continue
        if "fwd8_kernel" in name:   # three four-wave workgroups per compute unit
            seen.add("fwd8")
            assert waves_per_simd(regs) >= 3 and 3 * lds <= LDS_BYTES and scratch == 0, (name, regs, lds, scratch)
        elif "dkdv16v3_kernel" in name:   # one workgroup per compute unit
            seen.add("dkdv")
            assert lds <= LDS_BYTES and scratch == 0, (name, lds, scratch)
        elif any(k in name for k in ("quant8_kernel", "fwd_split16_kernel", "merge_split_kernel")):
            seen.add(name.split("_kernel")[0][-10:])
            assert scratch == 0 and lds <= LDS_BYTES, (name, lds, scratch)
    assert {"fwd", "dq", "fwd8", "dkdv"} <= seen, seen
