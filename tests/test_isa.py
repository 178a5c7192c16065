"""Checks of the compiler's gfx950 output for the kernels (CPU: hipcc cross-compiles).

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


@pytest.mark.skipif(not shutil.which(fabuild.HIPCC) and not os.path.exists(fabuild.HIPCC),
                    reason="hipcc is not installed")
def test_no_lds_read_waits_for_the_next_tiles_copies(tmp_path):
    srcs = fabuild.sources()
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        asms = list(ex.map(lambda s: _asm(s, str(tmp_path / (os.path.basename(s) + ".s"))), srcs))
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
