"""Compile libfa355.so (HIP kernels + C-ABI) for gfx950, in-tree.

    python -m exact_attention_99_amd.build
    python -m exact_attention_99_amd.build --out /tmp/alt.so -DFA355_FWD_NW128=4

Always recompiles.  Each ``csrc/*.hip`` file is compiled to an object in
parallel, then the objects are linked into ``exact_attention_99_amd/libfa355.so``.
With ``--out`` and -D overrides of the tile parameters (fa_common.h) it builds
an alternative library elsewhere, for measurements only (select it with the
FA355_LIB environment variable); the package's own library keeps the defaults.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa355.so")
ARCH = os.environ.get("FA355_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]

# Per-file options.  The backward kernels keep their dK/dV (or dQ) accumulators
# in the accumulation registers and need S and dP in vector registers for the
# softmax: MFMAs in the vector-register form avoid a copy of every S/dP tile.
FILE_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, obj: str, extra) -> str:
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="fa355_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], list(extra)), zip(srcs, objs)))
        tmp_lib = out + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out = LIB
    if "--out" in args:
        i = args.index("--out")
        out = os.path.abspath(args[i + 1])
        del args[i:i + 2]
    build(verbose=True, extra=args, out=out)
