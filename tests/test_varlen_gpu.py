"""Variable-length batches on the GPU (through the C-ABI) against the oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads
from exact_attention_99_amd import fa_bwd_varlen, fa_fwd, fa_fwd_varlen
from oracle import varlen as ovl

from .parity import TOL, check_grads, errs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # B, Hq, Hkv, N, d, lengths
    (3, 2, 2, 300, 128, [300, 1, 177]),
    (4, 4, 2, 520, 128, [0, 520, 257, 64]),     # an empty sequence, GQA
    (2, 2, 2, 513, 64, [500, 129]),
    (2, 1, 1, 64, 64, [33, 64]),
]


def _check(o, lse, dq, dk, dv, ref, lens, dtype, what):
    O, L, dQ, dK, dV = ref
    for b, n in enumerate(lens):
        assert torch.all(o[b, :, n:] == 0), what
        assert torch.all(torch.isneginf(lse[b, :, n:])), what
        assert torch.all(dq[b, :, n:] == 0) and torch.all(dk[b, :, n:] == 0) and torch.all(dv[b, :, n:] == 0), what
    omax, _ = errs(o, O)
    assert omax <= TOL[dtype]["o_max"], (what, omax)
    # mean error over the valid rows only (the exact zeros of the padding
    # would dilute it)
    g = o.double().cpu().numpy()
    valid = [np.abs(g[b, :, :n] - O[b, :, :n]).ravel() for b, n in enumerate(lens) if n > 0]
    omean = float(np.concatenate(valid).mean()) if valid else 0.0
    assert omean <= TOL[dtype]["o_mean"], (what, omean)
    fin = np.isfinite(L)
    assert np.abs(lse.double().cpu().numpy()[fin] - L[fin]).max(initial=0) <= TOL[dtype]["lse_max"], what
    check_grads(dq, dk, dv, dQ, dK, dV, dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_parity(dtype, causal):
    for i, (B, Hq, Hkv, N, d, lens) in enumerate(CASES):
        print(f"case dtype={dtype} causal={causal} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} lens={lens}", flush=True)
        q, k, v, do = workloads.make_inputs(B, Hq, Hkv, N, d, dtype, 1300 + i, with_dout=True)
        sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(d)
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        o, lse = fa_fwd_varlen(qd, kd, vd, sl, causal, scale)
        dq, dk, dv = fa_bwd_varlen(qd, kd, vd, o, lse, dod, sl, causal, scale)
        torch.cuda.synchronize()
        f = workloads.to_f64
        ref = ovl.attention_backward_varlen(f(q), f(k), f(v), f(do), scale, causal, lens)
        _check(o, lse, dq, dk, dv, ref, lens, dtype, f"case {i}")


def test_full_lengths_equal_the_dense_forward():
    q, k, v, _ = workloads.make_inputs(2, 4, 2, 777, 128, "bf16", 1310)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sl = torch.tensor([777, 777], dtype=torch.int32, device=DEV)
    for causal in (False, True):
        o0, l0 = fa_fwd(qd, kd, vd, causal, 0.09)
        o1, l1 = fa_fwd_varlen(qd, kd, vd, sl, causal, 0.09)
        torch.cuda.synchronize()
        assert (o0.float() - o1.float()).abs().max().item() <= 1e-2
        assert (l0 - l1).abs().max().item() <= 1e-5


def test_padding_values_do_not_matter():
    B, H, N, d = 2, 2, 400, 128
    q, k, v, do = workloads.make_inputs(B, H, H, N, d, "bf16", 1311, with_dout=True)
    lens = [150, 333]
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    outs = []
    for trial in range(2):
        if trial:
            for x in (q, k, v, do):
                x[0, :, 150:] = 1e3
                x[1, :, 333:] = -1e3
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        o, lse = fa_fwd_varlen(qd, kd, vd, sl, True, 0.088)
        g = fa_bwd_varlen(qd, kd, vd, o, lse, dod, sl, True, 0.088)
        torch.cuda.synchronize()
        outs.append([o, lse, *g])
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), *outs):
        same = (a == b) | (torch.isnan(a) & torch.isnan(b))
        bad = (~same).nonzero()
        assert bad.numel() == 0, (name, bad[:6].tolist(), a[tuple(bad[0])].item(), b[tuple(bad[0])].item(),
                                  int(torch.isnan(a).sum()), int(torch.isnan(b).sum()))


def test_long_sequences():
    """An 8k-token batch of four lengths (causal, d = 128) on every element."""
    B, H, N, d = 4, 2, 8192, 128
    lens = [8192, 5000, 3001, 100]
    q, k, v, do = workloads.make_inputs(B, H, H, N, d, "bf16", 1312, with_dout=True)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd_varlen(qd, kd, vd, sl, True, scale)
    dq, dk, dv = fa_bwd_varlen(qd, kd, vd, o, lse, dod, sl, True, scale)
    torch.cuda.synchronize()
    f = workloads.to_f64
    ref = ovl.attention_backward_varlen(f(q), f(k), f(v), f(do), scale, True, lens)
    _check(o, lse, dq, dk, dv, ref, lens, "bf16", "8k varlen")
