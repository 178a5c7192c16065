"""Block-sparse attention on the GPU (through the C-ABI) against the oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_bwd_blocksparse, fa_fwd, fa_fwd_blocksparse
from oracle import blocksparse as obs

from .parity import TOL, check_fwd, check_grads, errs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # B, Hq, Hkv, N, d, mask_heads, density
    (1, 2, 2, 300, 128, 1, 0.5),
    (1, 4, 2, 700, 128, 4, 0.3),     # per-head masks, GQA
    (2, 2, 2, 513, 64, 2, 0.5),
    (1, 2, 1, 1000, 128, 1, 1.0),    # dense mask
    (1, 1, 1, 100, 64, 1, 0.0),      # diagonal blocks only
]


def _run(B, Hq, Hkv, N, d, mh, density, dtype, causal, seed, diag=True):
    q, k, v, do = workloads.make_inputs(B, Hq, Hkv, N, d, dtype, seed, with_dout=True)
    M = workloads.make_block_mask(mh, N, density, seed + 1, diag)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod, Md = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), M.to(DEV)
    o, lse = fa_fwd_blocksparse(qd, kd, vd, Md, causal, scale)
    dq, dk, dv = fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, Md, causal, scale)
    torch.cuda.synchronize()
    f = workloads.to_f64
    ref = obs.attention_backward_blocksparse(f(q), f(k), f(v), f(do), scale, causal, M.numpy())
    return (o, lse, dq, dk, dv), ref


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_parity(dtype, causal):
    for i, (B, Hq, Hkv, N, d, mh, dens) in enumerate(CASES):
        print(f"case dtype={dtype} causal={causal} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} heads={mh} "
              f"density={dens}", flush=True)
        (o, lse, dq, dk, dv), (O, L, dQ, dK, dV) = _run(B, Hq, Hkv, N, d, mh, dens, dtype, causal, 1100 + i)
        check_fwd(o, lse, O, L, dtype, f"case {i}")
        check_grads(dq, dk, dv, dQ, dK, dV, dtype, f"case {i}")


def test_empty_rows():
    """Rows whose visible blocks all lie above the diagonal see no key: o = 0,
    lse = -inf, no gradient; other rows as the oracle."""
    B, H, N, d = 1, 2, 512, 128
    M = torch.zeros((1, 4, 4), dtype=torch.uint8)
    M[0, 1, 3] = 1      # rows 128..255 see only keys 384..511: empty under the causal mask
    M[0, 2, 0] = 1
    M[0, 3, 2:] = 1
    q, k, v, do = workloads.make_inputs(B, H, H, N, d, "bf16", 1200, with_dout=True)
    qd, kd, vd, dod, Md = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), M.to(DEV)
    o, lse = fa_fwd_blocksparse(qd, kd, vd, Md, True, 0.088)
    dq, dk, dv = fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, Md, True, 0.088)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, :256] == 0) and torch.all(torch.isneginf(lse[:, :, :256]))
    assert torch.all(dq[:, :, :256] == 0)
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    f = workloads.to_f64
    O, L, dQ, dK, dV = obs.attention_backward_blocksparse(f(q), f(k), f(v), f(do), 0.088, True, M.numpy())
    fin = np.isfinite(L)
    assert np.abs(lse.double().cpu().numpy()[fin] - L[fin]).max() <= 1e-3
    assert errs(o, O)[0] <= TOL["bf16"]["o_max"]
    check_grads(dq, dk, dv, dQ, dK, dV, "bf16", "empty rows")


def test_all_blocks_equal_the_dense_forward():
    q, k, v, _ = workloads.make_inputs(2, 4, 2, 777, 128, "bf16", 1201)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    M = torch.ones((1, 7, 7), dtype=torch.uint8, device=DEV)
    for causal in (False, True):
        o0, l0 = fa_fwd(qd, kd, vd, causal, 0.09)
        o1, l1 = fa_fwd_blocksparse(qd, kd, vd, M, causal, 0.09)
        torch.cuda.synchronize()
        assert (o0.float() - o1.float()).abs().max().item() <= 1e-2
        assert (l0 - l1).abs().max().item() <= 1e-5


def test_long_context_band_mask():
    """8k tokens, causal, a local band of 4 blocks plus the first key block:
    every element against the oracle."""
    B, H, N, d = 1, 2, 8192, 128
    M = workloads.make_band_mask(N, 4, 1)
    q, k, v, do = workloads.make_inputs(B, H, H, N, d, "bf16", 1202, with_dout=True)
    qd, kd, vd, dod, Md = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), M.to(DEV)
    o, lse = fa_fwd_blocksparse(qd, kd, vd, Md, True, 1 / math.sqrt(d))
    dq, dk, dv = fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, Md, True, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    f = workloads.to_f64
    O, L, dQ, dK, dV = obs.attention_backward_blocksparse(f(q), f(k), f(v), f(do), 1 / math.sqrt(d), True,
                                                         M.numpy())
    check_fwd(o, lse, O, L, "bf16", "band")
    check_grads(dq, dk, dv, dQ, dK, dV, "bf16", "band")
