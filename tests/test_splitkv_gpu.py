"""Split-KV forward on the GPU (through the C-ABI) against the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_fwd, fa_fwd_splitkv, fa_fwd_splitkv_workspace_size

from .oracle_pins import parse_exact
from .parity import check_fwd, errs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(B, Hq, Hkv, Nq, Nkv, d, dtype, causal, splits, seed):
    q, k, v = workloads.make_decode_inputs(B, Hq, Hkv, Nq, Nkv, d, dtype, seed)
    o, lse = fa_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), causal, 1.0 / math.sqrt(d), splits)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward_kv(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                       1.0 / math.sqrt(d), causal)
    return o, lse, O, L


CASES = [
    # B, Hq, Hkv, Nq, Nkv, d, splits
    (1, 4, 1, 1, 1000, 128, 0),       # one new token, G = 4 stacked rows
    (2, 8, 2, 3, 777, 64, 5),         # ragged key chunks
    (1, 2, 2, 17, 300, 128, 1),       # one chunk
    (1, 2, 2, 17, 300, 128, 7),
    (1, 2, 2, 17, 300, 128, 64),      # more chunks than key tiles: empty chunks
    (1, 32, 8, 8, 4096, 128, 0),      # 32 stacked rows fill one tile
    (1, 8, 2, 40, 513, 64, 3),        # 160 stacked rows: five row blocks
    (1, 1, 1, 64, 64, 128, 2),        # N_q == N_kv
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_sweep(dtype, causal):
    for i, (B, Hq, Hkv, Nq, Nkv, d, splits) in enumerate(CASES):
        print(f"case dtype={dtype} causal={causal} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} "
              f"splits={splits}", flush=True)
        o, lse, O, L = _run(B, Hq, Hkv, Nq, Nkv, d, dtype, causal, splits, 300 + i)
        check_fwd(o, lse, O, L, dtype, f"case {i}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_hand_examples(dtype):
    """The N_q != N_kv hand-worked cases, zero-padded to d = 64."""
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "hand_examples.json")) as f:
        cases = json.load(f)["kv_cases"]
    tdt = workloads.DTYPES[dtype]
    for c in cases:
        Q, K, V = (np.asarray(c[x], dtype=np.float64) for x in ("Q", "K", "V"))

        def pad(x):
            y = np.zeros((1, 1, x.shape[0], 64))
            y[0, 0, :, :x.shape[1]] = x
            return torch.tensor(y, dtype=tdt, device=DEV)

        for splits in (1, 2):
            o, lse = fa_fwd_splitkv(pad(Q), pad(K), pad(V), c["causal"], parse_exact(c["scale"]), splits)
            torch.cuda.synchronize()
            expO = np.vectorize(parse_exact)(np.asarray(c["O"], dtype=object)).astype(np.float64)
            explse = np.array([parse_exact(x) for x in c["lse"]])
            got = o.double().cpu().numpy()[0, 0, :, :expO.shape[1]]
            assert np.abs(got - expO).max() <= 2e-2, (c["name"], splits, got, expO)
            assert np.abs(lse.double().cpu().numpy()[0, 0] - explse).max() <= 1e-3, (c["name"], splits)


def test_equal_lengths_match_the_forward_kernel():
    """With N_q == N_kv the split path and fa_fwd compute the same attention."""
    q, k, v = workloads.make_decode_inputs(2, 4, 2, 300, 300, 128, "bf16", 41)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o1, l1 = fa_fwd(q, k, v, causal, 0.088)
        o2, l2 = fa_fwd_splitkv(q, k, v, causal, 0.088, 4)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
        assert (l1 - l2).abs().max().item() <= 1e-4


def test_partials_in_the_workspace():
    """Each chunk's partial output and logsumexp against the oracle on that chunk."""
    B, Hq, Hkv, Nq, Nkv, d, splits = 1, 4, 2, 5, 700, 128, 3
    q, k, v = workloads.make_decode_inputs(B, Hq, Hkv, Nq, Nkv, d, "bf16", 77)
    ws = torch.empty(fa_fwd_splitkv_workspace_size(B, Hq, Nq, d, splits), dtype=torch.uint8, device=DEV)
    fa_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), False, 0.1, splits, workspace=ws)
    torch.cuda.synchronize()
    rows = B * Hq * Nq
    part_bytes = (splits * rows * d * 4 + 255) // 256 * 256
    Op = ws[:splits * rows * d * 4].view(torch.float32).view(splits, B, Hq, Nq, d).double().cpu().numpy()
    Lp = ws[part_bytes:part_bytes + splits * rows * 4].view(torch.float32).view(splits, B, Hq, Nq)
    Lp = Lp.double().cpu().numpy()
    tile = 32  # keys per tile of the split kernel at d = 128
    chunk = ((Nkv + splits - 1) // splits + tile - 1) // tile * tile
    f = workloads.to_f64
    for s in range(splits):
        a, b = s * chunk, min(Nkv, (s + 1) * chunk)
        O, L = oracle.attention_forward_kv(f(q), f(k)[:, :, a:b], f(v)[:, :, a:b], 0.1, False)
        assert np.abs(Op[s] - O).max() <= 1e-2, s
        assert np.abs(Lp[s] - L).max() <= 1e-3, s


def test_full_size_decode_sampled():
    """The long-context GQA decode shape (one token, 64k keys) on every row."""
    w = workloads.DECODE_WORKLOADS["genome_gqa_64k_decode"]
    q, k, v = workloads.make_decode_inputs(w.B, w.H_q, w.H_kv, w.N_q, w.N_kv, w.d, w.dtype, w.seed)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = fa_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), w.causal, scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward_kv(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                       scale, w.causal)
    check_fwd(o, lse, O, L, w.dtype, w.name)


def test_deterministic_and_writes_only_outputs():
    B, Hq, Hkv, Nq, Nkv, d = 1, 8, 2, 4, 2000, 64
    q, k, v = workloads.make_decode_inputs(B, Hq, Hkv, Nq, Nkv, d, "bf16", 5)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    guard = torch.full((q.numel() + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = guard[2048:2048 + q.numel()].view(q.shape)
    o1, l1 = fa_fwd_splitkv(q, k, v, True, 0.125, 6, o=o)
    o2, l2 = fa_fwd_splitkv(q, k, v, True, 0.125, 6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isnan(guard[:2048].float()).all() and torch.isnan(guard[2048 + q.numel():].float()).all()
