"""Backward pass on the GPU (through the C-ABI) against the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_bwd, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_prepare, fa_fwd

from .parity import TOL, check_grads, errs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
f64 = workloads.to_f64


def _run(q, k, v, do, causal, scale):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd(qd, kd, vd, causal, scale)
    dq, dk, dv = fa_bwd(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


SWEEP_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 257, 700]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_sweep(dtype, d, causal):
    """Ragged N on both the key-block and the query-block side, MHA, GQA, MQA."""
    for N in SWEEP_N:
        for (Hq, Hkv) in ((2, 2), (4, 1), (8, 2)):
            print(f"case dtype={dtype} d={d} causal={causal} N={N} Hq={Hq} Hkv={Hkv}", flush=True)
            q, k, v, do = workloads.make_inputs(1, Hq, Hkv, N, d, dtype, 500 + N + d, with_dout=True)
            scale = 1.0 / math.sqrt(d)
            dq, dk, dv = _run(q, k, v, do, causal, scale)
            dQ, dK, dV, _, _ = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), scale, causal)
            check_grads(dq, dk, dv, dQ, dK, dV, dtype, f"N={N} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("name", ["llama_mha_8k", "train_bwd_16k"])
def test_full_size_workloads(name):
    """Full-size backward in the default launch configuration; whole heads
    (first and last) against the oracle, all heads against the identities."""
    w = workloads.WORKLOADS[name]
    q, k, v, do = workloads.workload_inputs(w, with_dout=True)
    causal = True
    print(f"workload {name}", flush=True)
    dq, dk, dv = _run(q, k, v, do, causal, w.scale)
    for (b, h) in ((0, 0), (w.B - 1, w.H_q - 1)):
        print(f"  oracle head b={b} h={h}", flush=True)
        dQ, dK, dV, _, _ = oracle.attention_backward(
            f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]), f64(v[b:b + 1, h:h + 1]),
            f64(do[b:b + 1, h:h + 1]), w.scale, causal)
        res = check_grads(dq[b:b + 1, h:h + 1], dk[b:b + 1, h:h + 1], dv[b:b + 1, h:h + 1],
                          dQ, dK, dV, w.dtype, f"{name} b={b} h={h}")
        print(f"  errors {res}", flush=True)
    _identities(dk, dv, do, w.H_q // w.H_kv)


def _identities(dk, dv, do, G):
    """rowsum(dS) = 0: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (per K/V head)."""
    dk64 = dk.to(torch.float64)
    dv64 = dv.to(torch.float64)
    do64 = do.to(DEV).to(torch.float64)
    B, Hkv, N, d = dk.shape
    sk = dk64.sum(dim=2)
    assert (sk.abs() <= 1e-3 * dk64.abs().sum(dim=2) + 1e-3).all(), sk.abs().max().item()
    target = do64.view(B, Hkv, G, N, d).sum(dim=(2, 3))
    sv = dv64.sum(dim=2)
    assert ((sv - target).abs() <= 1e-3 * dv64.abs().sum(dim=2) + 1e-3).all(), (sv - target).abs().max().item()


def test_gqa_backward_moderate_size():
    """Grouped heads (G = 4) at N = 2048, d = 128: dK, dV sum four query heads."""
    q, k, v, do = workloads.make_inputs(2, 8, 2, 2048, 128, "bf16", 31, with_dout=True)
    for causal in (False, True):
        dq, dk, dv = _run(q, k, v, do, causal, 1 / math.sqrt(128))
        dQ, dK, dV, _, _ = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                                     1 / math.sqrt(128), causal)
        check_grads(dq, dk, dv, dQ, dK, dV, "bf16", f"gqa causal={causal}")
        _identities(dk, dv, do, 4)


def test_deterministic_and_fully_written():
    """Two runs agree bitwise; NaN-poisoned gradient buffers are fully written;
    canary bytes around them are untouched."""
    B, Hq, Hkv, N, d = 2, 4, 2, 333, 128
    q, k, v, do = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 78, with_dout=True)
    q, k, v, do = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    pad = 4096
    for causal in (False, True):
        o, lse = fa_fwd(q, k, v, causal, 0.09)
        bufs, views = [], []
        for like in (q, k, v):
            buf = torch.full((like.numel() + 2 * pad,), float("nan"), dtype=like.dtype, device=DEV)
            buf[:pad] = 5.0
            buf[-pad:] = 5.0
            bufs.append(buf)
            views.append(buf[pad:pad + like.numel()].view(like.shape))
        fa_bwd(q, k, v, o, lse, do, causal, 0.09, dq=views[0], dk=views[1], dv=views[2])
        dq2, dk2, dv2 = fa_bwd(q, k, v, o, lse, do, causal, 0.09)
        torch.cuda.synchronize()
        for vw, again in zip(views, (dq2, dk2, dv2)):
            assert torch.isfinite(vw).all()
            assert torch.equal(vw, again)
        for buf in bufs:
            assert (buf[:pad] == 5.0).all() and (buf[-pad:] == 5.0).all()


def test_workspace_too_small_is_rejected():
    from exact_attention_99_amd import FaError
    q, k, v, do = workloads.make_inputs(1, 2, 2, 64, 64, "bf16", 1, with_dout=True)
    q, k, v, do = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd(q, k, v, False, 0.125)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(FaError):
        fa_bwd(q, k, v, o, lse, do, False, 0.125, workspace=ws)


def test_phases_on_two_streams_match_fa_bwd():
    """prepare, then dK/dV and dQ on two streams concurrently: bitwise equal to fa_bwd."""
    q, k, v, do = workloads.make_inputs(2, 8, 2, 1500, 128, "bf16", 41, with_dout=True)
    q, k, v, do = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    for causal in (False, True):
        o, lse = fa_fwd(q, k, v, causal, 0.1)
        dq, dk, dv = fa_bwd(q, k, v, o, lse, do, causal, 0.1)
        delta = fa_bwd_prepare(o, do)
        ev = torch.cuda.Event()
        ev.record()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        s1.wait_event(ev)
        s2.wait_event(ev)
        with torch.cuda.stream(s1):
            dk2, dv2 = fa_bwd_dkdv(q, k, v, lse, do, delta, causal, 0.1, stream=s1)
        with torch.cuda.stream(s2):
            dq2 = fa_bwd_dq(q, k, v, lse, do, delta, causal, 0.1, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
