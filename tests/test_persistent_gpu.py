"""Many short heads: the row and key blocks outnumber the compute units, so the
forward and the dK/dV pass run on their persistent grids (each workgroup walks
several blocks, and under grouped K/V heads the dK/dV pass walks the query
heads of a group per step), with a ragged sequence end in every head.

B = 16, H_q = 32, H_kv = 8 (G = 4), N = 700, d in {64, 128}, bf16 and fp16,
both masks.  Sampled heads (first, last and one whole K/V group) are compared
with the fp64 oracle; every head is checked through properties that hold at
any size: the Q = 0 closed form of the forward, and the backward identities
sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i over each K/V group.
"""
from __future__ import annotations

import math

import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_bwd, fa_fwd

from .parity import TOL, check_fwd, check_grads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
f64 = workloads.to_f64

B, HQ, HKV, N = 16, 32, 8, 700
G = HQ // HKV
HEADS = ((0, 0), (7, 4), (7, 5), (7, 6), (7, 7), (B - 1, HQ - 1))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_short_heads_forward_and_backward(dtype, d, causal):
    print(f"case dtype={dtype} d={d} causal={causal}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = workloads.make_inputs(B, HQ, HKV, N, d, dtype, 4100 + d + (7 if causal else 0),
                                        with_dout=True)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd(qd, kd, vd, causal, scale)
    dq, dk, dv = fa_bwd(qd, kd, vd, o, lse, dod, causal, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()

    for (b, h) in HEADS:
        hk = h // G
        O, L = oracle.attention_forward(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, hk:hk + 1]),
                                        f64(v[b:b + 1, hk:hk + 1]), scale, causal)
        check_fwd(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], O, L, dtype, f"b={b} h={h}")

    # backward: one whole K/V group (its dK, dV sum the group's G query heads)
    for (b, hk) in ((0, 0), (7, 1), (B - 1, HKV - 1)):
        hs = slice(hk * G, (hk + 1) * G)
        dQ, dK, dV, _, _ = oracle.attention_backward(
            f64(q[b:b + 1, hs]), f64(k[b:b + 1, hk:hk + 1]), f64(v[b:b + 1, hk:hk + 1]),
            f64(do[b:b + 1, hs]), scale, causal)
        check_grads(dq[b:b + 1, hs], dk[b:b + 1, hk:hk + 1], dv[b:b + 1, hk:hk + 1], dQ, dK, dV,
                    dtype, f"b={b} kv head {hk}")

    # every K/V group: rowsum(dS) = 0 gives sum_j dK_j = 0 and
    # sum_j dV_j = sum over the group's query heads and rows of dO
    dk64, dv64 = dk.to(torch.float64), dv.to(torch.float64)
    sk = dk64.sum(dim=2)
    assert (sk.abs() <= 1e-3 * dk64.abs().sum(dim=2) + 1e-3).all(), sk.abs().max().item()
    target = dod.to(torch.float64).view(B, HKV, G, N, d).sum(dim=(2, 3))
    sv = dv64.sum(dim=2)
    err = (sv - target).abs()
    assert (err <= 1e-3 * dv64.abs().sum(dim=2) + 1e-3).all(), err.max().item()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_short_heads_closed_form(dtype, d, causal):
    """Q = 0 on every row of every head: causal row i is the mean of V[0..i]
    with lse ln(i + 1); without the mask every row is the mean of V, lse ln N."""
    _, k, v, _ = workloads.make_inputs(B, HQ, HKV, N, d, dtype, 4200 + d)
    q = torch.zeros((B, HQ, N, d), dtype=k.dtype, device=DEV)
    o, lse = fa_fwd(q, k.to(DEV), v.to(DEV), causal, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    vv = v.to(DEV).to(torch.float64)
    if causal:
        ref = torch.cumsum(vv, dim=2) / torch.arange(1, N + 1, device=DEV, dtype=torch.float64)[:, None]
        lref = torch.log(torch.arange(1, N + 1, device=DEV, dtype=torch.float64))
    else:
        ref = vv.mean(dim=2, keepdim=True).expand(-1, -1, N, -1)
        lref = torch.full((N,), math.log(N), device=DEV, dtype=torch.float64)
    ref = ref.repeat_interleave(G, dim=1)
    err = (o.to(torch.float64) - ref).abs()
    tol = TOL[dtype]
    assert err.max().item() <= tol["o_max"], err.max().item()
    assert err.mean().item() <= tol["o_mean"], err.mean().item()
    assert (lse.to(torch.float64) - lref).abs().max().item() <= tol["lse_max"]


@pytest.mark.parametrize("kind", ["varlen", "blockmask"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_short_heads_masked(kind, d, causal):
    """The masked path on the persistent grids: per-sequence lengths (one empty
    sequence, one full, the rest ragged) or a per-head block mask over the same
    many short heads; three whole K/V groups against the oracle."""
    from exact_attention_99_amd import fa_bwd_blocksparse, fa_bwd_varlen, fa_fwd_blocksparse, fa_fwd_varlen
    from oracle import blocksparse as obs
    from oracle import varlen as ovl

    from .test_varlen_gpu import _check

    print(f"case kind={kind} d={d} causal={causal}", flush=True)
    dtype = "bf16"
    scale = 1.0 / math.sqrt(d)
    seed = 4300 + d + (7 if causal else 0) + (1 if kind == "blockmask" else 0)
    q, k, v, do = workloads.make_inputs(B, HQ, HKV, N, d, dtype, seed, with_dout=True)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    if kind == "varlen":
        g = torch.Generator().manual_seed(seed + 1)
        lens = torch.randint(1, N + 1, (B,), generator=g)
        lens[0], lens[7] = 0, N
        sl = lens.to(torch.int32).to(DEV)
        o, lse = fa_fwd_varlen(qd, kd, vd, sl, causal, scale)
        dq, dk, dv = fa_bwd_varlen(qd, kd, vd, o, lse, dod, sl, causal, scale)
    else:
        M = workloads.make_block_mask(HQ, N, 0.4, seed + 1, True)
        Md = M.to(DEV)
        o, lse = fa_fwd_blocksparse(qd, kd, vd, Md, causal, scale)
        dq, dk, dv = fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, Md, causal, scale)
    torch.cuda.synchronize()
    for (b, hk) in ((0, 0), (7, 1), (B - 1, HKV - 1)):
        hs = slice(hk * G, (hk + 1) * G)
        args = (f64(q[b:b + 1, hs]), f64(k[b:b + 1, hk:hk + 1]), f64(v[b:b + 1, hk:hk + 1]),
                f64(do[b:b + 1, hs]), scale, causal)
        got = (o[b:b + 1, hs], lse[b:b + 1, hs], dq[b:b + 1, hs], dk[b:b + 1, hk:hk + 1],
               dv[b:b + 1, hk:hk + 1])
        what = f"b={b} kv head {hk}"
        if kind == "varlen":
            n = int(lens[b])
            _check(*got, ovl.attention_backward_varlen(*args, [n]), [n], dtype, what)
        else:
            ref = obs.attention_backward_blocksparse(*args, M[hs].numpy())
            check_fwd(*got[:2], *ref[:2], dtype, what)
            check_grads(*got[2:], *ref[2:], dtype, what)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hkv", [4, 16, 32])
def test_many_short_heads_other_groups(hkv, causal):
    """Groups of 8 query heads (two stacks of 4 heads per K/V head: heads 17
    and 31 below lie in the first and second stack of theirs), groups of 2
    (one stack of 2) and no grouping, on the persistent grid at d = 128:
    sampled heads against the oracle, every head through the Q = 0 closed
    form."""
    d = 128
    G2 = HQ // hkv
    print(f"case hkv={hkv} causal={causal}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, _ = workloads.make_inputs(B, HQ, hkv, N, d, "bf16", 4400 + hkv + (7 if causal else 0))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa_fwd(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (0, 1), (5, 17), (B - 1, HQ - 1)):
        hk = h // G2
        O, L = oracle.attention_forward(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, hk:hk + 1]),
                                        f64(v[b:b + 1, hk:hk + 1]), scale, causal)
        check_fwd(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], O, L, "bf16", f"b={b} h={h}")
    q0 = torch.zeros_like(qd)
    o, lse = fa_fwd(q0, kd, vd, causal, scale)
    torch.cuda.synchronize()
    vv = vd.to(torch.float64)
    if causal:
        ref = torch.cumsum(vv, dim=2) / torch.arange(1, N + 1, device=DEV, dtype=torch.float64)[:, None]
    else:
        ref = vv.mean(dim=2, keepdim=True).expand(-1, -1, N, -1)
    ref = ref.repeat_interleave(G2, dim=1)
    err = (o.to(torch.float64) - ref).abs()
    assert err.max().item() <= TOL["bf16"]["o_max"], err.max().item()
    assert err.mean().item() <= TOL["bf16"]["o_mean"], err.mean().item()


def test_shared_tail_repeats_and_streams():
    """The persistent forward hands the last rounds' blocks out through counters
    that each launch takes from a ring of slots and resets when it ends: 80
    launches in a row (more than the ring holds) and launches on two streams
    without waits between them all give bitwise the same output and lse."""
    d, causal = 128, True
    print("case repeats", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, _ = workloads.make_inputs(B, HQ, HKV, N, d, "bf16", 4500)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o0, l0 = fa_fwd(qd, kd, vd, causal, scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(f64(q[3:4, 9:10]), f64(k[3:4, 2:3]), f64(v[3:4, 2:3]), scale, causal)
    check_fwd(o0[3:4, 9:10], l0[3:4, 9:10], O, L, "bf16", "b=3 h=9")
    o, lse = torch.empty_like(o0), torch.empty_like(l0)
    for i in range(80):
        fa_fwd(qd, kd, vd, causal, scale, o=o, lse=lse)
        assert torch.equal(o, o0) and torch.equal(lse, l0), f"launch {i}"
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.empty_like(o0), torch.empty_like(l0)) for _ in range(8)]
    torch.cuda.synchronize()
    for i, (oi, li) in enumerate(outs):
        fa_fwd(qd, kd, vd, causal, scale, o=oi, lse=li, stream=streams[i % 2])
    torch.cuda.synchronize()
    for i, (oi, li) in enumerate(outs):
        assert torch.equal(oi, o0) and torch.equal(li, l0), f"stream launch {i}"
