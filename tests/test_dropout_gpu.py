"""Fused dropout on the GPU (through the C-ABI) against the dropout oracle.

The keep mask is integer work, so it is checked exactly: with Q = 0 every
probability of a row is 1 / n, so O = V-weighted sums of Z / n and, with V
and dO identity matrices, O and dV show the mask element by element.  Values
are compared with the 16-bit tolerances of the other parity tests.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_bwd_dropout, fa_fwd, fa_fwd_dropout
from oracle import dropout as odrop

from .parity import check_fwd, check_grads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


CASES = [
    # B, Hq, Hkv, N, d, p
    (1, 2, 2, 64, 128, 0.1),
    (1, 2, 1, 300, 128, 0.25),    # GQA, ragged tail
    (2, 2, 2, 257, 64, 0.1),
    (1, 4, 2, 700, 128, 0.5),     # several row and key blocks
    (1, 1, 1, 33, 64, 0.3),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_parity(dtype, causal):
    for i, (B, Hq, Hkv, N, d, p) in enumerate(CASES):
        print(f"case dtype={dtype} causal={causal} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} p={p}", flush=True)
        q, k, v, do = workloads.make_inputs(B, Hq, Hkv, N, d, dtype, 900 + i, with_dout=True)
        scale = 1 / math.sqrt(d)
        seed, offset = 12345 + i, 7 * i
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        o, lse = fa_fwd_dropout(qd, kd, vd, causal, scale, p, seed, offset)
        dq, dk, dv = fa_bwd_dropout(qd, kd, vd, o, lse, dod, causal, scale, p, seed, offset)
        torch.cuda.synchronize()
        f = workloads.to_f64
        O, L, dQ, dK, dV = odrop.attention_backward_dropout(f(q), f(k), f(v), f(do), scale, causal, p,
                                                            seed, offset)
        check_fwd(o, lse, O, L, dtype, f"case {i}")
        check_grads(dq, dk, dv, dQ, dK, dV, dtype, f"case {i}")


def _mask_from_uniform_forward(N, d, p, seed, offset, causal):
    """O of Q = 0 (uniform probabilities) and V = identity: O_ij = Z_ij s / n_i."""
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((1, 1, N, d), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, 1, N, d), dtype=torch.bfloat16, device=DEV)
    v[0, 0, :, :N] = torch.eye(N, dtype=torch.bfloat16, device=DEV)
    o, _ = fa_fwd_dropout(q, k, v, causal, 0.1, p, seed, offset)
    torch.cuda.synchronize()
    return o[0, 0, :, :N].float().cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_mask_is_exact(causal):
    N, d = 128, 128
    for p, seed, offset in ((0.1, 1, 0), (0.5, 2 ** 63 + 5, 2 ** 40 + 3), (0.8, 99, 1)):
        got = _mask_from_uniform_forward(N, d, p, seed, offset, causal) != 0
        Z = odrop.keep_mask(1, 1, N, N, p, seed, offset)[0, 0]
        if causal:
            Z = Z & np.tril(np.ones((N, N), dtype=bool))
        assert np.array_equal(got, Z), (p, seed, offset, int((got != Z).sum()))


def test_backward_mask_is_exact():
    """dV = (P o Z s)^T dO with dO = identity reads Z^T through the key-major
    pass; dQ and dK of the same call are checked against the oracle."""
    N, d, p, seed, offset = 128, 128, 0.3, 4242, 17
    g = torch.Generator().manual_seed(5)
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    k = torch.randn((1, 1, N, d), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, N, d), generator=g).to(torch.bfloat16)
    do = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    do[0, 0, :, :N] = torch.eye(N)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    for causal in (False, True):
        o, lse = fa_fwd_dropout(qd, kd, vd, causal, 0.1, p, seed, offset)
        dq, dk, dv = fa_bwd_dropout(qd, kd, vd, o, lse, dod, causal, 0.1, p, seed, offset)
        torch.cuda.synchronize()
        Z = odrop.keep_mask(1, 1, N, N, p, seed, offset)[0, 0]
        if causal:
            Z = Z & np.tril(np.ones((N, N), dtype=bool))
        got = dv[0, 0, :, :N].float().cpu().numpy() != 0     # dV[j, i] = P~_ij
        assert np.array_equal(got, Z.T), int((got != Z.T).sum())
        f = workloads.to_f64
        O, L, dQ, dK, dV = odrop.attention_backward_dropout(f(q), f(k), f(v), f(do), 0.1, causal, p,
                                                            seed, offset)
        check_grads(dq, dk, dv, dQ, dK, dV, "bf16", f"causal={causal}")


def test_no_dropout_matches_the_plain_forward():
    """With p = 0 the dropout entry point computes the plain forward.  The two
    run different kernel generations (their running maxima, and so the
    rounding of the probabilities, differ), so they agree to the rounding of
    the 16-bit probabilities and outputs, not bit for bit."""
    for d in (128, 64):
        q, k, v, _ = workloads.make_inputs(2, 4, 2, 500, d, "bf16", 61)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        for causal in (False, True):
            o0, l0 = fa_fwd(qd, kd, vd, causal, 0.09)
            o1, l1 = fa_fwd_dropout(qd, kd, vd, causal, 0.09, 0.0, 3, 4)
            torch.cuda.synchronize()
            a, b = o0.float(), o1.float()
            assert ((a - b).abs() <= 2e-3 + 2.0 ** -6 * a.abs()).all(), float((a - b).abs().max())
            assert float((l0 - l1).abs().max()) <= 1e-5


def test_seed_and_offset_select_the_mask():
    q, k, v, _ = workloads.make_inputs(1, 2, 2, 256, 64, "bf16", 62)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a, la = fa_fwd_dropout(qd, kd, vd, True, 0.125, 0.2, 10, 0)
    b, lb = fa_fwd_dropout(qd, kd, vd, True, 0.125, 0.2, 10, 0)
    c, lc = fa_fwd_dropout(qd, kd, vd, True, 0.125, 0.2, 10, 1)
    e, le = fa_fwd_dropout(qd, kd, vd, True, 0.125, 0.2, 11, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert not torch.equal(a, c) and not torch.equal(a, e)
    assert torch.equal(la, lc) and torch.equal(la, le)     # statistics of the undropped scores


def test_long_sequence_sampled():
    """An 8k-token causal head pair at d = 128: the forward on every row, the
    backward on every element, against the oracle."""
    B, H, N, d, p = 1, 2, 8192, 128, 0.1
    q, k, v, do = workloads.make_inputs(B, H, H, N, d, "bf16", 63, with_dout=True)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd_dropout(qd, kd, vd, True, scale, p, 77, 1)
    dq, dk, dv = fa_bwd_dropout(qd, kd, vd, o, lse, dod, True, scale, p, 77, 1)
    torch.cuda.synchronize()
    f = workloads.to_f64
    O, L, dQ, dK, dV = odrop.attention_backward_dropout(f(q), f(k), f(v), f(do), scale, True, p, 77, 1)
    check_fwd(o, lse, O, L, "bf16", "8k")
    check_grads(dq, dk, dv, dQ, dK, dV, "bf16", "8k")


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_many_heads_persistent_grid(d, causal):
    """Enough key blocks (3 per head, 6 x 16 K/V heads) that the dK/dV pass runs
    on its persistent grid, each workgroup drawing the keep bytes of several
    key blocks and steps in turn (and, at d = 64 under the causal mask, the
    forward too); every element against the oracle."""
    B, Hq, Hkv, N, p = 6, 32, 16, 300, 0.2
    print(f"case d={d} causal={causal}", flush=True)
    q, k, v, do = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 950 + d + int(causal), with_dout=True)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa_fwd_dropout(qd, kd, vd, causal, scale, p, 2024, 3)
    dq, dk, dv = fa_bwd_dropout(qd, kd, vd, o, lse, dod, causal, scale, p, 2024, 3)
    torch.cuda.synchronize()
    f = workloads.to_f64
    O, L, dQ, dK, dV = odrop.attention_backward_dropout(f(q), f(k), f(v), f(do), scale, causal, p, 2024, 3)
    check_fwd(o, lse, O, L, "bf16", f"d={d} causal={causal}")
    check_grads(dq, dk, dv, dQ, dK, dV, "bf16", f"d={d} causal={causal}")
