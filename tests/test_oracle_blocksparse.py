"""The block-sparse oracle against facts outside itself (CPU only): the plain
oracle under all-ones masks, float64 SDPA with the element mask written out,
a pure-Python brute force, empty rows and finite differences."""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.blocksparse as bs_real


def _rand_mask(rng, Hm, nb, density=0.5):
    return (rng.random((Hm, nb, nb)) < density).astype(np.uint8)


def _brute(Q, K, V, scale, causal, M, blk):
    B, Hq, N, d = Q.shape
    G = Hq // K.shape[1]
    O = np.zeros((B, Hq, N, d))
    lse = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hm = 0 if M.shape[0] == 1 else h
            for i in range(N):
                js = [j for j in range(N) if M[hm, i // blk, j // blk] and (not causal or j <= i)]
                if not js:
                    continue
                s = [scale * sum(Q[b, h, i, c] * K[b, h // G, j, c] for c in range(d)) for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                lse[b, h, i] = m + math.log(z)
                for jj, j in enumerate(js):
                    O[b, h, i] += e[jj] / z * V[b, h // G, j]
    return O, lse


def check_all_ones_is_plain_attention(mod):
    rng = np.random.default_rng(1)
    Q, K, V = (rng.standard_normal((2, 2, 70, 8)) for _ in range(3))
    for causal in (False, True):
        M = np.ones((1, 3, 3), dtype=np.uint8)
        O, L = mod.attention_forward_blocksparse(Q, K, V, 0.3, causal, M, 32)
        O0, L0 = oracle.attention_forward(Q, K, V, 0.3, causal)
        assert np.allclose(O, O0, atol=1e-13) and np.allclose(L, L0, atol=1e-13)


def check_sdpa_with_element_mask(mod):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, N, d, blk = 1, 4, 2, 90, 16, 16
    Q = rng.standard_normal((B, Hq, N, d))
    K, V = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    M = _rand_mask(rng, Hq, 6, 0.6)
    M[:, np.arange(6), np.arange(6)] = 1     # diagonal blocks: no empty row under the causal mask
    for causal in (False, True):
        O, L = mod.attention_forward_blocksparse(Q, K, V, 0.25, causal, M, blk)
        idx = np.arange(N) // blk
        allowed = M[:, idx][:, :, idx] != 0
        if causal:
            allowed &= np.tril(np.ones((N, N), dtype=bool))
        Kr = np.repeat(K, Hq // Hkv, axis=1)
        Vr = np.repeat(V, Hq // Hkv, axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q), torch.tensor(Kr), torch.tensor(Vr), attn_mask=torch.tensor(allowed[None]),
            scale=0.25).numpy()
        assert np.allclose(O, ref, atol=1e-12)


def check_brute_force(mod):
    rng = np.random.default_rng(3)
    for causal in (False, True):
        for Hm in (1, 2):
            Q, K, V = (rng.standard_normal((1, 2, 13, 3)) for _ in range(3))
            M = _rand_mask(rng, Hm, 4, 0.5)
            O, L = mod.attention_forward_blocksparse(Q, K, V, 0.7, causal, M, 4)
            Ob, Lb = _brute(Q, K, V, 0.7, causal, M, 4)
            assert np.allclose(O, Ob, atol=1e-12)
            assert np.array_equal(np.isinf(L), np.isinf(Lb)) and np.allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)])


def check_empty_rows(mod):
    rng = np.random.default_rng(4)
    Q, K, V, dO = (rng.standard_normal((1, 1, 40, 4)) for _ in range(4))
    M = np.zeros((1, 5, 5), dtype=np.uint8)
    M[0, 1, 3] = 1           # rows 8..15 see keys 24..31 only: empty under the causal mask
    M[0, 2, 0] = 1
    O, L, dQ, dK, dV = mod.attention_backward_blocksparse(Q, K, V, dO, 0.5, True, M, 8)
    assert np.all(O[0, 0, 8:16] == 0) and np.all(np.isneginf(L[0, 0, 8:16]))
    assert np.all(O[0, 0, :8] == 0) and np.all(dQ[0, 0, :16] == 0)
    assert np.all(np.isfinite(L[0, 0, 16:24]))
    assert np.all(dK[0, 0, 8:] == 0) and np.all(dV[0, 0, 8:] == 0)   # keys nobody sees


def check_finite_differences(mod):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N, d, blk = 1, 2, 1, 20, 3, 5
    Q = rng.standard_normal((B, Hq, N, d))
    K, V = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    dO = rng.standard_normal((B, Hq, N, d))
    M = _rand_mask(rng, Hq, 4, 0.6)
    M[:, 0, 0] = 1
    for causal in (False, True):
        _, _, dQ, dK, dV = mod.attention_backward_blocksparse(Q, K, V, dO, 0.6, causal, M, blk)

        def f(Q_, K_, V_):
            return float((mod.attention_forward_blocksparse(Q_, K_, V_, 0.6, causal, M, blk)[0] * dO).sum())

        eps = 1e-6
        for X, Gr in ((Q, dQ), (K, dK), (V, dV)):
            for idx in [(0, 0, 2, 1), (0, X.shape[1] - 1, 17, 2), (0, 0, 11, 0), (0, X.shape[1] - 1, 6, 1)]:
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += eps
                Xm[idx] -= eps
                num = (f(*[Xp if Y is X else Y for Y in (Q, K, V)]) -
                       f(*[Xm if Y is X else Y for Y in (Q, K, V)])) / (2 * eps)
                assert abs(num - Gr[idx]) < 1e-6 * max(1.0, abs(num)), (causal, idx, num, Gr[idx])


CHECKS = [check_all_ones_is_plain_attention, check_sdpa_with_element_mask, check_brute_force,
          check_empty_rows, check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check(bs_real)


MUTATIONS = [
    ("block mask read transposed", "vis = M[:, idx][:, :, idx] != 0",
     "vis = M[:, idx][:, :, idx].transpose(0, 2, 1) != 0"),
    ("block index off by one row", "idx = np.arange(N) // blk", "idx = np.minimum((np.arange(N) + 1) // blk, M.shape[1] - 1)"),
    ("causal mask transposed", "np.tril(np.ones((N, N), dtype=bool))[None]", "np.triu(np.ones((N, N), dtype=bool))[None]"),
    ("masked entries kept in the row sum", "E = np.where(vis, np.exp(S - m), 0.0)", "E = np.exp(np.where(vis, S, 0.0) - m)"),
    ("per-head mask ignored", "return vis[0] if vis.shape[0] == 1 else vis[h]", "return vis[0]"),
    ("empty rows get a finite lse", "lse = np.where(empty[:, 0], -np.inf,", "lse = np.where(empty[:, 0], 0.0,"),
    ("D term dropped", "dS = P * (dP - D)", "dS = P * dP"),
]


def _mutant(old, new):
    with open(bs_real.__file__) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.blocksparse_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<blocksparse mutant>", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    for chk in CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _caught(_mutant(old, new)), f"no pin catches: {name}"


def test_unmutated_module_passes_every_check():
    assert not _caught(_mutant("", ""))
