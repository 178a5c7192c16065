"""The variable-length oracle against facts outside itself (CPU only): the
plain oracle at full lengths, float64 SDPA with a key-padding mask, a
pure-Python brute force, padding invariance and finite differences."""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.varlen as vl_real


def check_full_lengths_are_plain_attention(mod):
    rng = np.random.default_rng(1)
    Q, K, V, dO = (rng.standard_normal((2, 2, 40, 8)) for _ in range(4))
    for causal in (False, True):
        O, L, dQ, dK, dV = mod.attention_backward_varlen(Q, K, V, dO, 0.3, causal, [40, 40])
        dQ0, dK0, dV0, O0, L0 = oracle.attention_backward(Q, K, V, dO, 0.3, causal)
        for a, b in ((O, O0), (L, L0), (dQ, dQ0), (dK, dK0), (dV, dV0)):
            assert np.allclose(a, b, atol=1e-13)


def check_sdpa_with_key_padding(mod):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, N, d = 3, 4, 2, 50, 16
    Q = rng.standard_normal((B, Hq, N, d))
    K, V = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    lens = [50, 17, 33]
    for causal in (False, True):
        O, L = mod.attention_forward_varlen(Q, K, V, 0.25, causal, lens)
        Kr = torch.tensor(np.repeat(K, Hq // Hkv, axis=1))
        Vr = torch.tensor(np.repeat(V, Hq // Hkv, axis=1))
        for b, n in enumerate(lens):
            allowed = np.zeros((N, N), dtype=bool)
            allowed[:, :n] = True
            if causal:
                allowed &= np.tril(np.ones((N, N), dtype=bool))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(Q[b:b + 1]), Kr[b:b + 1], Vr[b:b + 1], attn_mask=torch.tensor(allowed),
                scale=0.25).numpy()
            assert np.allclose(O[b, :, :n], ref[0, :, :n], atol=1e-12)
            assert np.all(O[b, :, n:] == 0) and np.all(np.isneginf(L[b, :, n:]))


def check_brute_force(mod):
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 1, 9, 3
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    lens = [6, 9]
    for causal in (False, True):
        O, L = mod.attention_forward_varlen(Q, K, V, 0.8, causal, lens)
        for b, n in enumerate(lens):
            for i in range(N):
                if i >= n:
                    assert np.all(O[b, 0, i] == 0) and L[b, 0, i] == -np.inf
                    continue
                js = [j for j in range(n) if not causal or j <= i]
                s = [0.8 * sum(Q[b, 0, i, c] * K[b, 0, j, c] for c in range(d)) for j in js]
                m = max(s)
                z = sum(math.exp(x - m) for x in s)
                ref = sum(math.exp(x - m) / z * V[b, 0, j] for x, j in zip(s, js))
                assert np.allclose(O[b, 0, i], ref, atol=1e-12)
                assert abs(L[b, 0, i] - (m + math.log(z))) < 1e-12


def check_padding_is_inert(mod):
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 2, 30, 4
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    lens = [11, 30]
    a = mod.attention_backward_varlen(Q, K, V, dO, 0.5, True, lens)
    Q2, K2, V2, dO2 = (x.copy() for x in (Q, K, V, dO))
    for X in (Q2, K2, V2, dO2):
        X[0, :, 11:] = rng.standard_normal((H, N - 11, d)) * 100
    b = mod.attention_backward_varlen(Q2, K2, V2, dO2, 0.5, True, lens)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    O, L, dQ, dK, dV = a
    assert np.all(dQ[0, :, 11:] == 0) and np.all(dK[0, :, 11:] == 0) and np.all(dV[0, :, 11:] == 0)


def check_finite_differences(mod):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N, d = 2, 2, 1, 10, 3
    Q = rng.standard_normal((B, Hq, N, d))
    K, V = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    dO = rng.standard_normal((B, Hq, N, d))
    lens = [7, 10]
    for causal in (False, True):
        _, _, dQ, dK, dV = mod.attention_backward_varlen(Q, K, V, dO, 0.6, causal, lens)

        def f(Q_, K_, V_):
            return float((mod.attention_forward_varlen(Q_, K_, V_, 0.6, causal, lens)[0] * dO).sum())

        eps = 1e-6
        for X, Gr in ((Q, dQ), (K, dK), (V, dV)):
            for idx in [(0, 0, 2, 1), (0, X.shape[1] - 1, 6, 2), (1, 0, 9, 0), (0, 0, 8, 1)]:
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += eps
                Xm[idx] -= eps
                num = (f(*[Xp if Y is X else Y for Y in (Q, K, V)]) -
                       f(*[Xm if Y is X else Y for Y in (Q, K, V)])) / (2 * eps)
                assert abs(num - Gr[idx]) < 1e-6 * max(1.0, abs(num)), (causal, idx, num, Gr[idx])


CHECKS = [check_full_lengths_are_plain_attention, check_sdpa_with_key_padding, check_brute_force,
          check_padding_is_inert, check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check(vl_real)


def test_rejects_bad_lengths():
    Z = np.zeros((2, 1, 4, 2))
    for lens in ([5, 1], [-1, 2], [1]):
        with pytest.raises(ValueError):
            vl_real.attention_forward_varlen(Z, Z, Z, 1.0, False, lens)


MUTATIONS = [
    ("length off by one", "Ob, lb = attention_forward(Q[b:b + 1, :, :n], K[b:b + 1, :, :n], V[b:b + 1, :, :n], scale, causal)",
     "Ob, lb = attention_forward(Q[b:b + 1, :, :n], K[b:b + 1, :, :n + 1], V[b:b + 1, :, :n + 1], scale, causal)"),
    ("padded lse zero", "lse = np.full((B, Hq, N), -np.inf)\n    for b in range(B):\n        n = int(L[b])\n        if n == 0:\n            continue\n        Ob",
     "lse = np.zeros((B, Hq, N))\n    for b in range(B):\n        n = int(L[b])\n        if n == 0:\n            continue\n        Ob"),
    ("keys of the whole row block", "sl = (slice(b, b + 1), slice(None), slice(0, n))",
     "sl = (slice(b, b + 1), slice(None), slice(0, N))"),
]


def _mutant(old, new):
    with open(vl_real.__file__) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.varlen_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<varlen mutant>", "exec"), mod.__dict__)
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
