"""The fp64 oracle against facts that do not come from the oracle itself.

CPU only.  Also plants mistakes in copies of the oracle (source-level
mutations, executed on the CPU) and checks that every one of them is caught
by at least one pin.
"""
from __future__ import annotations

import math
import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as oracle_mod

from . import oracle_pins as pins


def _rng(seed=1234):
    return np.random.default_rng(seed)


def test_golden_hand_examples():
    pins.pin_golden(oracle.attention_forward, oracle.attention_backward)


def test_brute_force_tiny():
    pins.pin_brute_force(oracle.attention_forward, _rng(1))


def test_invariants():
    pins.pin_invariants(oracle.attention_forward, oracle.attention_probs, _rng(2))


def test_gqa_equals_repeated_heads():
    pins.pin_gqa(oracle.attention_forward, oracle.attention_backward, _rng(3))


def test_finite_differences():
    pins.pin_finite_differences(oracle.attention_forward, oracle.attention_backward, _rng(4))


def test_backward_identities():
    pins.pin_backward_identities(oracle.attention_backward, _rng(5))


def test_torch_float64_sdpa():
    pins.pin_torch_sdpa(oracle.attention_forward, oracle.attention_backward, _rng(6))


def test_row_subset():
    pins.pin_row_subset(oracle.attention_forward, _rng(7))


def test_chunking_does_not_change_result():
    rng = _rng(8)
    Q = rng.standard_normal((1, 2, 70, 4))
    K = rng.standard_normal((1, 2, 70, 4))
    V = rng.standard_normal((1, 2, 70, 4))
    dO = rng.standard_normal((1, 2, 70, 4))
    for causal in (False, True):
        a = oracle.attention_forward(Q, K, V, 0.5, causal, chunk=1024)
        b = oracle.attention_forward(Q, K, V, 0.5, causal, chunk=9)
        assert np.allclose(a[0], b[0], atol=1e-14) and np.allclose(a[1], b[1], atol=1e-14)
        ga = oracle.attention_backward(Q, K, V, dO, 0.5, causal, chunk=1024)
        gb = oracle.attention_backward(Q, K, V, dO, 0.5, causal, chunk=7)
        for x, y in zip(ga, gb):
            assert np.allclose(x, y, atol=1e-13)


def test_memory_wall_arithmetic():
    """The initnode page's N = 16,384 example: S has 268,435,456 entries, 536.8 MB at 2 bytes."""
    n = 16384
    assert n * n == 268_435_456
    assert abs(n * n * 2 / 1e6 - 536.8) < 0.1


def test_online_softmax_recurrence_reaches_the_definition():
    """The blockwise recurrence ("FlashAttention and the Kernel Era", The Mathematics,
    online-softmax equation; "FlashAttention 1, 2, and 3 Explained", section 2) with
    the reading P~ = exp(S - m_new) and a final division by l gives the oracle's O and
    lse.  This pins the reading of the recurrence the kernels implement."""
    rng = _rng(9)
    N, d, bc = 45, 6, 8
    Q = rng.standard_normal((N, d)); K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    s = 0.45
    for causal in (False, True):
        O_ref, l_ref = oracle.attention_forward(Q[None, None], K[None, None], V[None, None], s, causal)
        m = np.full(N, -np.inf); ell = np.zeros(N); acc = np.zeros((N, d))
        for j0 in range(0, N, bc):
            Sj = s * Q @ K[j0:j0 + bc].T
            if causal:
                Sj = np.where(np.arange(j0, min(N, j0 + bc))[None, :] <= np.arange(N)[:, None], Sj, -np.inf)
            m_new = np.maximum(m, Sj.max(axis=1))
            alpha = np.exp(np.where(np.isinf(m), -np.inf, m - m_new))
            Pt = np.exp(Sj - m_new[:, None])
            ell = alpha * ell + Pt.sum(axis=1)
            acc = alpha[:, None] * acc + Pt @ V[j0:j0 + bc]
            m = m_new
        assert np.allclose(acc / ell[:, None], O_ref[0, 0], atol=1e-13)
        assert np.allclose(m + np.log(ell), l_ref[0, 0], atol=1e-13)


def test_kv_golden_hand_examples():
    pins.pin_kv_golden(oracle.attention_forward_kv)


def test_kv_brute_force_tiny():
    pins.pin_kv_brute_force(oracle.attention_forward_kv, _rng(11))


def test_kv_suffix_of_square_attention():
    pins.pin_kv_suffix(oracle.attention_forward_kv, oracle.attention_forward, _rng(12))


def test_kv_torch_float64_sdpa_with_explicit_mask():
    pins.pin_kv_torch_sdpa(oracle.attention_forward_kv, _rng(13))


def test_kv_chunk_merge_identity():
    pins.pin_kv_merge(oracle.attention_forward_kv, _rng(14))


def test_kv_rejects_causal_with_more_queries_than_keys():
    with pytest.raises(ValueError):
        oracle.attention_forward_kv(np.zeros((1, 1, 3, 2)), np.zeros((1, 1, 2, 2)),
                                    np.zeros((1, 1, 2, 2)), 1.0, True)


# ------------------------------------------------------- planted mistakes --

MUTATIONS = [
    ("mask off by one", "cols[None, :] <= row_idx[:, None]", "cols[None, :] < row_idx[:, None]"),
    ("mask transposed", "cols[None, :] <= row_idx[:, None]", "cols[None, :] >= row_idx[:, None]"),
    ("scale dropped from scores", "S = scale * (q_rows @ Kh.T)", "S = (q_rows @ Kh.T)"),
    ("lse without the max", "(m + np.log(ell))[:, 0]", "(np.log(ell))[:, 0]"),
    ("wrong K/V head for a query head", "hk = h // G", "hk = h % G"),
    ("D term dropped from dS", "dS = P * (dP - D)", "dS = P * dP"),
    ("sign of D flipped", "dS = P * (dP - D)", "dS = P * (dP + D)"),
    ("D summed over the wrong axis", "D = (dor * Or).sum(axis=1, keepdims=True)",
     "D = (dor * Or).sum(axis=0, keepdims=True)"),
    ("scale dropped from dQ", "dQ[b, h, idx] = scale * (dS @ Kh)", "dQ[b, h, idx] = (dS @ Kh)"),
    ("scale dropped from dK", "dK[b, hk] += scale * (dS.T @ qr)", "dK[b, hk] += (dS.T @ qr)"),
    ("P not transposed in dV", "dV[b, hk] += P.T @ dor", "dV[b, hk] += P[:, :P.shape[0]] @ dor"),
    ("dP contracted over the wrong dimension order", "dP = dor @ Vh.T", "dP = dor @ Vh.T[::-1]"),
    ("queries aligned to the start of the keys", "shift = Nkv - Nq", "shift = 0"),
    ("query positions off by one", "pos = np.arange(Nq) + shift", "pos = np.arange(Nq) + shift - 1"),
    ("split-KV head mapping wrong", "            hk = h // G\n            Kh = np.asarray(K[b, hk], dtype=np.float64)\n            Vh = np.asarray(V[b, hk], dtype=np.float64)\n            qr = np.asarray(Q[b, h], dtype=np.float64)",
     "            hk = h % G\n            Kh = np.asarray(K[b, hk], dtype=np.float64)\n            Vh = np.asarray(V[b, hk], dtype=np.float64)\n            qr = np.asarray(Q[b, h], dtype=np.float64)"),
]


def _mutant(src_old: str, src_new: str) -> types.ModuleType:
    path = oracle_mod.__file__
    with open(path) as f:
        src = f.read()
    assert src_old in src, f"mutation anchor not found: {src_old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_old, src_new), "<oracle mutant>", "exec"), mod.__dict__)
    return mod


def _caught(mod) -> bool:
    checks = [
        lambda: pins.pin_golden(mod.attention_forward, mod.attention_backward),
        lambda: pins.pin_brute_force(mod.attention_forward, _rng(1)),
        lambda: pins.pin_invariants(mod.attention_forward, mod.attention_probs, _rng(2)),
        lambda: pins.pin_gqa(mod.attention_forward, mod.attention_backward, _rng(3)),
        lambda: pins.pin_finite_differences(mod.attention_forward, mod.attention_backward, _rng(4)),
        lambda: pins.pin_kv_golden(mod.attention_forward_kv),
        lambda: pins.pin_kv_brute_force(mod.attention_forward_kv, _rng(5)),
    ]
    for chk in checks:
        try:
            with np.errstate(all="ignore"):
                chk()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _caught(_mutant(old, new)), f"no pin catches: {name}"


def test_unmutated_oracle_passes_every_check():
    assert not _caught(_mutant("", ""))
