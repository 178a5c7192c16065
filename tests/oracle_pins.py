"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle breaks the
fact it checks.  ``test_oracle.py`` runs every pin against the oracle as it
stands, and also against deliberately broken copies of the oracle (planted on
the CPU) to show that a plausible mistake is caught by at least one pin.

Sources of truth used here (none of them is the oracle's own code):
  * hand-worked exact examples (``golden/hand_examples.json``);
  * closed forms: Q = 0 gives prefix means and lse_i = ln(i + 1);
  * invariants of softmax attention (row sums, shift and permutation
    invariance, causal row 0);
  * a pure-Python brute force of the definition on tiny inputs (no numpy);
  * central finite differences of L = sum(dO * O) for the backward pass;
  * PyTorch's float64 CPU ``scaled_dot_product_attention`` with autograd,
    the library routine the pages name ("Flash Attention" (21medien), Code
    Example).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------- golden --

def parse_exact(s) -> float:
    """'a/b', 'ln a', 'c*ln a', 'c/b*ln a', or a plain number."""
    if isinstance(s, (int, float)):
        return float(s)
    s = s.strip()
    if "ln" in s:
        coef, _, arg = s.partition("ln")
        coef = coef.strip().rstrip("*").strip()
        c = Fraction(coef) if coef else Fraction(1)
        return float(c) * math.log(float(Fraction(arg.strip())))
    return float(Fraction(s))


def load_golden():
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        return json.load(f)["cases"]


def _as4(x):
    a = np.asarray(x, dtype=np.float64)
    return a[None, None]


def pin_golden(fwd, bwd, atol=1e-12):
    for c in load_golden():
        scale = parse_exact(c["scale"])
        Q, K, V = _as4(c["Q"]), _as4(c["K"]), _as4(c["V"])
        O, lse = fwd(Q, K, V, scale, c["causal"])
        expO = np.vectorize(parse_exact)(np.asarray(c["O"], dtype=object)).astype(np.float64)
        explse = np.array([parse_exact(x) for x in c["lse"]])
        assert np.allclose(O[0, 0], expO, atol=atol, rtol=0), (c["name"], "O", O[0, 0], expO)
        assert np.allclose(lse[0, 0], explse, atol=atol, rtol=0), (c["name"], "lse", lse[0, 0], explse)
        if "dO" in c:
            dQ, dK, dV, _, _ = bwd(Q, K, V, _as4(c["dO"]), scale, c["causal"])
            for nm, got in (("dQ", dQ), ("dK", dK), ("dV", dV)):
                exp = np.vectorize(parse_exact)(np.asarray(c[nm], dtype=object)).astype(np.float64)
                assert np.allclose(got[0, 0], exp, atol=atol, rtol=0), (c["name"], nm, got[0, 0], exp)


# ------------------------------------------------------------- brute force --

def brute_force_attention(q, k, v, scale, causal):
    """Pure-Python evaluation of the definition for one head (lists of lists).

    Uses no numpy: every dot product, exponential and sum is written out.
    """
    n = len(q)
    d = len(q[0])
    dv = len(v[0])
    out, lse = [], []
    for i in range(n):
        scores = []
        for j in range(n):
            if causal and j > i:
                continue
            s = 0.0
            for t in range(d):
                s += q[i][t] * k[j][t]
            scores.append((j, scale * s))
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        row = [0.0] * dv
        for j, x in w:
            for t in range(dv):
                row[t] += x / tot * v[j][t]
        out.append(row)
        lse.append(mx + math.log(tot))
    return out, lse


def pin_brute_force(fwd, rng, atol=1e-12):
    for (N, d, Hq, Hkv, causal) in [(1, 1, 1, 1, False), (3, 2, 1, 1, True), (5, 3, 2, 1, False),
                                     (7, 4, 4, 2, True), (8, 4, 3, 3, True), (6, 2, 4, 1, False)]:
        Q = rng.standard_normal((1, Hq, N, d))
        K = rng.standard_normal((1, Hkv, N, d))
        V = rng.standard_normal((1, Hkv, N, d))
        scale = 0.7
        O, lse = fwd(Q, K, V, scale, causal)
        G = Hq // Hkv
        for h in range(Hq):
            bo, bl = brute_force_attention(Q[0, h].tolist(), K[0, h // G].tolist(),
                                           V[0, h // G].tolist(), scale, causal)
            assert np.allclose(O[0, h], np.array(bo), atol=atol, rtol=0), (N, d, h, causal)
            assert np.allclose(lse[0, h], np.array(bl), atol=atol, rtol=0), (N, d, h, causal)


# -------------------------------------------------------------- invariants --

def pin_invariants(fwd, probs, rng):
    N, d = 37, 8
    Q = rng.standard_normal((1, 1, N, d))
    K = rng.standard_normal((1, 1, N, d))
    V = rng.standard_normal((1, 1, N, d))
    s = 0.5
    # rows of P sum to one, and P is zero above the diagonal when causal
    for causal in (False, True):
        P = probs(Q[0, 0], K[0, 0], s, causal)
        assert np.allclose(P.sum(axis=1), 1.0, atol=1e-13)
        assert (P >= 0).all()
        if causal:
            assert np.all(np.triu(P, 1) == 0.0)
    # equal scores (Q = 0): O is the mean of the visible V rows, lse = ln(count)
    Z = np.zeros_like(Q)
    O, lse = fwd(Z, K, V, s, False)
    assert np.allclose(O[0, 0], V[0, 0].mean(axis=0)[None, :], atol=1e-13)
    assert np.allclose(lse[0, 0], math.log(N), atol=1e-13)
    O, lse = fwd(Z, K, V, s, True)
    prefix = np.cumsum(V[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert np.allclose(O[0, 0], prefix, atol=1e-13)
    assert np.allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-13)
    # causal row 0 sees only key 0: O_0 = V_0 and lse_0 = scale * q0 . k0
    O, lse = fwd(Q, K, V, s, True)
    assert np.allclose(O[0, 0, 0], V[0, 0, 0], atol=1e-14)
    assert math.isclose(lse[0, 0, 0], s * float(Q[0, 0, 0] @ K[0, 0, 0]), abs_tol=1e-13)
    # shift invariance: append a column kappa to every K row and delta_i to Q
    # row i; row i's scores all shift by s*delta_i*kappa, so O is unchanged
    # and lse_i shifts by exactly that amount
    for causal in (False, True):
        O0, l0 = fwd(Q, K, V, s, causal)
        delta = rng.standard_normal(N)
        kappa = 1.7
        Q2 = np.concatenate([Q, delta[None, None, :, None]], axis=3)
        K2 = np.concatenate([K, np.full((1, 1, N, 1), kappa)], axis=3)
        O2, l2 = fwd(Q2, K2, V, s, causal) if V.shape[3] == Q2.shape[3] else _fwd_dv(fwd, Q2, K2, V, s, causal)
        assert np.allclose(O2, O0, atol=1e-12)
        assert np.allclose(l2[0, 0], l0[0, 0] + s * delta * kappa, atol=1e-12)
    # permuting K and V rows together leaves O unchanged without a mask
    perm = rng.permutation(N)
    O0, l0 = fwd(Q, K, V, s, False)
    O1, l1 = fwd(Q, K[:, :, perm], V[:, :, perm], s, False)
    assert np.allclose(O0, O1, atol=1e-12) and np.allclose(l0, l1, atol=1e-12)
    # scaling: scale s with Q is the same as scale 1 with s*Q
    O0, l0 = fwd(Q, K, V, s, True)
    O1, l1 = fwd(s * Q, K, V, 1.0, True)
    assert np.allclose(O0, O1, atol=1e-12) and np.allclose(l0, l1, atol=1e-12)


def _fwd_dv(fwd, Q, K, V, s, causal):
    """Run fwd when V's width differs from Q/K's by padding V with zero columns."""
    extra = Q.shape[3] - V.shape[3]
    Vp = np.concatenate([V, np.zeros(V.shape[:3] + (extra,))], axis=3)
    O, l = fwd(Q, K, Vp, s, causal)
    return O[..., :V.shape[3]], l


def pin_gqa(fwd, bwd, rng):
    """A K/V head shared by G query heads equals G copies of it (repeat order h // G)."""
    B, Hq, Hkv, N, d = 2, 6, 2, 9, 4
    G = Hq // Hkv
    Q = rng.standard_normal((B, Hq, N, d))
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    dO = rng.standard_normal((B, Hq, N, d))
    Kr = np.repeat(K, G, axis=1)
    Vr = np.repeat(V, G, axis=1)
    for causal in (False, True):
        O, l = fwd(Q, K, V, 0.4, causal)
        Or, lr = fwd(Q, Kr, Vr, 0.4, causal)
        assert np.allclose(O, Or, atol=1e-13) and np.allclose(l, lr, atol=1e-13)
        dQ, dK, dV, _, _ = bwd(Q, K, V, dO, 0.4, causal)
        dQr, dKr, dVr, _, _ = bwd(Q, Kr, Vr, dO, 0.4, causal)
        assert np.allclose(dQ, dQr, atol=1e-12)
        assert np.allclose(dK, dKr.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-12)
        assert np.allclose(dV, dVr.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-12)


# ------------------------------------------------------- backward pins --

def pin_finite_differences(fwd, bwd, rng, h=1e-6, tol=1e-7):
    """Central differences of L = sum(dO * O) against the analytic gradients."""
    B, Hq, Hkv, N, d = 1, 2, 1, 7, 4
    Q = rng.standard_normal((B, Hq, N, d))
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    dO = rng.standard_normal((B, Hq, N, d))
    s = 0.6

    for causal in (False, True):
        def loss(Qx, Kx, Vx):
            O, _ = fwd(Qx, Kx, Vx, s, causal)
            return float((O * dO).sum())

        dQ, dK, dV, O, lse = bwd(Q, K, V, dO, s, causal)
        Of, lf = fwd(Q, K, V, s, causal)
        assert np.allclose(O, Of, atol=1e-13) and np.allclose(lse, lf, atol=1e-13)
        for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
            num = np.zeros_like(X)
            it = np.nditer(X, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                Xp = X.copy(); Xp[idx] += h
                Xm = X.copy(); Xm[idx] -= h
                args_p = {"Q": Q, "K": K, "V": V}; args_p[name] = Xp
                args_m = {"Q": Q, "K": K, "V": V}; args_m[name] = Xm
                num[idx] = (loss(**{k + "x": a for k, a in args_p.items()})
                            - loss(**{k + "x": a for k, a in args_m.items()})) / (2 * h)
            err = np.abs(num - G).max()
            assert err < tol, (name, causal, err)


def pin_backward_identities(bwd, rng):
    """rowsum(dS) = 0 gives sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (non-causal and causal)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 33, 8
    Q = rng.standard_normal((B, Hq, N, d))
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    dO = rng.standard_normal((B, Hq, N, d))
    for causal in (False, True):
        dQ, dK, dV, _, _ = bwd(Q, K, V, dO, 0.3, causal)
        assert np.allclose(dK.sum(axis=2), 0.0, atol=1e-11)
        exp = dO.reshape(B, Hkv, Hq // Hkv, N, d).sum(axis=(2, 3))
        assert np.allclose(dV.sum(axis=2), exp, atol=1e-11)
        # adding a constant vector to every K row shifts each score row by a
        # constant, so dQ is unchanged
        dQ2, _, _, _, _ = bwd(Q, K + rng.standard_normal(d), V, dO, 0.3, causal)
        assert np.allclose(dQ, dQ2, atol=1e-11)


# --------------------------------------------------- library routine --

def pin_torch_sdpa(fwd, bwd, rng):
    """Cross-check against torch's float64 CPU scaled_dot_product_attention + autograd."""
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, N, d = 2, 4, 2, 19, 8
    G = Hq // Hkv
    Q = rng.standard_normal((B, Hq, N, d))
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    dO = rng.standard_normal((B, Hq, N, d))
    for causal in (False, True):
        tq = torch.tensor(Q, requires_grad=True)
        tk = torch.tensor(K, requires_grad=True)
        tv = torch.tensor(V, requires_grad=True)
        out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, dim=1),
                                             tv.repeat_interleave(G, dim=1),
                                             is_causal=causal, scale=0.35)
        out.backward(torch.tensor(dO))
        O, _ = fwd(Q, K, V, 0.35, causal)
        dQ, dK, dV, _, _ = bwd(Q, K, V, dO, 0.35, causal)
        assert np.allclose(O, out.detach().numpy(), atol=1e-13)
        assert np.allclose(dQ, tq.grad.numpy(), atol=1e-12)
        assert np.allclose(dK, tk.grad.numpy(), atol=1e-12)
        assert np.allclose(dV, tv.grad.numpy(), atol=1e-12)


def pin_row_subset(fwd, rng):
    """Rows computed on their own equal the same rows of the full result."""
    Q = rng.standard_normal((1, 2, 50, 4))
    K = rng.standard_normal((1, 1, 50, 4))
    V = rng.standard_normal((1, 1, 50, 4))
    rows = np.array([0, 3, 17, 49, 48])
    for causal in (False, True):
        O, l = fwd(Q, K, V, 0.5, causal)
        Os, ls = fwd(Q, K, V, 0.5, causal, rows=rows)
        assert np.allclose(O[:, :, rows], Os, atol=1e-14) and np.allclose(l[:, :, rows], ls, atol=1e-14)


# ------------------------------------------ N_q != N_kv (split-KV forward) --

def brute_force_attention_kv(q, k, v, scale, causal):
    """Pure-Python evaluation for one head with N_q queries at the last N_q
    positions of an N_kv-key sequence (no numpy)."""
    nq, nk = len(q), len(k)
    d, dv = len(q[0]), len(v[0])
    out, lse = [], []
    for i in range(nq):
        pos = i + nk - nq
        scores = []
        for j in range(nk):
            if causal and j > pos:
                continue
            s = 0.0
            for t in range(d):
                s += q[i][t] * k[j][t]
            scores.append((j, scale * s))
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        row = [0.0] * dv
        for j, x in w:
            for t in range(dv):
                row[t] += x / tot * v[j][t]
        out.append(row)
        lse.append(mx + math.log(tot))
    return out, lse


def pin_kv_golden(fwd_kv, atol=1e-12):
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        cases = json.load(f)["kv_cases"]
    for c in cases:
        scale = parse_exact(c["scale"])
        O, lse = fwd_kv(_as4(c["Q"]), _as4(c["K"]), _as4(c["V"]), scale, c["causal"])
        expO = np.vectorize(parse_exact)(np.asarray(c["O"], dtype=object)).astype(np.float64)
        explse = np.array([parse_exact(x) for x in c["lse"]])
        assert np.allclose(O[0, 0], expO, atol=atol, rtol=0), (c["name"], O[0, 0], expO)
        assert np.allclose(lse[0, 0], explse, atol=atol, rtol=0), (c["name"], lse[0, 0], explse)


def pin_kv_brute_force(fwd_kv, rng, atol=1e-12):
    for (Nq, Nk, d, Hq, Hkv, causal) in [(1, 1, 2, 1, 1, True), (1, 7, 3, 2, 1, True),
                                         (3, 5, 2, 1, 1, True), (4, 9, 3, 4, 2, False),
                                         (5, 5, 2, 2, 2, True), (6, 2, 3, 1, 1, False)]:
        Q = rng.standard_normal((1, Hq, Nq, d))
        K = rng.standard_normal((1, Hkv, Nk, d))
        V = rng.standard_normal((1, Hkv, Nk, d))
        O, lse = fwd_kv(Q, K, V, 0.6, causal)
        G = Hq // Hkv
        for h in range(Hq):
            bo, bl = brute_force_attention_kv(Q[0, h].tolist(), K[0, h // G].tolist(),
                                              V[0, h // G].tolist(), 0.6, causal)
            assert np.allclose(O[0, h], np.array(bo), atol=atol, rtol=0), (Nq, Nk, h, causal)
            assert np.allclose(lse[0, h], np.array(bl), atol=atol, rtol=0), (Nq, Nk, h, causal)


def pin_kv_suffix(fwd_kv, fwd, rng):
    """The last N_q rows of square attention over N_kv positions (computed
    by the pinned square oracle, row subset) equal N_q queries at the end."""
    B, Hq, Hkv, N, d = 1, 4, 2, 40, 5
    Qf = rng.standard_normal((B, Hq, N, d))
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    for nq in (1, 3, 17, 40):
        rows = np.arange(N - nq, N)
        for causal in (False, True):
            Oref, lref = fwd(Qf, K, V, 0.45, causal, rows=rows)
            O, l = fwd_kv(Qf[:, :, N - nq:], K, V, 0.45, causal)
            assert np.allclose(O, Oref, atol=1e-13) and np.allclose(l, lref, atol=1e-13), (nq, causal)


def pin_kv_torch_sdpa(fwd_kv, rng):
    """torch float64 SDPA with the bottom-right causal mask written out."""
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 1, 6, 23, 8
    G = Hq // Hkv
    Q = rng.standard_normal((B, Hq, Nq, d))
    K = rng.standard_normal((B, Hkv, Nk, d))
    V = rng.standard_normal((B, Hkv, Nk, d))
    pos = torch.arange(Nq)[:, None] + (Nk - Nq)
    mask = torch.arange(Nk)[None, :] <= pos      # True = visible
    for causal in (False, True):
        ref = F.scaled_dot_product_attention(torch.tensor(Q), torch.tensor(K).repeat_interleave(G, dim=1),
                                             torch.tensor(V).repeat_interleave(G, dim=1),
                                             attn_mask=mask if causal else None, scale=0.3)
        O, _ = fwd_kv(Q, K, V, 0.3, causal)
        assert np.allclose(O, ref.numpy(), atol=1e-13), causal


def merge_partials(parts):
    """Combine per-chunk (O_s, lse_s) with the online-softmax rescale
    ("FlashAttention 1, 2, and 3 Explained", section 2): lse = ln sum exp(lse_s),
    O = sum_s exp(lse_s - lse) O_s."""
    lses = np.stack([l for _, l in parts])
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    lse = m + np.log(w.sum(axis=0))
    O = sum(np.exp(l - lse)[..., None] * o for o, l in parts)
    return O, lse


def pin_kv_merge(fwd_kv, rng):
    """Chunks of the keys processed on their own and merged give the whole."""
    Q = rng.standard_normal((1, 2, 3, 4))
    K = rng.standard_normal((1, 2, 29, 4))
    V = rng.standard_normal((1, 2, 29, 4))
    O, l = fwd_kv(Q, K, V, 0.8, False)
    for cuts in ([0, 10, 29], [0, 1, 2, 15, 29], [0, 29]):
        parts = [fwd_kv(Q, K[:, :, a:b], V[:, :, a:b], 0.8, False) for a, b in zip(cuts[:-1], cuts[1:])]
        Om, lm = merge_partials(parts)
        assert np.allclose(Om, O, atol=1e-13) and np.allclose(lm, l, atol=1e-13), cuts
