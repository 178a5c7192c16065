"""fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package entry's ``smoke()``
check and the benchmark's CPU-baseline leg use it.  It shares no code, tables
or helpers with the HIP library; the only thing both sides share is the
seeded input generator (``workloads.py``), which holds no attention
arithmetic.

What it computes is the plain definition, not the tiled algorithm.  The pages
state that FlashAttention returns the same result as standard attention, up to
floating-point rounding (the "FlashAttention" glossary page, first paragraph;
"FlashAttention and the Kernel Era", The Breakthrough), so the reference
answer is standard attention evaluated in float64, materialising S and P:

    S = scale * Q K^T                 ("FlashAttention and the Kernel Era",
    P = softmax(S)  (row-wise)          The Mathematics, the SDPA equation;
    O = P V                             "FlashAttention 1, 2, and 3 Explained",
                                        section 1, the S / P / O equations)

Readings taken where the pages leave a step open:

* ``scale`` is an argument.  The SDPA equation divides by sqrt(d); the
  initnode page's S = QK^T has no factor.  Every workload passes 1/sqrt(d).
* Causal mask ("Flash Attention" (21medien), Code Example, ``is_causal=True``):
  key j is visible to query i iff j <= i (N_q == N_k, so there is no
  alignment question).
* Saved statistic: the per-row natural-log logsumexp of the scaled, masked
  scores, lse_i = log sum_j exp(S_ij).  The pages say the backward pass
  reuses stored softmax statistics ("FlashAttention Kernel" glossary, the
  Tiling / Recomputation bullets) without fixing which; the logsumexp is the
  one statistic from which P can be rebuilt in one pass.
* Grouped K/V heads (GQA/MQA, "FlashAttention" glossary, KV-cache
  paragraph): query head h reads K/V head floor(h / G) with G = H_q / H_kv.
* Backward: the pages give no gradient formulas, only that P is recomputed
  from Q, K, V and the statistics.  The gradients below are the textbook
  chain rule through O = P V and the row-wise softmax Jacobian
  (dS = P * (dP - rowsum(dP * P)), and rowsum(dP * P) = rowsum(dO * O)).
  They are pinned by central finite differences in the tests.

Parity status: every function here is pinned (hand-worked examples, closed
forms, invariants, brute force, finite differences, and a float64 library
routine) -- see ``tests/test_oracle.py``.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["attention_forward", "attention_forward_kv", "attention_backward", "attention_probs"]


def _check(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> Tuple[int, int, int, int, int, int]:
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("Q, K, V must be [B, H, N, d]")
    B, Hq, N, d = Q.shape
    Bk, Hkv, Nk, dk = K.shape
    if K.shape != V.shape or Bk != B or Nk != N or dk != d:
        raise ValueError("K and V must be [B, H_kv, N, d] matching Q")
    if Hq % Hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return B, Hq, Hkv, N, d, Hq // Hkv


def _scores(q_rows: np.ndarray, row_idx: np.ndarray, Kh: np.ndarray, scale: float,
            causal: bool) -> np.ndarray:
    """S = scale * Q[rows] K^T with -inf where the causal mask hides a key."""
    S = scale * (q_rows @ Kh.T)
    if causal:
        cols = np.arange(Kh.shape[0])
        S = np.where(cols[None, :] <= row_idx[:, None], S, -np.inf)
    return S


def _softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise softmax and natural-log logsumexp, with the max subtracted."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    ell = E.sum(axis=1, keepdims=True)
    return E / ell, (m + np.log(ell))[:, 0]


def attention_probs(Q: np.ndarray, K: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """The full probability matrix P = softmax(scale * Q K^T) for one head.

    Q, K are [N, d].  Only for small N (it is N x N).
    """
    N = Q.shape[0]
    P, _ = _softmax_rows(_scores(Q, np.arange(N), K, scale, causal))
    return P


def attention_forward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                      causal: bool, rows: Optional[np.ndarray] = None,
                      chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax(scale * Q K^T) V and the per-row logsumexp, in float64.

    Q is [B, H_q, N, d]; K, V are [B, H_kv, N, d].  Returns O [B, H_q, R, d]
    and lse [B, H_q, R], where R = N, or R = len(rows) when ``rows`` selects
    a subset of query rows (each output row depends only on its own query row,
    so a subset is computed exactly as the full result would be).
    """
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    row_idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    O = np.empty((B, Hq, R, d), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Kh = np.asarray(K[b, hk], dtype=np.float64)
            Vh = np.asarray(V[b, hk], dtype=np.float64)
            for r0 in range(0, R, chunk):
                idx = row_idx[r0:r0 + chunk]
                qr = np.asarray(Q[b, h, idx], dtype=np.float64)
                P, l = _softmax_rows(_scores(qr, idx, Kh, scale, causal))
                O[b, h, r0:r0 + len(idx)] = P @ Vh
                lse[b, h, r0:r0 + len(idx)] = l
    return O, lse


def attention_forward_kv(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                         causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of N_q query rows against N_kv keys (the split-KV / decoding
    case, "FlashAttention" glossary, FlashDecoding paragraph), in float64.

    Q is [B, H_q, N_q, d]; K, V are [B, H_kv, N_kv, d].  Returns O
    [B, H_q, N_q, d] and the natural-log lse [B, H_q, N_q].

    Reading taken (the pages fix no alignment for N_q != N_kv): the queries
    are the last N_q positions of the sequence, so under the causal mask query
    i sees keys j <= i + N_kv - N_q (which requires N_q <= N_kv, so every row
    sees at least key 0).  With N_q == N_kv this is ``attention_forward``.
    """
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4 or K.shape != V.shape:
        raise ValueError("Q must be [B, H_q, N_q, d] and K, V [B, H_kv, N_kv, d]")
    B, Hq, Nq, d = Q.shape
    Bk, Hkv, Nkv, dk = K.shape
    if Bk != B or dk != d or Hq % Hkv != 0:
        raise ValueError("K and V must match Q's batch and head dimension")
    shift = Nkv - Nq
    if causal and shift < 0:
        raise ValueError("causal attention needs N_q <= N_kv")
    G = Hq // Hkv
    pos = np.arange(Nq) + shift          # sequence position of each query
    O = np.empty((B, Hq, Nq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Kh = np.asarray(K[b, hk], dtype=np.float64)
            Vh = np.asarray(V[b, hk], dtype=np.float64)
            qr = np.asarray(Q[b, h], dtype=np.float64)
            P, l = _softmax_rows(_scores(qr, pos, Kh, scale, causal))
            O[b, h] = P @ Vh
            lse[b, h] = l
    return O, lse


def attention_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                       scale: float, causal: bool, chunk: int = 1024,
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of L = sum(dO * O) with respect to Q, K, V, in float64.

    P is rebuilt from the definition, then, per query row chunk:
        D   = rowsum(dO * O)
        dV += P^T dO
        dP  = dO V^T
        dS  = P * (dP - D)
        dQ  = scale * dS K
        dK += scale * dS^T Q
    dK and dV of a K/V head sum the contributions of the G query heads that
    read it.  Returns (dQ, dK, dV, O, lse); O and lse are the oracle's own.
    """
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    if dO.shape != Q.shape:
        raise ValueError("dO must have Q's shape")
    dQ = np.zeros(Q.shape, dtype=np.float64)
    dK = np.zeros(K.shape, dtype=np.float64)
    dV = np.zeros(V.shape, dtype=np.float64)
    O = np.empty(Q.shape, dtype=np.float64)
    lse = np.empty(Q.shape[:3], dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Kh = np.asarray(K[b, hk], dtype=np.float64)
            Vh = np.asarray(V[b, hk], dtype=np.float64)
            for r0 in range(0, N, chunk):
                idx = np.arange(r0, min(N, r0 + chunk))
                qr = np.asarray(Q[b, h, idx], dtype=np.float64)
                dor = np.asarray(dO[b, h, idx], dtype=np.float64)
                P, l = _softmax_rows(_scores(qr, idx, Kh, scale, causal))
                Or = P @ Vh
                O[b, h, idx] = Or
                lse[b, h, idx] = l
                D = (dor * Or).sum(axis=1, keepdims=True)
                dV[b, hk] += P.T @ dor
                dP = dor @ Vh.T
                dS = P * (dP - D)
                dQ[b, h, idx] = scale * (dS @ Kh)
                dK[b, hk] += scale * (dS.T @ qr)
    return dQ, dK, dV, O, lse
