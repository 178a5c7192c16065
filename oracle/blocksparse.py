"""Attention under a block mask (block-sparse attention), in float64.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the
product path imports or runs it.

The block-sparse extension of the kernel skips the blocks of the attention
matrix that a sparsity mask zeroes ("FlashAttention and the Kernel Era", The
Breakthrough: the block-sparse extension and its Path-X / Path-256 results).
The pages give no mask format; the reading taken:

* A block mask M [H_m, ceil(N / blk), ceil(N / blk)] (H_m = 1 for one mask
  shared by every head, or H_q for one per query head, the same for every
  batch element); query i may see key j iff M[h_m, i // blk, j // blk] != 0
  and, under the causal mask, j <= i.
* Attention is the plain definition restricted to the visible keys: the
  softmax runs over them only.  A row with no visible key has output 0 and
  logsumexp -inf, and contributes no gradient.

Pinned in ``tests/test_oracle_blocksparse.py`` (all-ones masks against the
plain oracle, float64 SDPA with the element mask written out, a pure-Python
brute force, empty rows, finite differences).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import _check

__all__ = ["expand_block_mask", "attention_forward_masked", "attention_backward_masked",
           "attention_forward_blocksparse", "attention_backward_blocksparse"]


def expand_block_mask(M: np.ndarray, N: int, blk: int, causal: bool) -> np.ndarray:
    """Element visibility [H_m, N, N] of a block mask (and the causal mask)."""
    M = np.asarray(M)
    if M.ndim != 3 or M.shape[1] != (N + blk - 1) // blk or M.shape[2] != (N + blk - 1) // blk:
        raise ValueError("block mask must be [H_m, ceil(N / blk), ceil(N / blk)]")
    idx = np.arange(N) // blk
    vis = M[:, idx][:, :, idx] != 0
    if causal:
        vis = vis & np.tril(np.ones((N, N), dtype=bool))[None]
    return vis


def _head_mask(vis: np.ndarray, h: int) -> np.ndarray:
    return vis[0] if vis.shape[0] == 1 else vis[h]


def _masked_softmax(S: np.ndarray, vis: np.ndarray):
    """Row softmax over visible entries; rows with none give P = 0, lse = -inf."""
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    E = np.where(vis, np.exp(S - m), 0.0)
    ell = E.sum(axis=1, keepdims=True)
    P = np.where(empty, 0.0, E / np.where(empty, 1.0, ell))
    lse = np.where(empty[:, 0], -np.inf, (m + np.log(np.where(empty, 1.0, ell)))[:, 0])
    return P, lse


def attention_forward_masked(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                             vis: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax over the visible keys of scale * Q K^T, times V; vis is
    [1 or H_q, N, N] bool."""
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    O = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            Kh = np.asarray(K[b, h // G], dtype=np.float64)
            Vh = np.asarray(V[b, h // G], dtype=np.float64)
            S = scale * (np.asarray(Q[b, h], dtype=np.float64) @ Kh.T)
            P, l = _masked_softmax(S, _head_mask(vis, h))
            O[b, h] = P @ Vh
            lse[b, h] = l
    return O, lse


def attention_backward_masked(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                              scale: float, vis: np.ndarray):
    """(O, lse, dQ, dK, dV) of sum(dO * O) for the masked attention above."""
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    O = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    dQ = np.zeros((B, Hq, N, d))
    dK = np.zeros((B, Hkv, N, d))
    dV = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Kh = np.asarray(K[b, hk], dtype=np.float64)
            Vh = np.asarray(V[b, hk], dtype=np.float64)
            qr = np.asarray(Q[b, h], dtype=np.float64)
            dor = np.asarray(dO[b, h], dtype=np.float64)
            P, l = _masked_softmax(scale * (qr @ Kh.T), _head_mask(vis, h))
            Or = P @ Vh
            O[b, h] = Or
            lse[b, h] = l
            dV[b, hk] += P.T @ dor
            dP = dor @ Vh.T
            D = (dor * Or).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dQ[b, h] = scale * (dS @ Kh)
            dK[b, hk] += scale * (dS.T @ qr)
    return O, lse, dQ, dK, dV


def attention_forward_blocksparse(Q, K, V, scale: float, causal: bool, M: np.ndarray, blk: int = 128):
    N = np.asarray(Q).shape[2]
    return attention_forward_masked(Q, K, V, scale, expand_block_mask(M, N, blk, causal))


def attention_backward_blocksparse(Q, K, V, dO, scale: float, causal: bool, M: np.ndarray, blk: int = 128):
    N = np.asarray(Q).shape[2]
    return attention_backward_masked(Q, K, V, dO, scale, expand_block_mask(M, N, blk, causal))
