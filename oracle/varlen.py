"""Attention over a batch of sequences of different lengths, in float64.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the
product path imports or runs it.

The variable-length case generalises the ragged end of one sequence to a
batch ("FlashAttention and the Kernel Era", The Breakthrough: the kernel's
block-level skipping of what a mask excludes; "Flash Attention" (21medien),
the [batch, heads, seq_len, head_dim] layout of its code example).  The
reading taken: the tensors keep the padded layout [B, H, N, d]; sequence b
has L_b <= N valid tokens (a length per batch element); its queries and keys
at positions >= L_b take no part (padding):

    O[b, :, i] = attention of Q[b, :, i] over keys j < L_b   (j <= i if causal)
    O[b, :, i] = 0, lse = -inf                               for i >= L_b

and no gradient reaches padded positions.  Pinned in
``tests/test_oracle_varlen.py``.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention import _check, attention_backward, attention_forward

__all__ = ["attention_forward_varlen", "attention_backward_varlen"]


def _lengths(seqlens: Sequence[int], B: int, N: int) -> np.ndarray:
    L = np.asarray(seqlens, dtype=np.int64)
    if L.shape != (B,) or np.any(L < 0) or np.any(L > N):
        raise ValueError("seqlens must hold B lengths in [0, N]")
    return L


def attention_forward_varlen(Q, K, V, scale: float, causal: bool,
                             seqlens: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    L = _lengths(seqlens, B, N)
    O = np.zeros((B, Hq, N, d))
    lse = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        n = int(L[b])
        if n == 0:
            continue
        Ob, lb = attention_forward(Q[b:b + 1, :, :n], K[b:b + 1, :, :n], V[b:b + 1, :, :n], scale, causal)
        O[b, :, :n] = Ob[0]
        lse[b, :, :n] = lb[0]
    return O, lse


def attention_backward_varlen(Q, K, V, dO, scale: float, causal: bool, seqlens: Sequence[int]):
    """(O, lse, dQ, dK, dV) of sum(dO * O) for the forward above."""
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    L = _lengths(seqlens, B, N)
    O = np.zeros((B, Hq, N, d))
    lse = np.full((B, Hq, N), -np.inf)
    dQ = np.zeros((B, Hq, N, d))
    dK = np.zeros((B, Hkv, N, d))
    dV = np.zeros((B, Hkv, N, d))
    for b in range(B):
        n = int(L[b])
        if n == 0:
            continue
        sl = (slice(b, b + 1), slice(None), slice(0, n))
        dq, dk, dv, ob, lb = attention_backward(Q[sl], K[sl], V[sl], dO[sl], scale, causal)
        O[b, :, :n], lse[b, :, :n] = ob[0], lb[0]
        dQ[b, :, :n], dK[b, :, :n], dV[b, :, :n] = dq[0], dk[0], dv[0]
    return O, lse, dQ, dK, dV
