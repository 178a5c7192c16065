"""Attention with dropout on the probabilities, and its counter-based mask.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the
product path imports or runs it.

Dropout is one of the operations the fused kernel applies to the attention
matrix without writing it out ("FlashAttention Kernel" glossary, opening
paragraph; "FlashAttention" glossary, kernel-fusion paragraph; "Flash
Attention" (21medien), fusion bullet, and its code example's dropout_p
argument).  The pages fix neither where the mask comes from nor its scaling;
the readings taken:

* Mask: element (b, h, i, j) (query head h, query row i, key j) is kept iff
  its random byte u is below t = round((1 - p) 256), with u drawn by the
  counter-based generator Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): key (seed, offset), counter
  (j // 32, i, b H_q + h, 0); the four 64-bit outputs hold 32 bytes,
  little-endian, and byte j % 32 belongs to key j.
* Kept probabilities are multiplied by 256 / t, the inverse of the keep
  probability t / 256, so that the expected output is the output without
  dropout.  p must leave t >= 1.
* The softmax statistics are those of the undropped scores:
      P = softmax(scale Q K^T),  O = (P o Z) V * 256 / t,
      lse = ln sum_j exp(scale q_i . k_j)   (as without dropout).
* Backward (chain rule through O): with Pd = P o Z * 256 / t,
      dV = Pd^T dO,   dP = (dO V^T) o Z * 256 / t,
      D_i = sum_c dO_ic O_ic,   dS = P o (dP - D),
      dQ = scale dS K,   dK = scale dS^T Q.

Pinned in ``tests/test_oracle_dropout.py``: the generator against numpy's
``Philox`` bit generator, a pure-Python brute force with its own scalar
generator, p = 0 against the plain oracle, keep statistics, and finite
differences of the backward pass.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import _check, _scores, _softmax_rows

__all__ = ["PHILOX_M", "PHILOX_W", "philox4x64", "keep_threshold", "keep_scale", "random_bytes",
           "keep_mask", "attention_forward_dropout", "attention_backward_dropout"]

# Philox4x64 multipliers and Weyl key increments (Salmon et al., table 2 and
# section 5.1)
PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)
_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: int) -> Tuple[np.ndarray, np.ndarray]:
    """(high, low) 64-bit halves of the 128-bit product a * m, from four
    32 x 32-bit partial products (uint64 arithmetic wraps modulo 2^64)."""
    a0, a1 = a & _M32, a >> _S32
    m0, m1 = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> _S32) + (p01 & _M32) + (p10 & _M32)
    lo = (p00 & _M32) | ((mid & _M32) << _S32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64(ctr, key, rounds: int = 10):
    """Philox4x64-R on arrays of counters.  ctr: four uint64 arrays (or
    scalars) c0..c3; key: two uint64 values.  Each round: (hi0, lo0) =
    M0 c0, (hi1, lo1) = M1 c2, then c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1,
    lo0), and the key advances by the Weyl constants."""
    with np.errstate(over="ignore"):
        c = [np.asarray(x, dtype=np.uint64) for x in ctr]
        k0, k1 = np.uint64(key[0]), np.uint64(key[1])
        for _ in range(rounds):
            hi0, lo0 = _mulhilo(c[0], PHILOX_M[0])
            hi1, lo1 = _mulhilo(c[2], PHILOX_M[1])
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
            k0 = k0 + np.uint64(PHILOX_W[0])
            k1 = k1 + np.uint64(PHILOX_W[1])
    return c


def keep_threshold(p: float) -> int:
    """t = round((1 - p) 256); a byte u keeps its element iff u < t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    t = int(np.floor((1.0 - p) * 256.0 + 0.5))
    if t < 1:
        raise ValueError("dropout probability leaves no byte below the threshold")
    return t


def keep_scale(p: float) -> float:
    return 256.0 / keep_threshold(p)


def random_bytes(bh: int, rows: np.ndarray, n_keys: int, seed: int, offset: int) -> np.ndarray:
    """The random byte of every (row, key) of one (batch * H_q + head) index:
    uint8 [len(rows), n_keys]."""
    rows = np.asarray(rows, dtype=np.uint64)
    nblk = (n_keys + 31) // 32
    blk = np.arange(nblk, dtype=np.uint64)
    c0 = np.broadcast_to(blk[None, :], (len(rows), nblk))
    c1 = np.broadcast_to(rows[:, None], (len(rows), nblk))
    c2 = np.full_like(c0, np.uint64(bh))
    c3 = np.zeros_like(c0)
    out = philox4x64([c0, c1, c2, c3], (seed, offset))
    words = np.stack(out, axis=-1)                       # [rows, nblk, 4] uint64
    by = words.astype("<u8").view(np.uint8)              # little-endian bytes, 32 per block
    return by.reshape(len(rows), nblk * 32)[:, :n_keys]


def keep_mask(B: int, H: int, N_rows: int, N_keys: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep mask [B, H, N_rows, N_keys] (query head index h)."""
    t = keep_threshold(p)
    Z = np.empty((B, H, N_rows, N_keys), dtype=bool)
    for b in range(B):
        for h in range(H):
            Z[b, h] = random_bytes(b * H + h, np.arange(N_rows), N_keys, seed, offset) < t
    return Z


def attention_forward_dropout(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                              causal: bool, p: float, seed: int, offset: int
                              ) -> Tuple[np.ndarray, np.ndarray]:
    """O = (P o Z) V * 256 / t and the (undropped) row logsumexp, float64."""
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    s = keep_scale(p)
    t = keep_threshold(p)
    O = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            Kh = np.asarray(K[b, h // G], dtype=np.float64)
            Vh = np.asarray(V[b, h // G], dtype=np.float64)
            P, l = _softmax_rows(_scores(np.asarray(Q[b, h], dtype=np.float64), rows, Kh, scale, causal))
            Z = random_bytes(b * Hq + h, rows, N, seed, offset) < t
            O[b, h] = (P * Z * s) @ Vh
            lse[b, h] = l
    return O, lse


def attention_backward_dropout(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                               scale: float, causal: bool, p: float, seed: int, offset: int):
    """(O, lse, dQ, dK, dV) of sum(dO * O) with the dropout forward above."""
    B, Hq, Hkv, N, d, G = _check(Q, K, V)
    s = keep_scale(p)
    t = keep_threshold(p)
    O = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    dQ = np.zeros((B, Hq, N, d))
    dK = np.zeros((B, Hkv, N, d))
    dV = np.zeros((B, Hkv, N, d))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Kh = np.asarray(K[b, hk], dtype=np.float64)
            Vh = np.asarray(V[b, hk], dtype=np.float64)
            qr = np.asarray(Q[b, h], dtype=np.float64)
            dor = np.asarray(dO[b, h], dtype=np.float64)
            P, l = _softmax_rows(_scores(qr, rows, Kh, scale, causal))
            Zs = (random_bytes(b * Hq + h, rows, N, seed, offset) < t) * s
            Pd = P * Zs
            Or = Pd @ Vh
            O[b, h] = Or
            lse[b, h] = l
            dV[b, hk] += Pd.T @ dor
            dP = (dor @ Vh.T) * Zs
            D = (dor * Or).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dQ[b, h] = scale * (dS @ Kh)
            dK[b, hk] += scale * (dS.T @ qr)
    return O, lse, dQ, dK, dV
