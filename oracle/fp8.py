"""FP8 block quantization and attention on the quantized values, in NumPy.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the
product path imports or runs it.

The FP8 forward ("FlashAttention 1, 2, and 3 Explained", section 4: FP8 with
block quantization and incoherent processing; "FlashAttention" glossary,
FA3 paragraph) is not exact attention of the inputs: Q, K and V are rounded to
8-bit floats first.  Its oracle is therefore two plain definitions:

1. The quantizer.  For a tensor x [..., N, d] split into blocks of
   ``block_rows`` consecutive rows:
     * optional rotation ("incoherent processing"): y = (x * s) H / sqrt(d),
       with s a given vector of +-1 signs and H the d x d Sylvester Hadamard
       matrix.  A random orthogonal rotation applied to both Q and K leaves
       every score q . k unchanged and spreads outlier features over all
       dimensions before rounding.
     * per block: amax = max |y|, inv = 448 / amax, scale = amax / 448, and
       the code of y * inv rounded to nearest (ties to even) in the OCP
       e4m3 format (4 exponent bits, bias 7, 3 mantissa bits, largest finite
       value 448, no infinities).  A block with amax = 0, or with amax so
       small (below 448 / FLT_MAX, about 1.3e-36) that 448 / amax overflows
       float32, gets scale 1 and zero codes: its values are below anything
       e4m3 times a float32 scale can resolve, and flushing them keeps every
       code finite.
   Every step is written in float32 in a fixed order (the butterflies of the
   fast Walsh-Hadamard transform with strides 1, 2, 4, ..., then the scale),
   so that the rounded codes are a deterministic function of the input and
   can be compared bit for bit.

2. Attention of the dequantized values (code value * block scale), the plain
   definition of ``attention.attention_forward`` evaluated in float64.

Pinned in ``tests/test_oracle_fp8.py`` against torch's float8_e4m3fn casts,
scipy's Hadamard matrix, exhaustive code tables and closed forms.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

E4M3_MAX = 448.0

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "wht_fp32", "quantize_blocks",
           "dequantize_blocks", "attention_fp8"]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 codes (uint8) to float64: sign, 4-bit exponent (bias 7),
    3-bit mantissa; exponent 0 is subnormal (m * 2^-9); code 0x7f / 0xff is
    NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_POS = e4m3_decode(np.arange(127, dtype=np.uint8))   # codes 0..126: every finite value >= 0


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float values with |x| <= 448 to the nearest e4m3 code, ties to
    the even code (even mantissa); the sign bit follows the input's sign."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode takes finite values with |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_POS, a, side="left")           # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    # the sign bit is kept, also when the magnitude rounds to zero (-0)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def wht_fp32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """(x * signs) H / sqrt(d) along the last axis, in float32: butterflies
    (a, b) -> (a + b, a - b) with strides 1, 2, 4, ..., d/2, then one
    multiplication by float32(1 / sqrt(d))."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*y.shape[:-3], d)
        h *= 2
    return y * np.float32(1.0 / np.sqrt(d))


def quantize_blocks(x: np.ndarray, block_rows: int,
                    signs: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """x [B, H, N, d] -> (codes uint8 [B, H, N, d], scales float32
    [B, H, ceil(N / block_rows)]) as described in the module docstring."""
    x = np.asarray(x, dtype=np.float32)
    y = wht_fp32(x, signs) if signs is not None else x
    B, H, N, d = y.shape
    nb = (N + block_rows - 1) // block_rows
    codes = np.empty(y.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for i in range(nb):
        blk = y[:, :, i * block_rows:(i + 1) * block_rows]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        with np.errstate(divide="ignore", over="ignore"):
            raw = (np.float32(E4M3_MAX) / np.where(amax == 0, np.float32(1), amax)).astype(np.float32)
        zero = (amax == 0) | ~np.isfinite(raw)
        inv = np.where(zero, np.float32(1), raw).astype(np.float32)
        scales[:, :, i] = np.where(zero, np.float32(1), amax / np.float32(E4M3_MAX)).astype(np.float32)
        v = (blk * inv[:, :, None, None]).astype(np.float32)
        v = np.clip(v, -E4M3_MAX, E4M3_MAX)
        c = e4m3_encode(v)
        c[zero] = 0
        codes[:, :, i * block_rows:(i + 1) * block_rows] = c
    return codes, scales


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block_rows: int) -> np.ndarray:
    """Code values times their block's scale, float64 [B, H, N, d]."""
    vals = e4m3_decode(codes)
    rep = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=2)[:, :, :codes.shape[2]]
    return vals * rep[..., None]


def attention_fp8(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool,
                  block_rows: int = 64, signs: Optional[np.ndarray] = None,
                  rows: Optional[np.ndarray] = None):
    """Attention of block-quantized inputs: Q and K are rotated with the same
    signs (when given), Q, K and V are quantized in blocks of ``block_rows``
    rows, and the oracle's exact attention runs on the dequantized values.
    Returns (O, lse) in float64, as ``attention.attention_forward`` (``rows``
    selects query rows there)."""
    from .attention import attention_forward
    qc, qs = quantize_blocks(Q, block_rows, signs)
    kc, ks = quantize_blocks(K, block_rows, signs)
    vc, vs = quantize_blocks(V, block_rows)
    return attention_forward(dequantize_blocks(qc, qs, block_rows), dequantize_blocks(kc, ks, block_rows),
                             dequantize_blocks(vc, vs, block_rows), scale, causal, rows=rows)
