"""FP8 path on the GPU (through the C-ABI) against the oracle.

* The quantizer is compared bit for bit (codes and scales) with
  ``oracle.fp8.quantize_blocks``: both evaluate the same float32 steps and
  round to e4m3 to nearest even.
* The forward receives codes and scales made by the oracle and is compared
  with the oracle's float64 attention of the dequantized values.  The kernel
  rounds the probabilities to e4m3 before the P V product; its error bound
  per output element, with p the exact probabilities of the dequantized
  scores and V the dequantized values:
      |o - O| <= 2^-4 sum_j p_j |V_jc|      (relative rounding of each p_j)
               + 2^-8 |O|                   (bf16 / fp16 output rounding)
               + 2^-10 max |V|              (probabilities below the normal
                                             e4m3 range, whose spacing is
                                             absolute; random-signed sums)
  and, as the roundings are independent with relative RMS at most
  2^-4 / sqrt(3), the mean error stays below
      2^-4 / sqrt(3) * mean sqrt(sum_j p_j^2 V_jc^2) + 2^-9 mean |O|.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_fp8_quantize, fa_fwd, fa_fwd_fp8
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BLK = 64


def _oracle_quant(x, signs=None):
    return ofp8.quantize_blocks(workloads.to_f64(x).astype(np.float32), BLK, signs)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# --------------------------------------------------------------- quantizer

QCASES = [
    # B, H, N, d
    (1, 2, 64, 128),
    (2, 3, 100, 128),     # ragged last block
    (1, 1, 1, 64),        # one row
    (1, 4, 257, 64),
    (2, 2, 1000, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rot", [False, True])
def test_quantizer_bit_exact(dtype, rot):
    for i, (B, H, N, d) in enumerate(QCASES):
        print(f"quant case dtype={dtype} rot={rot} B={B} H={H} N={N} d={d}", flush=True)
        x = workloads.make_inputs(B, H, H, N, d, dtype, 500 + i)[0] * 3
        signs = workloads.make_signs(d, 600 + i) if rot else None
        codes, scales = fa_fp8_quantize(x.to(DEV), signs.to(DEV) if rot else None)
        torch.cuda.synchronize()
        ref_c, ref_s = _oracle_quant(x, signs.numpy() if rot else None)
        got_c = codes.cpu().numpy()
        assert np.array_equal(scales.cpu().numpy(), ref_s), f"case {i} scales"
        bad = np.argwhere(got_c != ref_c)
        assert bad.size == 0, f"case {i}: {len(bad)} codes differ, first at {bad[:4].tolist()}"


def test_quantizer_special_values():
    """Zero blocks (scale 1), signed zeros, values that round to zero, ties."""
    B, H, N, d = 1, 1, 192, 64
    x = torch.zeros((B, H, N, d), dtype=torch.float32)
    # block 1: +-0, tiny values, and an amax of 448 * 2^-4 = 28 so that the
    # multiplier 448 / amax is exactly 16
    x[0, 0, 64, 0] = 28.0
    x[0, 0, 64, 1] = -0.0
    x[0, 0, 64, 2:10] = torch.tensor([2.0 ** -14, -2.0 ** -14, 2.0 ** -13, -2.0 ** -13,
                                      3 * 2.0 ** -14, -3 * 2.0 ** -14, 2.0 ** -20, -2.0 ** -20])
    # block 2: every e4m3 midpoint below 28 (ties to even after the exact x16)
    pos = ofp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2) / 16
    x[0, 0, 128, 0] = 28.0
    x[0, 0, 129:131].view(-1)[:len(mids)] = torch.tensor(mids, dtype=torch.float32)
    x = x.to(torch.bfloat16)
    codes, scales = fa_fp8_quantize(x.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_s = _oracle_quant(x)
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert scales[0, 0, 0].item() == 1.0 and not codes[0, 0, :64].any()
    assert np.array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_quantizer_limits_of_the_block_scale(dtype):
    """Blocks at both ends of the scale's range, bit for bit against the oracle.

    block 0: amax = 0.60546875, a value whose product amax * fl(448 / amax)
             rounds above 448 in float32; that element (and its negation)
             must still encode as +-448.
    block 1 (bf16 only): amax = 2^-122, below 448 / FLT_MAX, where 448 / amax
             overflows: the block is stored as zeros (also its negative
             values) with scale 1.
    block 2: amax = 2^-119 (bf16) just above that limit: ordinary scale.
    block 3: random values, for contrast.
    """
    B, H, N, d = 1, 2, 4 * BLK, 128
    amax0 = np.float32(0.60546875)
    assert np.float32(amax0 * (np.float32(448) / amax0)) > np.float32(448)
    gen = torch.Generator().manual_seed(77)
    x = torch.randn((B, H, N, d), generator=gen) * 0.1
    x[:, :, 0:BLK] = x[:, :, 0:BLK].clamp(-0.5, 0.5)
    x[:, 0, 3, 7] = float(amax0)
    x[:, 1, 10, 0] = -float(amax0)
    x[:, 1, 11, 1] = float(amax0)
    if dtype == "bf16":
        x[:, :, BLK:2 * BLK] = torch.sign(torch.randn((B, H, BLK, d), generator=gen)) * 2.0 ** -124
        x[:, :, BLK + 5, 3] = -(2.0 ** -122)
        x[:, :, 2 * BLK:3 * BLK] = torch.sign(torch.randn((B, H, BLK, d), generator=gen)) * 2.0 ** -121
        x[:, :, 2 * BLK + 9, 2] = 2.0 ** -119
    x = x.to(workloads.DTYPES[dtype])
    codes, scales = fa_fp8_quantize(x.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_s = _oracle_quant(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s, ref_s)
    assert np.array_equal(got_c, ref_c), np.argwhere(got_c != ref_c)[:4].tolist()
    assert got_c[0, 0, 3, 7] == 0x7E and got_c[0, 1, 10, 0] == 0xFE and got_c[0, 1, 11, 1] == 0x7E
    if dtype == "bf16":
        assert (got_s[:, :, 1] == 1.0).all() and not got_c[:, :, BLK:2 * BLK].any()
        assert (got_s[:, :, 2] == np.float32(2.0 ** -119) / np.float32(448)).all()
        assert got_c[0, 0, 2 * BLK + 9, 2] == 0x7E


def test_quantizer_full_size_sampled_heads():
    """The bench workload's shape (B=4, H=32, N=8192, d=128, rotated), every
    head in one call; three heads bit for bit against the oracle, and every
    block's scale against the amax the codes imply."""
    B, H, N, d = 4, 32, 8192, 128
    x = workloads.make_inputs(B, H, H, N, d, "bf16", 4242)[0]
    signs = workloads.make_signs(d, 4243)
    codes, scales = fa_fp8_quantize(x.to(DEV), signs.to(DEV))
    torch.cuda.synchronize()
    codes, scales = codes.cpu(), scales.cpu()
    for b, h in ((0, 0), (1, 17), (3, 31)):
        print(f"quant full size head b={b} h={h}", flush=True)
        rc, rs = _oracle_quant(x[b:b + 1, h:h + 1], signs.numpy())
        assert np.array_equal(scales[b:b + 1, h:h + 1].numpy(), rs)
        assert np.array_equal(codes[b:b + 1, h:h + 1].numpy(), rc)
    # every block holds a code of magnitude 448 (its largest element), and
    # no NaN code anywhere
    c = codes.view(B, H, N // BLK, BLK * d).numpy()
    assert ((c & 0x7F) == 0x7E).any(axis=-1).all()
    assert not ((c & 0x7F) == 0x7F).any()


# ----------------------------------------------------------------- forward

def _bound(Qd, Kd, Vd, scale, causal, O, with_mean=False):
    """The per-element error bound of the module docstring (and the bound on
    the mean error)."""
    B, Hq, N, d = Qd.shape
    G = Hq // Kd.shape[1]
    A = np.empty_like(O)
    R = np.empty_like(O)
    vmax = np.empty((B, Hq, 1, 1))
    for b in range(B):
        for h in range(Hq):
            P = oracle.attention_probs(Qd[b, h], Kd[b, h // G], scale, causal)
            A[b, h] = P @ np.abs(Vd[b, h // G])
            R[b, h] = np.sqrt((P ** 2) @ (Vd[b, h // G] ** 2))
            vmax[b, h] = np.abs(Vd[b, h // G]).max()
    bound = 2.0 ** -4 * A + 2.0 ** -8 * np.abs(O) + 2.0 ** -10 * vmax
    if with_mean:
        return bound, 2.0 ** -4 / math.sqrt(3) * R.mean() + 2.0 ** -9 * np.abs(O).mean()
    return bound


def _run_fwd(q, k, v, causal, scale, signs=None, out="bf16"):
    qc, qs = _oracle_quant(q, signs)
    kc, ks = _oracle_quant(k, signs)
    vc, vs = _oracle_quant(v)
    o, lse = fa_fwd_fp8(_t(qc), _t(kc), _t(vc), _t(qs), _t(ks), _t(vs), causal, scale, out)
    torch.cuda.synchronize()
    Qd, Kd, Vd = (ofp8.dequantize_blocks(c, s, BLK) for c, s in ((qc, qs), (kc, ks), (vc, vs)))
    O, L = oracle.attention_forward(Qd, Kd, Vd, scale, causal)
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), O, L, (Qd, Kd, Vd)


FCASES = [
    # B, Hq, Hkv, N, d
    (1, 2, 2, 64, 128),
    (1, 2, 1, 300, 128),     # GQA, ragged tail
    (2, 2, 2, 257, 64),
    (1, 4, 2, 1000, 128),    # several row blocks and key tiles
    (1, 1, 1, 1, 128),       # one row
    (1, 2, 2, 513, 64),
]


@pytest.mark.parametrize("causal", [False, True])
def test_forward_parity(causal):
    for i, (B, Hq, Hkv, N, d) in enumerate(FCASES):
        print(f"fwd case causal={causal} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}", flush=True)
        q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 700 + i)
        scale = 1 / math.sqrt(d)
        o, lse, O, L, (Qd, Kd, Vd) = _run_fwd(q, k, v, causal, scale)
        bound, mean_bound = _bound(Qd, Kd, Vd, scale, causal, O, with_mean=True)
        err = np.abs(o - O)
        assert np.isfinite(o).all()
        assert (err <= bound).all(), f"case {i}: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"
        assert err.mean() <= mean_bound, f"case {i}: mean err {err.mean():.3e} > {mean_bound:.3e}"
        print(f"  max err {err.max():.3e} (worst ratio to bound {(err / bound).max():.3f}), "
              f"mean {err.mean():.3e} (bound {mean_bound:.3e})", flush=True)
        assert np.abs(lse - L).max() <= 1e-3, f"case {i}: lse err {np.abs(lse - L).max():.3e}"


@pytest.mark.parametrize("out", ["bf16", "fp16"])
def test_forward_rotated_inputs_and_output_types(out):
    B, Hq, Hkv, N, d = 1, 4, 4, 384, 128
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 801)
    signs = workloads.make_signs(d, 802).numpy()
    scale = 1 / math.sqrt(d)
    o, lse, O, L, (Qd, Kd, Vd) = _run_fwd(q, k, v, True, scale, signs, out)
    err = np.abs(o - O)
    assert (err <= _bound(Qd, Kd, Vd, scale, True, O)).all(), err.max()
    assert np.abs(lse - L).max() <= 1e-3


def test_forward_block_scales_spread():
    """Value blocks whose scales differ by 2^12 (their probabilities enter the
    product scaled by s_v / max s_v) and query/key blocks of mixed scale."""
    B, H, N, d = 1, 2, 512, 128
    q, k, v, _ = workloads.make_inputs(B, H, H, N, d, "bf16", 811)
    f = torch.tensor([2.0 ** (-(i % 4) * 4) for i in range(N // BLK)]).repeat_interleave(BLK)
    v = (v.float() * f[None, None, :, None]).to(torch.bfloat16)
    q = (q.float() * f.flip(0)[None, None, :, None] * 4).to(torch.bfloat16)
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        o, lse, O, L, (Qd, Kd, Vd) = _run_fwd(q, k, v, causal, scale)
        err = np.abs(o - O)
        assert (err <= _bound(Qd, Kd, Vd, scale, causal, O)).all(), err.max()
        assert np.abs(lse - L).max() <= 1e-3


def test_quantize_then_forward_end_to_end():
    """GPU quantizer feeding the GPU forward, against the oracle's FP8
    attention of the same 16-bit inputs, and the FP8 error against exact
    attention of the unquantized inputs next to the 16-bit kernel's."""
    B, Hq, Hkv, N, d = 1, 4, 2, 640, 128
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 821)
    signs = workloads.make_signs(d, 822)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, sd = q.to(DEV), k.to(DEV), v.to(DEV), signs.to(DEV)
    qc, qs = fa_fp8_quantize(qd, sd)
    kc, ks = fa_fp8_quantize(kd, sd)
    vc, vs = fa_fp8_quantize(vd)
    o, lse = fa_fwd_fp8(qc, kc, vc, qs, ks, vs, True, scale)
    o16, _ = fa_fwd(qd, kd, vd, True, scale)
    torch.cuda.synchronize()
    f = workloads.to_f64
    O8, L8 = ofp8.attention_fp8(f(q), f(k), f(v), scale, True, BLK, signs.numpy())
    O, _ = oracle.attention_forward(f(q), f(k), f(v), scale, True)
    got = o.double().cpu().numpy()
    assert np.abs(lse.double().cpu().numpy() - L8).max() <= 1e-3
    rms = lambda x: float(np.sqrt(np.mean(x ** 2)))
    e_kernel_vs_fp8 = rms(got - O8)
    e_fp8 = rms(O8 - O)
    e_kernel = rms(got - O)
    print(f"rms: kernel-vs-oracle-fp8 {e_kernel_vs_fp8:.3e}, oracle fp8 vs exact {e_fp8:.3e}, "
          f"kernel vs exact {e_kernel:.3e}, 16-bit kernel vs exact {rms(o16.double().cpu().numpy() - O):.3e}")
    # the kernel's own rounding (P to e4m3) adds less than the input quantization
    assert e_kernel_vs_fp8 < e_fp8 and e_kernel < 1.5 * e_fp8


def test_full_size_sampled():
    """The 8k-token, 32-head causal shape at batch 4: quantized on the GPU,
    rows of a few (batch, head) pairs compared with the oracle."""
    B, H, N, d = 4, 32, 8192, 128
    q, k, v, _ = workloads.make_inputs(B, H, H, N, d, "bf16", 1001)
    signs = workloads.make_signs(d, 1002)
    scale = 1 / math.sqrt(d)
    sd = signs.to(DEV)
    qc, qs = fa_fp8_quantize(q.to(DEV), sd)
    kc, ks = fa_fp8_quantize(k.to(DEV), sd)
    vc, vs = fa_fp8_quantize(v.to(DEV))
    o, lse = fa_fwd_fp8(qc, kc, vc, qs, ks, vs, True, scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 255, 256, 4095, 4096, 8000, 8191])
    for b, h in ((0, 0), (1, 17), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        f = lambda x: workloads.to_f64(x[sl])
        qq, kk, vv = (ofp8.quantize_blocks(f(x).astype(np.float32), BLK, s)
                      for x, s in ((q, signs.numpy()), (k, signs.numpy()), (v, None)))
        assert np.array_equal(qc[sl].cpu().numpy(), qq[0]) and np.array_equal(vs[sl].cpu().numpy(), vv[1])
        Qd, Kd, Vd = (ofp8.dequantize_blocks(c, s, BLK) for c, s in (qq, kk, vv))
        O, L = oracle.attention_forward(Qd, Kd, Vd, scale, True, rows=rows)
        got = o[sl][..., rows, :].double().cpu().numpy()
        # probabilities of the sampled rows (for the bound only)
        S = scale * (Qd[0, 0, rows] @ Kd[0, 0].T)
        S = np.where(np.arange(N)[None, :] <= rows[:, None], S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        bound = 2.0 ** -4 * (P @ np.abs(Vd[0, 0])) + 2.0 ** -8 * np.abs(O[0, 0]) + 2.0 ** -10 * np.abs(Vd).max()
        err = np.abs(got[0, 0] - O[0, 0])
        assert (err <= bound).all(), (b, h, err.max())
        assert np.abs(lse[sl][..., rows].double().cpu().numpy() - L).max() <= 1e-3


def test_deterministic_and_writes_only_outputs():
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 31)
    qc, qs = fa_fp8_quantize(q.to(DEV))
    kc, ks = fa_fp8_quantize(k.to(DEV))
    vc, vs = fa_fp8_quantize(v.to(DEV))
    guard = torch.full((q.numel() + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = guard[2048:2048 + q.numel()].view(q.shape)
    o1, l1 = fa_fwd_fp8(qc, kc, vc, qs, ks, vs, True, 0.09, o=o)
    o2, l2 = fa_fwd_fp8(qc, kc, vc, qs, ks, vs, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isnan(guard[:2048].float()).all() and torch.isnan(guard[2048 + q.numel():].float()).all()
