"""Forward pass on the GPU (through the C-ABI) against the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_attention_99_amd import fa_fwd

from .oracle_pins import load_golden, parse_exact
from .parity import TOL, check_fwd, errs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, Hq, Hkv, N, d, dtype, causal, seed):
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, dtype, seed)
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                    1.0 / math.sqrt(d), causal)
    return o, lse, O, L


SWEEP_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_sweep(dtype, d, causal):
    """Ragged N (partial tiles on both sides), MHA, GQA (G=4) and MQA (G=4, H_kv=1)."""
    seed = 10 + d + (100 if causal else 0)
    for N in SWEEP_N:
        for (Hq, Hkv) in ((2, 2), (4, 1), (8, 2)):
            print(f"case dtype={dtype} d={d} causal={causal} N={N} Hq={Hq} Hkv={Hkv}", flush=True)
            o, lse, O, L = _case(1, Hq, Hkv, N, d, dtype, causal, seed + N)
            check_fwd(o, lse, O, L, dtype, f"N={N} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_hand_examples(dtype):
    """The hand-worked examples, zero-padded to d = 64 (zero columns change no score)."""
    tdt = workloads.DTYPES[dtype]
    for c in load_golden():
        scale = parse_exact(c["scale"])
        Q, K, V = (np.asarray(c[x], dtype=np.float64) for x in ("Q", "K", "V"))
        N, dd = Q.shape

        def pad(x):
            y = np.zeros((1, 1, N, 64))
            y[0, 0, :, :x.shape[1]] = x
            return torch.tensor(y, dtype=tdt, device=DEV)

        o, lse = fa_fwd(pad(Q), pad(K), pad(V), c["causal"], scale)
        torch.cuda.synchronize()
        expO = np.zeros((1, 1, N, 64))
        expO[0, 0, :, :dd] = np.vectorize(parse_exact)(np.asarray(c["O"], dtype=object))
        explse = np.array([parse_exact(x) for x in c["lse"]])[None, None]
        check_fwd(o, lse, expO, explse, dtype, c["name"])


def _sample_rows(N, rng, k=48):
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(rng.choice(N, size=min(k, N), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size_workloads(name):
    """Every workload at its full size, in the default launch configuration; the
    oracle computes a sample of rows for a spread of heads (first, last, and a
    whole K/V group), each row exactly as the full result would have it."""
    w = workloads.WORKLOADS[name]
    q, k, v, _ = workloads.workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rng = np.random.default_rng(w.seed)
    G = w.H_q // w.H_kv
    for causal in w.causal_modes:
        print(f"workload {name} causal={causal}", flush=True)
        o, lse = fa_fwd(qd, kd, vd, causal, w.scale)
        torch.cuda.synchronize()
        heads = sorted(set([0, w.H_q - 1] + list(range(G, 2 * G if w.H_q >= 2 * G else G))))
        bs = sorted(set([0, w.B - 1]))
        rows = _sample_rows(w.N, rng)
        for b in bs:
            for h in heads:
                hk = h // G
                O, L = oracle.attention_forward(
                    workloads.to_f64(q[b:b + 1, h:h + 1]), workloads.to_f64(k[b:b + 1, hk:hk + 1]),
                    workloads.to_f64(v[b:b + 1, hk:hk + 1]), w.scale, causal, rows=rows)
                check_fwd(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], O, L, w.dtype,
                          f"{name} b={b} h={h}")
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("name", ["genome_gqa_64k", "llama_mha_8k", "gpt2_small"])
def test_closed_forms_full_size(name):
    """Q = 0: every visible key scores 0, so causal row i is the mean of V[0..i]
    and lse_i = ln(i + 1) (non-causal: mean of all V, ln N).  Checked on every row
    of every head at the full size."""
    w = workloads.WORKLOADS[name]
    _, k, v, _ = workloads.workload_inputs(w)
    q = torch.zeros((w.B, w.H_q, w.N, w.d), dtype=k.dtype)
    G = w.H_q // w.H_kv
    tol = TOL[w.dtype]
    for causal in w.causal_modes:
        o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, w.scale)
        torch.cuda.synchronize()
        vv = v.to(DEV).to(torch.float64)
        if causal:
            ref = torch.cumsum(vv, dim=2) / torch.arange(1, w.N + 1, device=DEV, dtype=torch.float64)[:, None]
            lref = torch.log(torch.arange(1, w.N + 1, device=DEV, dtype=torch.float64))
        else:
            ref = vv.mean(dim=2, keepdim=True).expand(-1, -1, w.N, -1)
            lref = torch.full((w.N,), math.log(w.N), device=DEV, dtype=torch.float64)
        ref = ref.repeat_interleave(G, dim=1)
        err = (o.to(torch.float64) - ref).abs()
        assert err.max().item() <= tol["o_max"], err.max().item()
        assert err.mean().item() <= tol["o_mean"]
        lerr = (lse.to(torch.float64) - lref).abs().max().item()
        assert lerr <= tol["lse_max"], lerr
        if causal:
            # row 0 sees only key 0: O_0 equals V_0 exactly (P = 1)
            assert torch.equal(o[:, :, 0], v.to(DEV).repeat_interleave(G, dim=1)[:, :, 0])


def test_deterministic_and_fully_written():
    """Two runs agree bitwise; NaN-poisoned outputs are fully overwritten; canary
    bytes around the outputs are untouched."""
    B, Hq, Hkv, N, d = 2, 4, 2, 333, 128
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "bf16", 77)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        pad = 4096
        obuf = torch.full((q.numel() + 2 * pad,), float("nan"), dtype=q.dtype, device=DEV)
        lbuf = torch.full((B * Hq * N + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
        obuf[:pad] = 7.0
        obuf[-pad:] = 7.0
        lbuf[:pad] = 7.0
        lbuf[-pad:] = 7.0
        o = obuf[pad:pad + q.numel()].view(q.shape)
        lse = lbuf[pad:pad + B * Hq * N].view(B, Hq, N)
        fa_fwd(q, k, v, causal, 0.09, o=o, lse=lse)
        o2, lse2 = fa_fwd(q, k, v, causal, 0.09)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        assert (obuf[:pad] == 7.0).all() and (obuf[-pad:] == 7.0).all()
        assert (lbuf[:pad] == 7.0).all() and (lbuf[-pad:] == 7.0).all()


def test_non_default_stream():
    B, Hq, Hkv, N, d = 1, 2, 2, 500, 64
    q, k, v, _ = workloads.make_inputs(B, Hq, Hkv, N, d, "fp16", 5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa_fwd(qd, kd, vd, True, 0.125, stream=s)
    s.synchronize()
    O, L = oracle.attention_forward(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                    0.125, True)
    check_fwd(o, lse, O, L, "fp16")


@pytest.mark.parametrize("scale", [1e-3, 0.5, 2.0])
def test_scale_values(scale):
    """Other positive scales, including ones large enough that the running max
    moves often and by large steps."""
    q, k, v, _ = workloads.make_inputs(1, 2, 1, 700, 128, "bf16", 99)
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                    scale, True)
    # the 16-bit tolerances at every scale: the lse is an fp32 sum of exponentials
    # of fp32 scores (relative error ~1e-6 of its magnitude, which grows with
    # the scale to about 10^2 here), far below the 1e-3 bound
    check_fwd(o, lse, O, L, "bf16", f"scale={scale}")


@pytest.mark.parametrize("pattern", ["rising", "falling", "huge_first"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_running_max_paths(pattern, causal, d):
    """Score patterns that drive every path of the online softmax's running
    maximum: scores that rise along the keys (the maximum moves by more than
    the lazy-rescale threshold in every 32-key block), scores that fall (later
    probabilities underflow to zero against the first block's maximum), and a
    first block whose raw scores would overflow exp2 without the maximum."""
    N, H = 1000, 2
    g = torch.Generator().manual_seed(7 + d)
    q = torch.zeros(1, H, N, d)
    q[..., 0] = 1.0
    q[..., 1:] = 0.05 * torch.randn(1, H, N, d - 1, generator=g)
    j = torch.arange(N, dtype=torch.float32)
    k = 0.05 * torch.randn(1, H, N, d, generator=g)
    k[..., 0] = {"rising": 0.5 * j, "falling": -0.5 * j, "huge_first": 300.0 - 0.5 * j}[pattern]
    v = torch.randn(1, H, N, d, generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, 1.0)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                    1.0, causal)
    check_fwd(o, lse, O, L, "bf16", f"{pattern} causal={causal} d={d}")
