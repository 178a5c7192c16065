"""Tolerances and comparison helpers for GPU-vs-oracle parity.

Tolerances are absolute elementwise errors against the fp64 oracle:
  * bf16 / fp16 inputs: O max <= 2e-2 and mean <= 2e-3; dQ, dK, dV max <= 5e-2;
  * fp32 inputs: every output max <= 1e-4;
  * the logsumexp (no stated figure): <= 1e-3 for 16-bit inputs, 1e-4 for fp32.
The 16-bit figures cover bf16 rounding of P before the PV product and of the
outputs (relative 2^-8 on values of order 1), with fp32 accumulation.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {
    "bf16": {"o_max": 2e-2, "o_mean": 2e-3, "lse_max": 1e-3, "grad_max": 5e-2},
    "fp16": {"o_max": 2e-2, "o_mean": 2e-3, "lse_max": 1e-3, "grad_max": 5e-2},
    "fp32": {"o_max": 1e-4, "o_mean": 1e-4, "lse_max": 1e-4, "grad_max": 1e-4},
}


def errs(got: torch.Tensor, ref: np.ndarray):
    g = got.detach().to("cpu").to(torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    d = np.abs(g - ref)
    if not np.isfinite(g).all():
        return float("inf"), float("inf")
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def check_fwd(o, lse, O_ref, lse_ref, dtype: str, what: str = ""):
    t = TOL[dtype]
    omax, omean = errs(o, O_ref)
    lmax, _ = errs(lse, lse_ref)
    assert omax <= t["o_max"], f"{what} O max err {omax:.3e} > {t['o_max']}"
    assert omean <= t["o_mean"], f"{what} O mean err {omean:.3e} > {t['o_mean']}"
    assert lmax <= t["lse_max"], f"{what} lse max err {lmax:.3e} > {t['lse_max']}"
    return omax, omean, lmax


def check_grads(dq, dk, dv, dQ_ref, dK_ref, dV_ref, dtype: str, what: str = ""):
    t = TOL[dtype]
    out = {}
    for name, g, r in (("dQ", dq, dQ_ref), ("dK", dk, dK_ref), ("dV", dv, dV_ref)):
        mx, mean = errs(g, r)
        out[name] = (mx, mean)
        assert mx <= t["grad_max"], f"{what} {name} max err {mx:.3e} > {t['grad_max']}"
    return out
