#!/usr/bin/env python3
"""Throughput of exact tiled attention (forward + backward) on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
the forward kernel (O and the row logsumexp) followed by the three backward
phases (row terms D, dK/dV, dQ), on the Llama-style causal workload
B = 4, H = 32, N = 8192, d = 128, bf16 (Q, K, V, dO ~ N(0, 1), seeded).

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  `value` is the whole-step rate in TFLOP/s with the
conventional count: forward 4*B*H*N^2*d (halved under the causal mask) plus
backward 2.5x that.  Inputs are resident in HBM before the timed region.
Per-kernel durations come from HIP events recorded on the stream the kernels
run on, around every launch inside the timed region.  After it, every kernel
is also timed cold (each launch preceded by an untimed 512 MB fill that evicts
L2 and the MALL), reported as median and minimum per kernel.

The CPU baseline (`cpu_baseline`: the fp64 oracle, one process per host core)
runs first, before the GPU is touched.  `configs` holds every workload in each
of its masks and passes (forward; forward and backward where the workload has
one): times, TFLOP/s and % of the matrix-core peak.  Outside the timed steps
every call is timed as the per-call share of a batch of back-to-back launches
between two events (the host runs ahead of the GPU, as in the timed steps and
in a loop of calls, so no host launch latency is counted); the split-KV
records also give the isolated-call time (`ms_single_call`, launch latency
included).

Further objects in the same line: `splitkv` (the split-KV forward on
decoding shapes, K/V bytes per second against the HBM peak), `dropout` (the
forward and backward with fused dropout, p = 0.1, on the same workload),
`blocksparse` and `varlen` (the same workload under a band block mask, and
with per-sequence lengths N, 3N/4, N/2, N/4; rates over the valid elements) and
`fp8` (the block quantizer and the e4m3 forward on the same workload, against
the fp8 matrix-core peak).  `--splitkv-only NAME`, `--dropout-only`,
`--blocksparse-only` and `--fp8-only` run just those, for profiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOPS (bf16, causal, d=128) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 1 << 30        # size of the counter-calibration copy
FLUSH_BYTES = 512 << 20     # cache-evicting fill before each cold-timed launch


def source_sha() -> str:
    """Hash of the kernel sources: ties stored counter readings to a kernel version."""
    csrc = os.path.join(ROOT, "exact_attention_99_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        k = rec["kernels"][kernel]
        if rec.get("source_sha") != source_sha():
            return None
        return float(k["hbm_bytes_per_launch"])
    except (KeyError, ValueError, TypeError):
        return None


def cpu_model() -> str:
    """CPU model name of the host (from /proc/cpuinfo, else lscpu)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def _oracle_task(task):
    """One unit of the CPU baseline, in a worker process: the fp64 oracle on
    one head (or one slice of query rows of one head) of a workload's shape,
    inputs drawn as seeded N(0, 1) float64 values.  Returns (tag, seconds)."""
    import numpy as np
    import oracle
    tag, N, d, causal, scale, what, seed, rows = task
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    t0 = time.perf_counter()
    if what == "fwd":
        oracle.attention_forward(Q, K, V, scale, causal,
                                 rows=None if rows is None else np.arange(rows[0], rows[1]))
    else:   # forward and backward (the backward recomputes O and lse first)
        oracle.attention_backward(Q, K, V, dO, scale, causal)
    return tag, time.perf_counter() - t0


def _worker_init():
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def cpu_baseline(headline: str, max_workers: int = 16):
    """The fp64 oracle as it stands, timed on the host cores with one process
    per core (BLAS at one thread each), before the GPU is touched.

    GPT-2-small (both masks) and the single-head fp32 case are timed in full.
    The larger workloads are timed on a fixed sample and scaled to the whole
    workload (labelled "extrapolated"): whole heads (forward + backward) of the
    8k and 16k workloads, scaled by the head count; slices of 128 query rows of
    the 64k workload (the oracle's cost per row does not depend on the row,
    since it forms every score of the row before masking), scaled by the row
    count.  Each rate uses the conventional FLOPs of the full workload."""
    import multiprocessing as mp
    import workloads
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    tasks, plan = [], {}
    for name, w in workloads.WORKLOADS.items():
        for causal in w.causal_modes:
            tag = f"{name}|{'causal' if causal else 'full'}"
            what = "fwd+bwd" if "bwd" in w.passes else "fwd"
            if name in ("single_head_fp32", "gpt2_small"):
                heads = w.B * w.H_q
                tasks += [(tag, w.N, w.d, causal, w.scale, what, 10 * w.seed + i, None) for i in range(heads)]
                plan[tag] = (w, causal, what, 1.0, f"all {heads} heads", heads, w.N)
            elif name == "genome_gqa_64k":
                rows = 128
                starts = [int(w.N * (i + 0.5) / workers) // rows * rows for i in range(workers)]
                tasks += [(tag, w.N, w.d, causal, w.scale, what, 10 * w.seed + i, (r0, r0 + rows))
                          for i, r0 in enumerate(starts)]
                total_rows = w.B * w.H_q * w.N
                plan[tag] = (w, causal, what, total_rows / (rows * workers),
                             f"{workers} slices of {rows} rows spread over one head, "
                             f"scaled to {total_rows} rows (extrapolated)", workers, rows)
            else:
                n = workers if name == "llama_mha_8k" else max(1, workers // 2)
                tasks += [(tag, w.N, w.d, causal, w.scale, what, 10 * w.seed + i, None) for i in range(n)]
                heads = w.B * w.H_q
                plan[tag] = (w, causal, what, heads / n,
                             f"{n} whole heads, scaled to {heads} heads (extrapolated)", n, w.N)
    # longest tasks first (list scheduling over the pool)
    # cost of one task ~ rows x keys (x 3 with the backward)
    cost = {tag: rows * w.N * (3.0 if what != "fwd" else 1.0)
            for tag, (w, causal, what, _, _, _, rows) in plan.items()}
    tasks.sort(key=lambda t: -cost[t[0]])
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    t0 = time.perf_counter()
    try:
        with mp.get_context("spawn").Pool(workers, initializer=_worker_init) as pool:
            results = pool.map(_oracle_task, tasks, chunksize=1)
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    wall = time.perf_counter() - t0
    secs = {}
    for tag, t in results:
        secs[tag] = secs.get(tag, 0.0) + t
    configs = []
    head_rate = None
    for tag, (w, causal, what, factor, how, ntask, _) in plan.items():
        flops = w.flops_fwd(causal) + (w.flops_bwd(causal) if what != "fwd" else 0.0)
        # process-seconds of the sample, scaled to the whole workload and shared
        # by the pool's processes (a workload of fewer units than processes
        # cannot use them all)
        t_full = secs[tag] * factor / min(workers, ntask * factor)
        rate = flops / t_full / 1e12
        configs.append({"workload": w.name, "causal": causal, "pass": what, "sample": how,
                        "cpu_seconds_sample": secs[tag], "seconds_full_on_pool": t_full,
                        "tflops": rate})
        if w.name == headline and causal:
            head_rate = rate
    return {"value": head_rate, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"fp64 NumPy oracle, one process per core ({workers} processes, BLAS at 1 "
                       f"thread each), seeded N(0,1) inputs of each workload's per-head shape; "
                       f"value = {headline} causal forward+backward: conventional FLOPs of the "
                       f"whole workload / its time scaled from {workers} whole heads; "
                       f"pool wall time {wall:.1f} s for all configs"),
            "wall_seconds": wall, "configs": configs}


def measure_splitkv(dw, dev, stream, iters: int = 20, one_chunk: bool = True):
    """Split-KV forward on a decoding shape: median time of the whole call
    (chunk kernel + merge) per call of back-to-back calls (time_calls), K/V
    bytes per second against the HBM peak, the same call with a single chunk
    for comparison, and the median of isolated calls (host launch latency
    included)."""
    import torch
    import workloads
    from exact_attention_99_amd import fa_fwd_splitkv, fa_fwd_splitkv_default_splits, fa_fwd_splitkv_workspace_size
    q, k, v = workloads.make_decode_inputs(dw.B, dw.H_q, dw.H_kv, dw.N_q, dw.N_kv, dw.d, dw.dtype,
                                           dw.seed, device=dev)
    scale = 1.0 / math.sqrt(dw.d)
    o = torch.empty_like(q)
    lse = torch.empty((dw.B, dw.H_q, dw.N_q), dtype=torch.float32, device=dev)

    def timed(splits):
        ws = torch.empty(fa_fwd_splitkv_workspace_size(dw.B, dw.H_q, dw.N_q, dw.d, splits),
                         dtype=torch.uint8, device=dev)
        def call():
            fa_fwd_splitkv(q, k, v, dw.causal, scale, splits, o=o, lse=lse, workspace=ws, stream=stream)
        ts = time_calls(call, stream, iters, warmup=3)
        single = time_single(call, stream, iters)
        return ts[len(ts) // 2], ts[0], single[len(single) // 2]

    splits = fa_fwd_splitkv_default_splits(dw.B, dw.H_q, dw.H_kv, dw.N_q, dw.N_kv, dw.d)
    med, mn, single = timed(splits)
    one = timed(1)[0] if one_chunk else None
    gbs = dw.kv_bytes() / (med * 1e-3) / 1e9
    return {"workload": dw.name, "B": dw.B, "H_q": dw.H_q, "H_kv": dw.H_kv, "N_q": dw.N_q,
            "N_kv": dw.N_kv, "d": dw.d, "causal": dw.causal, "splits": splits,
            "ms_median": med, "ms_min": mn, "ms_single_call": single, "kv_bytes": dw.kv_bytes(),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS},
            "ms_one_chunk": one}


def measure_fp8(w, q, k, v, stream, iters: int = 20):
    """FP8 forward on the workload's own Q, K, V: block quantization of Q and K
    (with the rotation) and of V, then the e4m3 forward.  Median per-call time
    of each kernel (time_calls), warm."""
    import torch
    import workloads
    from exact_attention_99_amd import fa_fp8_quantize, fa_fwd_fp8
    causal = True in w.causal_modes
    signs = workloads.make_signs(w.d, w.seed + 1).to(q.device)
    qc, qs = fa_fp8_quantize(q, signs, stream=stream)
    kc, ks = fa_fp8_quantize(k, signs, stream=stream)
    vc, vs = fa_fp8_quantize(v, stream=stream)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=q.device)
    launches = {
        "quant_q": lambda: fa_fp8_quantize(q, signs, codes=qc, scales=qs, stream=stream),
        "quant_k": lambda: fa_fp8_quantize(k, signs, codes=kc, scales=ks, stream=stream),
        "quant_v": lambda: fa_fp8_quantize(v, codes=vc, scales=vs, stream=stream),
        "fwd_fp8": lambda: fa_fwd_fp8(qc, kc, vc, qs, ks, vs, causal, w.scale, o=o, lse=lse, stream=stream),
    }
    med = {}
    for name, fn in launches.items():
        ts = time_calls(fn, stream, iters, warmup=3)
        med[name] = ts[len(ts) // 2]
    F = w.flops_fwd(causal)
    tf = F / (med["fwd_fp8"] * 1e-3) / 1e12
    # quantizer traffic per tensor: 2-byte reads, 1-byte codes, one float per 64 rows
    def qbytes(h):
        n = w.B * h * w.N * w.d
        return 3.0 * n + 4.0 * w.B * h * ((w.N + 63) // 64)
    quant_bytes = qbytes(w.H_q) + 2 * qbytes(w.H_kv)
    quant_ms = med["quant_q"] + med["quant_k"] + med["quant_v"]
    gbs = quant_bytes / (quant_ms * 1e-3) / 1e9
    return {"workload": w.name, "causal": causal, "out_dtype": "bf16", "block_rows": 64,
            "rotation": "Q and K", "kernels_ms": med,
            "fwd_fp8": {"ms": med["fwd_fp8"], "tflops": tf,
                        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS,
                                     "unit": "TFLOP/s", "frac": tf / PEAK_FP8_TFLOPS,
                                     "traffic": stored_traffic("fwd_fp8")}},
            "quantize": {"ms": quant_ms, "bytes": quant_bytes,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "traffic_per_launch": stored_traffic("fp8_quantize")}},
            "path_ms": quant_ms + med["fwd_fp8"],
            "path_tflops": F / ((quant_ms + med["fwd_fp8"]) * 1e-3) / 1e12}


def measure_dropout(w, q, k, v, do, stream, p: float = 0.1, iters: int = 10):
    """Forward and backward with fused dropout (probability p) on the
    workload's tensors: median per-call durations (time_calls), and the
    rate with the same conventional FLOP count as the step without dropout."""
    import torch
    from exact_attention_99_amd import fa_bwd_dropout, fa_bwd_workspace_size, fa_fwd_dropout
    causal = True in w.causal_modes
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa_bwd_workspace_size(w.B, w.H_q, w.H_kv, w.N, w.d, w.dtype), 256),
                     dtype=torch.uint8, device=q.device)
    calls = {
        "fwd_dropout": lambda: fa_fwd_dropout(q, k, v, causal, w.scale, p, 1234, 0, o=o, lse=lse, stream=stream),
        "bwd_dropout": lambda: fa_bwd_dropout(q, k, v, o, lse, do, causal, w.scale, p, 1234, 0,
                                              dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream),
    }
    med = {}
    for name, fn in calls.items():
        ts = time_calls(fn, stream, iters)
        med[name] = ts[len(ts) // 2]
    F = w.flops_fwd(causal)
    Fb = w.flops_bwd(causal)
    return {"workload": w.name, "dropout_p": p, "causal": causal,
            "fwd_ms": med["fwd_dropout"], "bwd_ms": med["bwd_dropout"],
            "fwd_tflops": F / (med["fwd_dropout"] * 1e-3) / 1e12,
            "bwd_tflops": Fb / (med["bwd_dropout"] * 1e-3) / 1e12,
            "step_tflops": (F + Fb) / ((med["fwd_dropout"] + med["bwd_dropout"]) * 1e-3) / 1e12}


def measure_blocksparse(w, q, k, v, do, stream, width: int = 4, globals_: int = 1, iters: int = 10):
    """Forward and backward under a block mask (a local band of `width`
    128-key blocks plus the first `globals_` key blocks, with the workload's
    causal mask): median per-call durations (time_calls), and rates over the FLOPs of
    the visible elements only (4 d per visible score forward, 2.5x that
    backward)."""
    import torch
    import workloads
    from exact_attention_99_amd import fa_bwd_blocksparse, fa_bwd_workspace_size, fa_fwd_blocksparse
    causal = True in w.causal_modes
    M = workloads.make_band_mask(w.N, width, globals_).to(q.device)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa_bwd_workspace_size(w.B, w.H_q, w.H_kv, w.N, w.d, w.dtype), 256),
                     dtype=torch.uint8, device=q.device)
    calls = {
        "fwd": lambda: fa_fwd_blocksparse(q, k, v, M, causal, w.scale, o=o, lse=lse, stream=stream),
        "bwd": lambda: fa_bwd_blocksparse(q, k, v, o, lse, do, M, causal, w.scale, dq=dq, dk=dk, dv=dv,
                                          workspace=ws, stream=stream),
    }
    med = {}
    for name, fn in calls.items():
        ts = time_calls(fn, stream, iters)
        med[name] = ts[len(ts) // 2]
    # visible (row, key) pairs of one head
    idx = torch.arange(w.N, device="cpu") // 128
    Mc = M[0].cpu().bool()
    vis = 0
    for r0 in range(0, w.N, 1024):
        rows = torch.arange(r0, min(w.N, r0 + 1024))
        allowed = Mc[idx[rows]][:, idx]
        if causal:
            allowed &= torch.arange(w.N)[None, :] <= rows[:, None]
        vis += int(allowed.sum())
    F = 4.0 * w.d * vis * w.B * w.H_q
    density = vis / (w.N * (w.N + 1) / 2 if causal else w.N * w.N)
    return {"workload": w.name, "mask": f"band of {width} blocks + {globals_} global key block(s)",
            "causal": causal, "visible_fraction": density, "fwd_ms": med["fwd"], "bwd_ms": med["bwd"],
            "fwd_tflops": F / (med["fwd"] * 1e-3) / 1e12,
            "bwd_tflops": 2.5 * F / (med["bwd"] * 1e-3) / 1e12}


def measure_varlen(w, q, k, v, do, stream, iters: int = 10):
    """Forward and backward of the workload's batch with per-sequence lengths
    N, 3N/4, N/2, N/4 (cycled over the batch): median per-call durations (time_calls),
    and rates over the FLOPs of the valid elements only."""
    import torch
    from exact_attention_99_amd import fa_bwd_varlen, fa_bwd_workspace_size, fa_fwd_varlen
    causal = True in w.causal_modes
    lens = [w.N * (4 - (b % 4)) // 4 for b in range(w.B)]
    sl = torch.tensor(lens, dtype=torch.int32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(fa_bwd_workspace_size(w.B, w.H_q, w.H_kv, w.N, w.d, w.dtype), 256),
                     dtype=torch.uint8, device=q.device)
    calls = {
        "fwd": lambda: fa_fwd_varlen(q, k, v, sl, causal, w.scale, o=o, lse=lse, stream=stream),
        "bwd": lambda: fa_bwd_varlen(q, k, v, o, lse, do, sl, causal, w.scale, dq=dq, dk=dk, dv=dv,
                                     workspace=ws, stream=stream),
    }
    med = {}
    for name, fn in calls.items():
        ts = time_calls(fn, stream, iters)
        med[name] = ts[len(ts) // 2]
    pairs = sum((n * (n + 1) / 2 if causal else n * n) for n in lens)
    F = 4.0 * w.d * pairs * w.H_q
    return {"workload": w.name, "lengths": lens, "causal": causal,
            "fwd_ms": med["fwd"], "bwd_ms": med["bwd"],
            "fwd_tflops": F / (med["fwd"] * 1e-3) / 1e12,
            "bwd_tflops": 2.5 * F / (med["bwd"] * 1e-3) / 1e12}


def time_calls(fn, stream, iters: int, warmup: int = 2):
    """Per-call GPU durations (ms, sorted) of fn on stream.  Each of the
    `iters` samples times a batch of back-to-back launches between two events
    and divides by the batch size, so the host runs ahead of the GPU as in a
    loop of calls (and as in the timed steps) and the figure holds no host
    launch latency.  The batch is sized from one isolated call to last about
    2 ms (1 call for calls of 2 ms and more, at most 50)."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    e1.synchronize()
    batch = max(1, min(50, int(2.0 / max(e0.elapsed_time(e1), 1e-3))))
    ts = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / batch)
    return sorted(ts)


def time_single(fn, stream, iters: int, warmup: int = 2):
    """Durations (ms, sorted) of isolated calls: one launch between two events
    on an idle GPU, host launch latency included."""
    import torch
    for _ in range(warmup):
        fn()
    ts = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)


PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak


def measure_configs(dev, stream):
    """Every workload in each of its masks and passes, in the default launch
    configuration, on device-drawn inputs of its shape: median and minimum
    per-call time (time_calls), TFLOP/s with the conventional count, and % of the
    matrix-core peak of the workload's type (bf16 2.5 PF; fp32 157.3 TF).
    The backward is fa_bwd's three phases, also timed one by one."""
    import torch
    import workloads
    from exact_attention_99_amd import fa_bwd_dkdv, fa_bwd_dq, fa_bwd_prepare, fa_fwd
    out = []
    for name, w in workloads.WORKLOADS.items():
        q, k, v, do = workloads.workload_inputs(w, with_dout="bwd" in w.passes, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=dev)
        peak = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS
        F0 = w.flops_fwd(False)
        iters = max(5, min(50, int(2e13 / F0)))
        for causal in w.causal_modes:
            base = {"workload": name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N": w.N, "d": w.d,
                    "dtype": w.dtype, "causal": causal}
            ts = time_calls(lambda: fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse, stream=stream),
                            stream, iters)
            F = w.flops_fwd(causal)
            tf = F / (ts[len(ts) // 2] * 1e-3) / 1e12
            out.append(dict(base, **{"pass": "fwd", "iters": iters, "ms_median": ts[len(ts) // 2],
                                     "ms_min": ts[0], "tflops": tf, "peak_tflops": peak,
                                     "pct_of_peak": 100.0 * tf / peak}))
            if "bwd" not in w.passes:
                continue
            delta = torch.empty_like(lse)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse, stream=stream)
            phases = {
                "bwd_prepare": lambda: fa_bwd_prepare(o, do, delta, stream=stream),
                "bwd_dkdv": lambda: fa_bwd_dkdv(q, k, v, lse, do, delta, causal, w.scale, dk=dk, dv=dv,
                                                stream=stream),
                "bwd_dq": lambda: fa_bwd_dq(q, k, v, lse, do, delta, causal, w.scale, dq=dq, stream=stream),
            }
            kms = {n: time_calls(fn, stream, iters)[iters // 2] for n, fn in phases.items()}

            def whole():
                for fn in phases.values():
                    fn()
            ts = time_calls(whole, stream, iters)
            Fb = w.flops_bwd(causal)
            tf = Fb / (ts[len(ts) // 2] * 1e-3) / 1e12
            out.append(dict(base, **{"pass": "bwd", "iters": iters, "ms_median": ts[len(ts) // 2],
                                     "ms_min": ts[0], "tflops": tf, "peak_tflops": peak,
                                     "pct_of_peak": 100.0 * tf / peak, "phases_ms": kms}))
        del q, k, v, do, o, lse
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_mha_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the per-workload measurements")
    ap.add_argument("--configs-only", action="store_true",
                    help="only measure every workload in each of its masks and passes")
    ap.add_argument("--no-splitkv", dest="splitkv", action="store_false",
                    help="skip the split-KV decoding measurements")
    ap.add_argument("--splitkv-only", default=None, metavar="DECODE_WORKLOAD",
                    help="only measure the split-KV forward on one decoding shape")
    ap.add_argument("--no-fp8", dest="fp8", action="store_false",
                    help="skip the FP8 forward measurement")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only measure the FP8 path (quantizer + e4m3 forward)")
    ap.add_argument("--no-dropout", dest="dropout", action="store_false",
                    help="skip the fused-dropout measurement")
    ap.add_argument("--dropout-only", action="store_true",
                    help="only measure the forward and backward with dropout")
    ap.add_argument("--no-blocksparse", dest="blocksparse", action="store_false",
                    help="skip the block-sparse measurement")
    ap.add_argument("--blocksparse-only", action="store_true",
                    help="only measure the forward and backward under a band block mask")
    ap.add_argument("--flush-iters", type=int, default=20,
                    help="cold-cache timed launches per kernel (0 to skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--print-sha", action="store_true", help="print the kernel source hash and exit")
    args = ap.parse_args()
    if args.print_sha:
        print(source_sha())
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the attention path here has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        return 2

    # The CPU baseline runs first, in worker processes started before this
    # process touches the GPU.
    cpu = None
    if not (args.no_cpu_baseline or args.copy_calibration or args.splitkv_only or args.fp8_only
            or args.blocksparse_only or args.dropout_only or args.configs_only):
        cpu = cpu_baseline(args.workload)

    import torch
    import workloads
    from exact_attention_99_amd import fa_bwd_dkdv, fa_bwd_dq, fa_bwd_prepare, fa_fwd

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES}))
        return 0
    if args.splitkv_only:
        torch.cuda.set_device(0)
        # the default chunk count only, so that a profile of this run sees one configuration
        rec = measure_splitkv(workloads.DECODE_WORKLOADS[args.splitkv_only], "cuda:0",
                              torch.cuda.current_stream(), one_chunk=False)
        print(json.dumps({"splitkv": rec}), flush=True)
        return 0
    if args.configs_only:
        torch.cuda.set_device(0)
        print(json.dumps({"configs": measure_configs("cuda:0", torch.cuda.current_stream())}), flush=True)
        return 0
    w = workloads.WORKLOADS[args.workload]
    causal = True in w.causal_modes
    dev = "cuda:0"
    torch.cuda.set_device(0)
    q, k, v, do = workloads.workload_inputs(w, with_dout=True, device=dev)
    if args.fp8_only:
        print(json.dumps({"fp8": measure_fp8(w, q, k, v, torch.cuda.current_stream())}), flush=True)
        return 0
    if args.blocksparse_only:
        st = torch.cuda.current_stream()
        print(json.dumps({"blocksparse": measure_blocksparse(w, q, k, v, do, st),
                          "varlen": measure_varlen(w, q, k, v, do, st)}), flush=True)
        return 0
    if args.dropout_only:
        print(json.dumps({"dropout": measure_dropout(w, q, k, v, do, torch.cuda.current_stream())}),
              flush=True)
        return 0
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    names = ["fwd", "bwd_prepare", "bwd_dkdv", "bwd_dq"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fa_bwd_prepare(o, do, delta, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        fa_bwd_dkdv(q, k, v, lse, do, delta, causal, w.scale, dk=dk, dv=dv, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        fa_bwd_dq(q, k, v, lse, do, delta, causal, w.scale, dq=dq, stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {n: 0.0 for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: t / args.steps for n, t in per.items()}  # ms per launch

    # Cold-cache timing: each kernel launched after an untimed 512 MB fill that
    # evicts L2 and the 256 MB MALL; median and minimum over the iterations.
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    launches = {
        "fwd": lambda: fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse, stream=stream),
        "bwd_prepare": lambda: fa_bwd_prepare(o, do, delta, stream=stream),
        "bwd_dkdv": lambda: fa_bwd_dkdv(q, k, v, lse, do, delta, causal, w.scale, dk=dk, dv=dv, stream=stream),
        "bwd_dq": lambda: fa_bwd_dq(q, k, v, lse, do, delta, causal, w.scale, dq=dq, stream=stream),
    }
    cold = {n: [] for n in names}
    for _ in range(args.flush_iters):
        for n in names:
            flush_buf.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launches[n]()
            e1.record(stream)
            e1.synchronize()
            cold[n].append(e0.elapsed_time(e1))
    del flush_buf

    F = w.flops_fwd(causal)
    step_flops = F + w.flops_bwd(causal)
    ms_step = wall / args.steps * 1e3
    value = step_flops / (ms_step * 1e-3) / 1e12
    # FLOPs each kernel performs by design (matrix products of N x N x d):
    # forward 2 (QK^T, PV), dK/dV pass 4 (QK^T, dO V^T, P^T dO, dS^T Q),
    # dQ pass 3 (K Q^T, V dO^T, dS K); the row-term pass moves bytes only.
    kflops = {"fwd": F, "bwd_dkdv": 2.0 * F, "bwd_dq": 1.5 * F, "bwd_prepare": 0.0}
    elem = 2
    kbytes = {"bwd_prepare": 2.0 * w.B * w.H_q * w.N * w.d * elem + 4.0 * w.B * w.H_q * w.N}
    dominant = max(per, key=per.get)
    if kflops[dominant] > 0:
        achieved = kflops[dominant] / (per[dominant] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = kbytes[dominant] / (per[dominant] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof["kernel"] = dominant
    roof["traffic"] = stored_traffic(dominant)

    kernels = {}
    for n in names:
        ts = sorted(cold[n])
        rec = {"ms": per[n]}
        if ts:
            rec["cold_median_ms"] = ts[len(ts) // 2]
            rec["cold_min_ms"] = ts[0]
        if kflops[n] > 0:
            rec["tflops"] = kflops[n] / (per[n] * 1e-3) / 1e12
        else:
            rec["gbs"] = kbytes[n] / (per[n] * 1e-3) / 1e9
        kernels[n] = rec
    fwd_ms = per["fwd"]
    bwd_ms = per["bwd_prepare"] + per["bwd_dkdv"] + per["bwd_dq"]

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N": w.N, "d": w.d,
                   "causal": causal, "step": "forward + backward"},
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": F / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": w.flops_bwd(causal) / (bwd_ms * 1e-3) / 1e12,
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.splitkv:
        out["splitkv"] = [measure_splitkv(workloads.DECODE_WORKLOADS[n], dev, stream)
                          for n in ("genome_gqa_64k_decode", "genome_gqa_64k_chunk8", "llama_mha_8k_decode")]
    if args.dropout:
        out["dropout"] = measure_dropout(w, q, k, v, do, stream)
    if args.blocksparse:
        out["blocksparse"] = measure_blocksparse(w, q, k, v, do, stream)
        out["varlen"] = measure_varlen(w, q, k, v, do, stream)
    if args.fp8:
        out["fp8"] = measure_fp8(w, q, k, v, stream)
        out["fp8"]["speedup_vs_16bit_fwd"] = fwd_ms / out["fp8"]["fwd_fp8"]["ms"]
    if args.configs:
        del q, k, v, do, o, lse, delta, dq, dk, dv
        torch.cuda.empty_cache()
        out["configs"] = measure_configs(dev, stream)
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
