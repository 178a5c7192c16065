"""Seeded synthetic attention inputs and the named workload shapes.

This module is shared by the fp64 oracle side and the HIP side of every test
and benchmark, so it holds no attention arithmetic at all: it only fixes
shapes, seeds and the order in which the i.i.d. N(0, 1) tensors are drawn.

Draw order for one workload: Q, K, V and then dO, each as float32 N(0, 1)
from one ``torch.Generator`` seeded with the workload's seed, then cast to the
workload dtype with round-to-nearest-even (torch's ``.to``).  The values the
GPU receives are exactly these dtype values; the oracle receives the same
values upcast (exactly) to float64.

Shapes follow the layout of the pages' PyTorch example (``[batch, heads,
seq_len, head_dim]``, page "Flash Attention" (21medien), section "Code
Example"): Q, O, dO, dQ are ``[B, H_q, N, d]`` and K, V, dK, dV are
``[B, H_kv, N, d]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    d: int
    dtype: str
    causal_modes: Tuple[bool, ...]
    passes: Tuple[str, ...]  # subset of ("fwd", "bwd")
    seed: int
    note: str

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops_fwd(self, causal: bool) -> float:
        """4*B*H_q*N^2*d matmul FLOPs (QK^T and PV), halved for a causal mask."""
        f = 4.0 * self.B * self.H_q * self.N * self.N * self.d
        return f / 2 if causal else f

    def flops_bwd(self, causal: bool) -> float:
        """The backward pass runs five N x N x d products: 2.5x the forward."""
        return 2.5 * self.flops_fwd(causal)


# The five workloads.  Sizes come from the pages' examples:
#  * single_head_fp32: a one-head case small enough for a brute-force check.
#  * gpt2_small: the B = 16, H = 12, N = 2048 example of the Performance
#    Benchmarks section ("Flash Attention", 21medien), head_dim 64 as in that
#    page's code example.
#  * llama_mha_8k: 32 heads x 128 = hidden 4096 of the Llama-2-7b example and
#    the [4, 8192, .] input of the same page's training example.
#  * genome_gqa_64k: a single-GPU context window of more than 64k tokens,
#    the whole-genome case of the "FlashAttention Kernel" glossary page, with
#    grouped K/V heads (GQA).
#  * train_bwd_16k: the 16K-token training case ("Performance Benchmarks";
#    initnode section 1 uses N = 16,384).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("single_head_fp32", 1, 1, 1, 256, 64, "fp32", (False,), ("fwd",), 1001,
                 "single-head forward, fp32, non-causal"),
        Workload("gpt2_small", 16, 12, 12, 2048, 64, "bf16", (False, True), ("fwd",), 1002,
                 "GPT-2-small-shaped forward, both masks"),
        Workload("llama_mha_8k", 4, 32, 32, 8192, 128, "bf16", (True,), ("fwd", "bwd"), 1003,
                 "Llama-style causal MHA, forward and backward"),
        Workload("genome_gqa_64k", 1, 32, 8, 65536, 128, "bf16", (True,), ("fwd",), 1004,
                 "long-context GQA causal forward (4 query heads per K/V head)"),
        Workload("train_bwd_16k", 2, 16, 16, 16384, 128, "bf16", (True,), ("fwd", "bwd"), 1005,
                 "training-shaped causal backward"),
    ]
}


def make_inputs(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str, seed: int,
                with_dout: bool = False, device: str = "cpu",
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Draw Q, K, V (and dO) as described in the module docstring.

    ``device`` selects where the generator runs.  CPU draws are the canonical
    (machine-independent) values; device draws are only used where the whole
    tensor never has to meet the oracle.
    """
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = DTYPES[dtype]

    def draw(h: int) -> torch.Tensor:
        x = torch.randn((B, h, N, d), generator=g, dtype=torch.float32, device=device)
        return x.to(t)

    q = draw(H_q)
    k = draw(H_kv)
    v = draw(H_kv)
    do = draw(H_q) if with_dout else None
    return q, k, v, do


def workload_inputs(w: Workload, with_dout: bool = False, device: str = "cpu"):
    return make_inputs(w.B, w.H_q, w.H_kv, w.N, w.d, w.dtype, w.seed, with_dout, device)


def to_f64(x: torch.Tensor):
    """Exact upcast of a dtype tensor to a float64 numpy array (for the oracle)."""
    return x.detach().to("cpu").to(torch.float64).numpy()


# --------------------------------------------------------------------------
# Split-KV (decoding) shapes: a few query rows against a long key/value
# sequence ("FlashAttention" glossary, FlashDecoding paragraph).  The key/value
# sequences are those of the long-context workloads above; the query counts
# are one new token per sequence and an eight-token chunk.

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H_q: int
    H_kv: int
    N_q: int
    N_kv: int
    d: int
    dtype: str
    causal: bool
    seed: int

    def kv_bytes(self) -> int:
        """K and V bytes one pass must read."""
        return 2 * self.B * self.H_kv * self.N_kv * self.d * (4 if self.dtype == "fp32" else 2)


DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    w.name: w for w in (
        DecodeWorkload("genome_gqa_64k_decode", 1, 32, 8, 1, 65536, 128, "bf16", True, 1006),
        DecodeWorkload("genome_gqa_64k_chunk8", 1, 32, 8, 8, 65536, 128, "bf16", True, 1007),
        DecodeWorkload("llama_mha_8k_decode", 4, 32, 32, 1, 8192, 128, "bf16", True, 1008),
    )
}


def make_decode_inputs(B: int, H_q: int, H_kv: int, N_q: int, N_kv: int, d: int, dtype: str,
                       seed: int, device: str = "cpu"):
    """Q [B, H_q, N_q, d], then K and V [B, H_kv, N_kv, d]: fp32 N(0, 1) draws
    from one seeded generator, cast to the dtype (round to nearest even)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = DTYPES[dtype]

    def draw(h: int, n: int) -> torch.Tensor:
        return torch.randn((B, h, n, d), generator=g, dtype=torch.float32, device=device).to(t)

    q = draw(H_q, N_q)
    k = draw(H_kv, N_kv)
    v = draw(H_kv, N_kv)
    return q, k, v


# --------------------------------------------------------------------------
# FP8 forward inputs.  Block quantization with an incoherent-processing
# rotation ("FlashAttention" glossary, FlashAttention-3 paragraph: FP8 with
# block quantization and incoherent processing) matters most when a few
# entries are far larger than the rest.  The outlier recipe: i.i.d. N(0, 1)
# entries, plus, at a Bernoulli(p) subset of positions, an extra N(0, s^2)
# term; then cast to the dtype.  The rotation's random +-1 signs are drawn
# here too, so both sides receive them as inputs.

def make_outlier_inputs(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str, seed: int,
                        p: float = 1e-3, s: float = 10.0, device: str = "cpu"):
    """Q, K, V as in ``make_inputs`` with outliers added (draw order: Q, K, V
    bases, then for each of Q, K, V a uniform mask draw and an N(0, 1) draw)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shapes = [(B, H_q, N, d), (B, H_kv, N, d), (B, H_kv, N, d)]
    base = [torch.randn(sh, generator=g, dtype=torch.float32, device=device) for sh in shapes]
    out = []
    for x, sh in zip(base, shapes):
        mask = torch.rand(sh, generator=g, dtype=torch.float32, device=device) < p
        extra = torch.randn(sh, generator=g, dtype=torch.float32, device=device) * s
        out.append((x + mask * extra).to(DTYPES[dtype]))
    return tuple(out)


def make_signs(d: int, seed: int) -> torch.Tensor:
    """d random signs (+1.0 / -1.0, float32) for the rotation."""
    g = torch.Generator()
    g.manual_seed(seed)
    return torch.randint(0, 2, (d,), generator=g).to(torch.float32) * 2 - 1


# --------------------------------------------------------------------------
# Block masks for block-sparse attention ("FlashAttention and the Kernel
# Era", The Breakthrough: the block-sparse extension), one entry per 128 x 128
# block.  Random masks: i.i.d. Bernoulli(density) blocks, the diagonal blocks
# set when `diag` (so that no row is empty under the causal mask).  Band
# masks: a local window of `width` blocks at and below the diagonal plus the
# first `globals_` key blocks for every row (a long-context pattern).

def make_block_mask(heads: int, N: int, density: float, seed: int, diag: bool = True,
                    blk: int = 128) -> torch.Tensor:
    nb = (N + blk - 1) // blk
    g = torch.Generator()
    g.manual_seed(seed)
    m = (torch.rand((heads, nb, nb), generator=g) < density).to(torch.uint8)
    if diag:
        idx = torch.arange(nb)
        m[:, idx, idx] = 1
    return m


def make_band_mask(N: int, width: int, globals_: int, blk: int = 128) -> torch.Tensor:
    nb = (N + blk - 1) // blk
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    m = ((j <= i) & (j > i - width)) | (j < globals_)
    return m.to(torch.uint8)[None]
