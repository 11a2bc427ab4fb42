"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the attention method: it only draws random
tensors and packed-sample boundaries.  Both the HIP path's tests/benchmark and
the CPU oracle take their inputs from here, so the two sides see the same bits.

Recipe: for workload k (1-based), Q, K and V are drawn with
``torch.randn(shape, dtype=float32, generator=Generator('cpu').manual_seed(1000*k + i))``
for i = 1, 2, 3, then cast to bfloat16 (round to nearest even) unless the
workload is float32.  Packed-sample lengths for the variable-length workload
are log-uniform in [512, 16384] drawn with ``numpy.random.default_rng(5004)``
until the running sum reaches S; the last sample is cut to fit.  For the
per-sample split every length is rounded down to a multiple of 2 cp first.

The shapes follow the pages' Llama-style long-context workloads (32 query
heads, 8 KV heads for GQA, head dim 128); no dataset is involved.
"""
from dataclasses import dataclass
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based; fixes the seeds
    B: int
    S: int
    H: int
    Hkv: int
    D: int
    dtype: str          # "bf16" or "fp32"
    rd: int             # ring degree (cp)
    ud: int             # Ulysses degree
    packed: bool = False

    @property
    def chunk(self):
        return self.S // (2 * self.rd)

    @property
    def share(self):
        """Tokens of one ring rank's share (before the Ulysses split)."""
        return self.S // self.rd

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_causal_mha_fp32_s256_cp4", 1, 1, 256, 2, 2, 64, "fp32", 4, 1),
        Workload("causal_mha_s8k_cp4", 2, 1, 8192, 32, 32, 128, "bf16", 4, 1),
        Workload("causal_gqa_s32k_cp8", 3, 1, 32768, 32, 8, 128, "bf16", 8, 1),
        Workload("usp_hybrid_s128k_ud2_rd4", 4, 1, 131072, 32, 8, 128, "bf16", 4, 2),
        Workload("packed_varlen_s32k_cp4", 5, 1, 32768, 32, 8, 128, "bf16", 4, 1, packed=True),
    ]
}


def torch_dtype(dtype):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def randn(shape, seed, dtype="bf16"):
    """Seeded N(0, 1) CPU tensor, cast to ``dtype`` (bf16 by round to nearest even)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), dtype=torch.float32, generator=g)
    return x if dtype == "fp32" else x.to(torch_dtype(dtype))


def qkv(B, S, H, Hkv, D, dtype="bf16", seed_base=0):
    """(Q, K, V) CPU tensors in the [batch, seq, heads, head_dim] layout."""
    return (randn((B, S, H, D), seed_base + 1, dtype),
            randn((B, S, Hkv, D), seed_base + 2, dtype),
            randn((B, S, Hkv, D), seed_base + 3, dtype))


def workload_qkv(w):
    return qkv(w.B, w.S, w.H, w.Hkv, w.D, w.dtype, 1000 * w.index)


def packed_cu_seqlens(S, seed=5004, lo=512, hi=16384, multiple=1):
    """Boundaries (int32, n+1 entries from 0 to S) of samples with lengths
    log-uniform in [lo, hi], drawn until they cover S; the last is cut.
    ``multiple``: every length is rounded down to a multiple of it (at least
    one multiple), as a split of each sample into equal chunks needs; S must
    divide by it.  multiple = 1 draws exactly the unrounded lengths."""
    if S % multiple:
        raise ValueError("S must divide by multiple")
    rng = np.random.default_rng(seed)
    bounds = [0]
    while bounds[-1] < S:
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = max(multiple, n - n % multiple)
        bounds.append(min(S, bounds[-1] + n))
    return np.asarray(bounds, dtype=np.int32)


def workload_cu_seqlens(w, multiple=1):
    return packed_cu_seqlens(w.S, seed=1000 * w.index + 4, multiple=multiple) if w.packed else None
