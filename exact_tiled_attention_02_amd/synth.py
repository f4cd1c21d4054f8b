"""Seeded synthetic inputs for attention workloads.

This module only draws random numbers and packs them into tensors; it holds none of the
attention arithmetic.  Both the fp64 oracle side and the HIP side of every test and
benchmark consume the same draws from here.

Recipe: ``numpy.random.default_rng(seed)``; draw order q, k, v, then dO (when asked
for), each ``standard_normal(shape, dtype=float32)``, then one round-to-nearest-even
cast to the 16-bit dtype (numpy for fp16, torch's CPU cast for bf16).  A varlen
workload first draws its per-sequence lengths, ``integers(lo, hi + 1, n)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """Shape of one attention call.  Padded when ``lengths_q`` is None, else varlen with
    the given per-sequence lengths (``batch`` = number of sequences, ``seqlen_q``/
    ``seqlen_k`` = maxima)."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int
    seqlen_k: int
    headdim: int
    dtype: str
    causal: bool
    backward: bool = False
    lengths_q: list | None = None
    lengths_k: list | None = None
    seed: int = 0
    scale: float | None = None
    extra: dict = field(default_factory=dict)

    @property
    def varlen(self) -> bool:
        return self.lengths_q is not None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.headdim)

    def pairs(self):
        """(len_q, len_k) per sequence."""
        if self.varlen:
            return list(zip(self.lengths_q, self.lengths_k))
        return [(self.seqlen_q, self.seqlen_k)] * self.batch


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "fp16":
        return torch.from_numpy(x.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype}")


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    """Per-sequence lengths drawn uniformly from the inclusive range [lo, hi]."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, n)]


def make_inputs(w: Workload, rng: np.random.Generator | None = None) -> dict:
    """Draw q, k, v (and dO when ``w.backward``) as 16-bit CPU tensors.

    Padded: q/do (B, Sq, Hq, D), k/v (B, Sk, Hkv, D).  Varlen: q/do (total_q, Hq, D),
    k/v (total_k, Hkv, D) plus int32 ``cu_seqlens_q``/``cu_seqlens_k`` of length B+1."""
    if rng is None:
        rng = np.random.default_rng(w.seed)
    D = w.headdim
    if w.varlen:
        tq, tk = int(sum(w.lengths_q)), int(sum(w.lengths_k))
        sq, sk = (tq, w.heads_q, D), (tk, w.heads_kv, D)
    else:
        sq = (w.batch, w.seqlen_q, w.heads_q, D)
        sk = (w.batch, w.seqlen_k, w.heads_kv, D)
    out = {}
    out["q"] = _cast(rng.standard_normal(sq, dtype=np.float32), w.dtype)
    out["k"] = _cast(rng.standard_normal(sk, dtype=np.float32), w.dtype)
    out["v"] = _cast(rng.standard_normal(sk, dtype=np.float32), w.dtype)
    if w.backward:
        out["do"] = _cast(rng.standard_normal(sq, dtype=np.float32), w.dtype)
    if w.varlen:
        out["cu_seqlens_q"] = torch.tensor(np.concatenate([[0], np.cumsum(w.lengths_q)]), dtype=torch.int32)
        out["cu_seqlens_k"] = torch.tensor(np.concatenate([[0], np.cumsum(w.lengths_k)]), dtype=torch.int32)
    return out


def config(n: int) -> Workload:
    """The five reference workloads; workload ``n`` is drawn with seed ``n``."""
    if n == 1:
        return Workload("fwd_noncausal_b1_h2_s128_d64_fp16", 1, 2, 2, 128, 128, 64, "fp16", False, seed=1)
    if n == 2:
        return Workload("fwd_causal_mha_b4_h16_s2048_d128_bf16", 4, 16, 16, 2048, 2048, 128, "bf16", True, seed=2)
    if n == 3:
        return Workload("fwd_causal_gqa_b2_hq32_hkv8_s8192_d128_bf16", 2, 32, 8, 8192, 8192, 128, "bf16", True, seed=3)
    if n == 4:
        lens = varlen_lengths(4, 16, 128, 4096)
        return Workload("fwd_causal_varlen_16seq_h8_d256_fp16", len(lens), 8, 8, max(lens), max(lens), 256, "fp16",
                        True, lengths_q=lens, lengths_k=list(lens), seed=4)
    if n == 5:
        return Workload("fwdbwd_causal_mha_b2_h16_s4096_d128_bf16", 2, 16, 16, 4096, 4096, 128, "bf16", True,
                        backward=True, seed=5)
    raise ValueError(f"no workload {n}")


def draw_config(n: int) -> tuple[Workload, dict]:
    """Workload ``n`` and its inputs.  For the varlen workload the lengths come from the
    same generator, drawn before q, k, v."""
    w = config(n)
    rng = np.random.default_rng(w.seed)
    if w.varlen:
        lens = [int(x) for x in rng.integers(128, 4097, 16)]
        assert lens == w.lengths_q
    return w, make_inputs(w, rng)


def flops(w: Workload) -> tuple[float, float]:
    """Algorithmic FLOPs (forward, backward): 4*Hq*Lq*Lk*D per sequence, halved when
    causal; backward is 2.5x forward.  Masked work and recomputation are not counted."""
    f = 0.0
    for lq, lk in w.pairs():
        f += 4.0 * w.heads_q * lq * lk * w.headdim
    if w.causal:
        f *= 0.5
    return f, 2.5 * f
