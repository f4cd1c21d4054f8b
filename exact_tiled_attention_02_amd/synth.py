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
    window: tuple = (-1, -1)
    alibi: str | None = None  # None, "head" (Hq,) or "batch_head" (B, Hq) slopes

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


def alibi_slopes(rng: np.random.Generator, heads_q: int, batch: int, kind: str) -> torch.Tensor:
    """ALiBi slopes: the usual geometric schedule 2^(-8 (h+1) / Hq) times a uniform factor
    in [0.5, 1.5), one per query head ("head") or per (sequence, head) ("batch_head")."""
    base = 2.0 ** (-8.0 * (np.arange(heads_q) + 1) / heads_q)
    shape = (heads_q,) if kind == "head" else (batch, heads_q)
    return torch.tensor(base * rng.uniform(0.5, 1.5, shape), dtype=torch.float32)


def make_inputs(w: Workload, rng: np.random.Generator | None = None) -> dict:
    """Draw q, k, v (and dO when ``w.backward``, then ALiBi slopes when ``w.alibi``) as
    CPU tensors (16-bit data, fp32 slopes).

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
    if w.alibi is not None:
        out["alibi_slopes"] = alibi_slopes(rng, w.heads_q, w.batch, w.alibi)
    if w.varlen:
        out["cu_seqlens_q"] = torch.tensor(np.concatenate([[0], np.cumsum(w.lengths_q)]), dtype=torch.int32)
        out["cu_seqlens_k"] = torch.tensor(np.concatenate([[0], np.cumsum(w.lengths_k)]), dtype=torch.int32)
    return out


def make_inputs_on_device(w: Workload, device: str = "cuda", chunk_rows: int = 8192) -> dict:
    """Padded q, k, v (and dO when ``w.backward``) drawn on ``device`` itself, for tensors
    too large to draw on the host in reasonable time (K/V of several GiB).

    Recipe: one ``torch.Generator(device)`` seeded with ``w.seed``; draw order q, k, v,
    then dO; each tensor in slices of ``chunk_rows`` sequence positions (all batch
    entries and heads of a slice at once), each slice ``torch.randn(..., float32)`` cast
    once to the 16-bit dtype (round to nearest even).  The oracle side reads the same
    values back from the device."""
    if w.varlen:
        raise ValueError("device-side draws are for padded workloads")
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = DTYPES[w.dtype]
    D = w.headdim

    def draw(S, H):
        t = torch.empty((w.batch, S, H, D), dtype=dt, device=device)
        for s0 in range(0, S, chunk_rows):
            s1 = min(S, s0 + chunk_rows)
            t[:, s0:s1] = torch.randn((w.batch, s1 - s0, H, D), generator=g, dtype=torch.float32, device=device).to(dt)
        return t

    out = {"q": draw(w.seqlen_q, w.heads_q), "k": draw(w.seqlen_k, w.heads_kv), "v": draw(w.seqlen_k, w.heads_kv)}
    if w.backward:
        out["do"] = draw(w.seqlen_q, w.heads_q)
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


# ---------------------------------------------------------------------------- KV-cache decode

@dataclass
class KVCacheWorkload:
    """Attention of ``seqlen_q`` new query rows per sequence against a read-only KV cache.

    Contiguous cache (``page`` = 0): (cache_batch, capacity, Hkv, D).  Paged cache
    (``page`` > 0): a pool of ``cache_batch`` blocks of ``page`` rows; each sequence
    addresses ``capacity / page`` blocks through a block table.  ``lengths`` are the
    per-sequence cache lengths (None: every sequence uses the whole capacity);
    ``batch_idx`` maps sequence b to a cache entry.  ``alibi`` is None, "head" (one slope
    per query head) or "batch_head"."""
    name: str
    batch: int
    seqlen_q: int
    heads_q: int
    heads_kv: int
    headdim: int
    dtype: str
    capacity: int
    causal: bool = True
    cache_batch: int | None = None
    lengths: list | None = None
    batch_idx: list | None = None
    page: int = 0
    window: tuple = (-1, -1)
    alibi: str | None = None
    seed: int = 0
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.headdim)

    @property
    def max_blocks(self) -> int:
        return self.capacity // self.page if self.page else 0

    def cache_lengths(self) -> list:
        return list(self.lengths) if self.lengths is not None else [self.capacity] * self.batch


def make_kvcache_inputs(w: KVCacheWorkload) -> dict:
    """Draw q (B, Sq, Hq, D) and the caches as 16-bit CPU tensors, plus the int32
    ``cache_seqlens`` / ``cache_batch_idx`` / ``block_table`` and fp32 ``alibi_slopes``
    that the workload asks for (absent keys mean "not given").

    Draw order: q, k_cache, v_cache (standard normal, float32, one RNE cast), then the
    block-table permutation of the pool, then the ALiBi slopes: the usual geometric
    schedule 2^(-8 (h+1) / Hq) times a uniform factor in [0.5, 1.5)."""
    if w.page and w.capacity % w.page:
        raise ValueError("capacity must be a whole number of pages")
    rng = np.random.default_rng(w.seed)
    D = w.headdim
    if w.page:
        n_blocks = w.cache_batch if w.cache_batch is not None else w.batch * w.max_blocks + 3
        cache_shape = (n_blocks, w.page, w.heads_kv, D)
    else:
        n_entries = w.cache_batch if w.cache_batch is not None else w.batch
        cache_shape = (n_entries, w.capacity, w.heads_kv, D)
    out = {}
    out["q"] = _cast(rng.standard_normal((w.batch, w.seqlen_q, w.heads_q, D), dtype=np.float32), w.dtype)
    out["k_cache"] = _cast(rng.standard_normal(cache_shape, dtype=np.float32), w.dtype)
    out["v_cache"] = _cast(rng.standard_normal(cache_shape, dtype=np.float32), w.dtype)
    if w.page:
        if cache_shape[0] < w.batch * w.max_blocks:
            raise ValueError("block pool smaller than the block tables")
        perm = rng.permutation(cache_shape[0])[: w.batch * w.max_blocks]
        out["block_table"] = torch.tensor(perm.reshape(w.batch, w.max_blocks), dtype=torch.int32)
    if w.lengths is not None:
        out["cache_seqlens"] = torch.tensor(w.lengths, dtype=torch.int32)
    if w.batch_idx is not None:
        out["cache_batch_idx"] = torch.tensor(w.batch_idx, dtype=torch.int32)
    if w.alibi is not None:
        out["alibi_slopes"] = alibi_slopes(rng, w.heads_q, w.batch, w.alibi)
    return out


def make_kvcache_inputs_on_device(w: KVCacheWorkload, device: str = "cuda", chunk_rows: int = 8192) -> dict:
    """A contiguous KV cache drawn on ``device`` itself (caches of several GiB): one
    ``torch.Generator(device)`` seeded with ``w.seed``; draw order q, k_cache, v_cache,
    the caches in slices of ``chunk_rows`` positions (all entries and heads of a slice at
    once), each slice ``torch.randn(..., float32)`` cast once to the 16-bit dtype.
    ``cache_seqlens`` / ``cache_batch_idx`` come from the workload as int32 tensors."""
    if w.page or w.alibi is not None:
        raise ValueError("device-side draws are for contiguous caches without ALiBi")
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = DTYPES[w.dtype]
    D = w.headdim
    n_entries = w.cache_batch if w.cache_batch is not None else w.batch

    def randn(shape):
        return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dt)

    out = {"q": randn((w.batch, w.seqlen_q, w.heads_q, D))}
    for name in ("k_cache", "v_cache"):
        t = torch.empty((n_entries, w.capacity, w.heads_kv, D), dtype=dt, device=device)
        for s0 in range(0, w.capacity, chunk_rows):
            s1 = min(w.capacity, s0 + chunk_rows)
            t[:, s0:s1] = randn((n_entries, s1 - s0, w.heads_kv, D))
        out[name] = t
    if w.lengths is not None:
        out["cache_seqlens"] = torch.tensor(w.lengths, dtype=torch.int32, device=device)
    if w.batch_idx is not None:
        out["cache_batch_idx"] = torch.tensor(w.batch_idx, dtype=torch.int32, device=device)
    return out


def decode_workload() -> KVCacheWorkload:
    """Serving-style decode step: 16 sequences, one new token each, GQA 32:8 query/KV
    heads of 128, bf16 cache of 32768 positions per sequence, cache lengths drawn uniformly
    from [1, 32768] (seed 16)."""
    lens = varlen_lengths(16, 16, 1, 32768)
    return KVCacheWorkload("decode_b16_hq32_hkv8_d128_bf16_cache32k", 16, 1, 32, 8, 128, "bf16", 32768, causal=True,
                           lengths=lens, seed=16)


def kvcache_bytes(w: KVCacheWorkload) -> float:
    """Algorithmic HBM bytes of one decode call without a window: the first
    ``cache_seqlens[b]`` key and value rows of every KV head once, q read once, out written
    once (16-bit), the LSE written once (fp32)."""
    e = 2
    kv = sum(w.cache_lengths()) * w.heads_kv * w.headdim * e * 2
    qo = 2 * w.batch * w.seqlen_q * w.heads_q * w.headdim * e
    return float(kv + qo + w.batch * w.seqlen_q * w.heads_q * 4)
