"""Plain fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run this
module: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP kernels and never reads anything
they produce except to compare against it.

What it computes is the plain definition, written out and materialised (no tiling, no
online softmax, no blocking):

* Attention is ``softmax(Q @ K^T * softmax_scale) @ V`` with ``softmax_scale``
  defaulting to ``1/sqrt(headdim)``  -- FlashAttention (Dao-AILab/flash-attention
  README), section "How to use FlashAttention", the ``flash_attn_func`` docstring.
* Layouts ``q: (batch, seqlen, nheads, headdim)``, ``k, v: (batch, seqlen, nheads_k,
  headdim)``; query head ``h`` reads KV head ``h // (nheads // nheads_k)`` (6 query heads
  over 2 KV heads: 0,1,2 -> 0 and 3,4,5 -> 1) -- same docstring, MQA/GQA paragraph.
* The causal mask is aligned to the bottom-right corner of the score matrix: key ``j``
  is kept for query ``i`` iff ``j <= i + seqlen_k - seqlen_q``; a query row whose mask
  row is all zero produces an all-zero output -- same README, the
  ``flash_attn_with_kvcache`` docstring and changelog entry 2.1.
* The softmax log-sum-exp (LSE) is returned by the low-level ops -- the
  kernels-community/flash-attn2 repository card, section "Low-level ops".  Its base is
  the natural log of ``sum_j exp(scale * s_ij)``: the backward of the release notes
  "v1.4 - FlashAttention Fork: 2.9.0 -> 2.9.1", section 4.1 (``scale_apply_exp2`` with
  ``Scale_max=false``), multiplies the stored value by log2(e) before using it as an
  exp2 offset, which fixes natural-log units.
* The backward is the analytic gradient of the same definition: with
  ``P = softmax(S)``, ``dV = P^T dO``, ``dP = dO V^T``, ``Dsum_i = sum_d dO_id O_id``
  (which equals ``sum_j P_ij dP_ij``), ``dS = P * (dP - Dsum)``, ``dQ = scale dS K``,
  ``dK = scale dS^T Q``.  For GQA the gradients of a KV head sum over the query heads
  that read it.
* Sliding-window (local) attention, ``window = (left, right)`` with -1 meaning unbounded
  on that side: query ``i`` keeps keys ``j`` with
  ``i + seqlen_k - seqlen_q - left <= j <= i + seqlen_k - seqlen_q + right`` -- the
  ``flash_attn_func`` docstring (window paragraph) and changelog entry 2.3.  With
  ``causal`` both conditions must hold (the window is intersected with the causal mask).
* ALiBi: the bias ``-slope_h * |i + seqlen_k - seqlen_q - j|`` is added to the scaled
  score of query ``i`` and key ``j`` of query head ``h`` before the softmax -- the
  ``alibi_slopes`` argument of the same docstring.  Slopes are given per query head, or
  per (sequence, query head).  The returned LSE is that of the biased scores.
* KV cache (``flash_attn_with_kvcache`` docstring, read-only use): sequence ``b`` reads
  cache entry ``cache_batch_idx[b]`` (default ``b``), its first ``cache_seqlens[b]`` rows
  (default: all), and, with a block table, key row ``j`` lives in physical block
  ``block_table[b, j // page]`` at row ``j % page``.  Masks and biases use
  ``seqlen_k = cache_seqlens[b]``.

Readings taken where the pages are silent (each also listed in the design notes):

* A fully masked query row gets ``O = 0`` (printed) and ``LSE = +inf`` (so that
  ``exp(s - LSE) = 0`` when the backward recomputes probabilities); its gradients are 0.
* Variable-length ("varlen") packed batches: sequence ``b`` occupies rows
  ``[cu_seqlens[b], cu_seqlens[b+1])`` of the packed ``(total, nheads, headdim)`` arrays
  and is attended independently; the LSE is laid out ``(nheads, total_q)``.  In padded
  mode the LSE is ``(batch, nheads, seqlen_q)``.

All arithmetic is numpy float64.  Inputs of any float dtype are upcast exactly.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "kv_head_of",
    "causal_keep_mask",
    "keep_mask",
    "alibi_bias",
    "gather_kvcache",
    "forward_kvcache",
    "head_probabilities",
    "head_forward",
    "rows_forward",
    "head_backward",
    "forward",
    "backward",
]


def kv_head_of(h: int, n_heads_q: int, n_heads_kv: int) -> int:
    """KV head read by query head ``h``: contiguous groups of ``n_heads_q // n_heads_kv``
    query heads share one KV head (flash_attn_func docstring, MQA/GQA paragraph)."""
    if n_heads_q % n_heads_kv != 0:
        raise ValueError("number of query heads must be divisible by number of KV heads")
    return h // (n_heads_q // n_heads_kv)


def causal_keep_mask(len_q: int, len_k: int, causal: bool) -> np.ndarray:
    """Boolean (len_q, len_k) matrix, True where key j is kept for query i.

    Bottom-right alignment: keep iff ``j <= i + len_k - len_q`` (flash_attn_with_kvcache
    docstring; changelog entry 2.1 of the FlashAttention README)."""
    i = np.arange(len_q)[:, None]
    j = np.arange(len_k)[None, :]
    if not causal:
        return np.ones((len_q, len_k), dtype=bool)
    return j <= i + (len_k - len_q)


def keep_mask(len_q: int, len_k: int, causal: bool, window=(-1, -1), rows=None) -> np.ndarray:
    """Boolean (len(rows), len_k) matrix, True where key j is kept for query row i.

    ``rows`` are the query indices (default ``0 .. len_q-1``).  The causal condition is
    that of :func:`causal_keep_mask`; the window keeps
    ``i + len_k - len_q - left <= j <= i + len_k - len_q + right`` (a negative bound is
    unbounded) -- ``flash_attn_func`` docstring, window paragraph."""
    i = (np.arange(len_q) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(len_k)[None, :]
    diag = i + (len_k - len_q)
    keep = np.ones((i.shape[0], len_k), dtype=bool)
    if causal:
        keep &= j <= diag
    left, right = window
    if left >= 0:
        keep &= j >= diag - left
    if right >= 0:
        keep &= j <= diag + right
    return keep


def alibi_bias(len_q: int, len_k: int, slope: float, rows=None) -> np.ndarray:
    """(len(rows), len_k) float64 bias ``-slope * |i + len_k - len_q - j|`` added to the
    scaled scores (``alibi_slopes`` argument of the ``flash_attn_func`` docstring)."""
    i = (np.arange(len_q) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(len_k)[None, :]
    return -float(slope) * np.abs(i + (len_k - len_q) - j).astype(np.float64)


def _softmax_rows(s: np.ndarray, keep: np.ndarray):
    """Masked row softmax of the score matrix ``s``: (P, LSE); rows with no kept key get
    P = 0 and LSE = +inf."""
    s = np.where(keep, s, -np.inf)
    live = keep.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    z = e.sum(axis=1)
    p = np.zeros_like(e)
    p[live] = e[live] / z[live, None]
    lse = np.full(s.shape[0], np.inf)
    lse[live] = m[live] + np.log(z[live])
    return p, lse


def head_probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, window=(-1, -1),
                       alibi_slope=None):
    """Materialised softmax of one head.  Returns (P, LSE, keep) in float64.

    ``S = scale * q k^T`` (plus the ALiBi bias when ``alibi_slope`` is given); masked
    entries are excluded; rows with no kept key have P = 0 and LSE = +inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T)
    if alibi_slope is not None:
        s = s + alibi_bias(q.shape[0], k.shape[0], alibi_slope)
    keep = keep_mask(q.shape[0], k.shape[0], causal, window)
    p, lse = _softmax_rows(s, keep)
    return p, lse, keep


def head_forward(q, k, v, scale: float, causal: bool, window=(-1, -1), alibi_slope=None):
    """One head: O = P V (float64, (len_q, D)) and LSE ((len_q,))."""
    p, lse, _ = head_probabilities(q, k, scale, causal, window, alibi_slope)
    o = p @ np.asarray(v, dtype=np.float64)
    return o, lse


def rows_forward(q_rows, rows, k, v, scale: float, causal: bool, len_q: int, window=(-1, -1),
                 alibi_slope=None):
    """Output and LSE of selected query rows of one head: ``q_rows[n]`` is query row
    ``rows[n]`` of a sequence of ``len_q`` queries (the row index fixes its mask and
    bias).  Same definition as :func:`head_forward`, restricted to those rows, so that
    outputs of very long sequences can be checked one row at a time."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    len_k = k.shape[0]
    s = scale * (q_rows @ k.T)
    if alibi_slope is not None:
        s = s + alibi_bias(len_q, len_k, alibi_slope, rows)
    keep = keep_mask(len_q, len_k, causal, window, rows)
    p, lse = _softmax_rows(s, keep)
    return p @ v, lse


def head_backward(q, k, v, do, scale: float, causal: bool, window=(-1, -1), alibi_slope=None):
    """One head: analytic gradients (dq, dk, dv) of O = softmax(scale q k^T + bias) v
    w.r.t. q, k, v for the upstream gradient ``do`` (the bias does not depend on q, k, v,
    so the formulas are those of the unbiased case with the biased P).  Probabilities are
    recomputed here from the definition; nothing from a forward pass is reused."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    p, _, _ = head_probabilities(q, k, scale, causal, window, alibi_slope)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    dsum = (do * o).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _sequences(batch: int, seqlen: int, cu_seqlens):
    """List of (row_start, length) per sequence, padded or packed."""
    if cu_seqlens is None:
        return [(b * seqlen, seqlen) for b in range(batch)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1] - cu[b])) for b in range(len(cu) - 1)]


def _check(q, k, v, cu_q, cu_k):
    if (cu_q is None) != (cu_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    varlen = cu_q is not None
    if varlen:
        if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
            raise ValueError("varlen inputs are (total, heads, headdim)")
    elif q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("padded inputs are (batch, seqlen, heads, headdim)")
    hq, hkv = q.shape[-2], k.shape[-2]
    if hq % hkv != 0:
        raise ValueError("number of query heads must be divisible by number of KV heads")
    return varlen


def _flat(x, varlen):
    x = np.asarray(x)
    return x if varlen else x.reshape((-1,) + x.shape[2:])


def _slope(alibi_slopes, b, h):
    """Slope of (sequence b, query head h) from an (Hq,) or (B, Hq) array, or None."""
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return float(a[h] if a.ndim == 1 else a[b, h])


def forward(q, k, v, scale=None, causal=False, cu_seqlens_q=None, cu_seqlens_k=None,
            threads: int = 1, heads=None, window=(-1, -1), alibi_slopes=None):
    """Attention forward over a batch.

    Padded: q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D) -> O (B, Sq, Hq, D), LSE (B, Hq, Sq).
    Varlen: q (total_q, Hq, D), k/v (total_k, Hkv, D), cu_seqlens_* (B+1,) ->
    O (total_q, Hq, D), LSE (Hq, total_q).  Returns float64 arrays.

    ``heads`` optionally restricts the work to a list of (sequence, query head) pairs;
    the other entries of O and LSE are left NaN (used to time a bounded sample).
    ``window`` = (left, right) sliding window; ``alibi_slopes`` (Hq,) or (B, Hq)."""
    varlen = _check(q, k, v, cu_seqlens_q, cu_seqlens_k)
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hq, hkv = q.shape[-2], k.shape[-2]
    if varlen:
        seq_q = _sequences(None, None, cu_seqlens_q)
        seq_k = _sequences(None, None, cu_seqlens_k)
    else:
        seq_q = _sequences(q.shape[0], q.shape[1], None)
        seq_k = _sequences(k.shape[0], k.shape[1], None)
    qf, kf, vf = _flat(q, varlen), _flat(k, varlen), _flat(v, varlen)
    o = np.full(qf.shape, np.nan, dtype=np.float64)
    lse_flat = np.full((hq, qf.shape[0]), np.nan, dtype=np.float64)
    work = heads if heads is not None else [(b, h) for b in range(len(seq_q)) for h in range(hq)]

    def one(bh):
        b, h = bh
        (q0, lq), (k0, lk) = seq_q[b], seq_k[b]
        g = kv_head_of(h, hq, hkv)
        ob, lb = head_forward(qf[q0:q0 + lq, h], kf[k0:k0 + lk, g], vf[k0:k0 + lk, g], scale, causal,
                              window, _slope(alibi_slopes, b, h))
        o[q0:q0 + lq, h] = ob
        lse_flat[h, q0:q0 + lq] = lb

    _run(one, work, threads)
    if varlen:
        return o, lse_flat
    B, Sq = q.shape[0], q.shape[1]
    return o.reshape(q.shape), lse_flat.reshape(hq, B, Sq).transpose(1, 0, 2).copy()


def backward(do, q, k, v, scale=None, causal=False, cu_seqlens_q=None, cu_seqlens_k=None,
             threads: int = 1, heads=None, window=(-1, -1), alibi_slopes=None):
    """Attention backward over a batch: returns float64 (dq, dk, dv) in the layouts of
    q, k, v.  dk/dv of a KV head sum the contributions of every query head that reads
    it.  ``heads`` restricts the work as in :func:`forward` (then dk/dv hold partial
    sums and dq is NaN outside the listed heads)."""
    varlen = _check(q, k, v, cu_seqlens_q, cu_seqlens_k)
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    hq, hkv = q.shape[-2], k.shape[-2]
    if varlen:
        seq_q = _sequences(None, None, cu_seqlens_q)
        seq_k = _sequences(None, None, cu_seqlens_k)
    else:
        seq_q = _sequences(q.shape[0], q.shape[1], None)
        seq_k = _sequences(k.shape[0], k.shape[1], None)
    qf, kf, vf, dof = _flat(q, varlen), _flat(k, varlen), _flat(v, varlen), _flat(do, varlen)
    dq = np.full(qf.shape, np.nan if heads is not None else 0.0, dtype=np.float64)
    dk = np.zeros(kf.shape, dtype=np.float64)
    dv = np.zeros(vf.shape, dtype=np.float64)
    work = heads if heads is not None else [(b, h) for b in range(len(seq_q)) for h in range(hq)]
    results = {}

    def one(bh):
        b, h = bh
        (q0, lq), (k0, lk) = seq_q[b], seq_k[b]
        g = kv_head_of(h, hq, hkv)
        results[bh] = head_backward(qf[q0:q0 + lq, h], kf[k0:k0 + lk, g], vf[k0:k0 + lk, g],
                                    dof[q0:q0 + lq, h], scale, causal, window, _slope(alibi_slopes, b, h))

    _run(one, work, threads)
    # Accumulate in a fixed order so the result does not depend on thread timing.
    for (b, h) in work:
        (q0, lq), (k0, lk) = seq_q[b], seq_k[b]
        g = kv_head_of(h, hq, hkv)
        dqh, dkh, dvh = results[(b, h)]
        dq[q0:q0 + lq, h] = dqh
        dk[k0:k0 + lk, g] += dkh
        dv[k0:k0 + lk, g] += dvh
    if varlen:
        return dq, dk, dv
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


def gather_kvcache(k_cache, v_cache, b: int, cache_seqlens=None, cache_batch_idx=None, block_table=None):
    """The (len_k, Hkv, D) keys and values that sequence ``b`` reads from a KV cache
    (``flash_attn_with_kvcache`` docstring, arguments ``cache_seqlens``,
    ``cache_batch_idx`` and ``block_table``).

    Without a block table the caches are (batch_cache, seqlen_cache, Hkv, D) and the
    sequence reads rows ``0 .. len_k-1`` of entry ``cache_batch_idx[b]``.  With one they
    are (num_blocks, page, Hkv, D) and key row ``j`` is row ``j % page`` of block
    ``block_table[b, j // page]``.  ``len_k`` is ``cache_seqlens[b]`` (default: every row
    the sequence can address)."""
    if block_table is not None:
        table = np.asarray(block_table, dtype=np.int64)
        page = k_cache.shape[1]
        cap = table.shape[1] * page
    else:
        cap = k_cache.shape[1]
    len_k = cap if cache_seqlens is None else int(np.asarray(cache_seqlens)[b])
    if not 0 <= len_k <= cap:
        raise ValueError("cache_seqlens out of range")
    j = np.arange(len_k)
    if block_table is not None:
        if cache_batch_idx is not None:
            raise ValueError("cache_batch_idx and block_table are exclusive")
        blk = table[b, j // page]
        return k_cache[blk, j % page], v_cache[blk, j % page]
    e = b if cache_batch_idx is None else int(np.asarray(cache_batch_idx)[b])
    return k_cache[e, :len_k], v_cache[e, :len_k]


def forward_kvcache(q, k_cache, v_cache, cache_seqlens=None, cache_batch_idx=None, block_table=None,
                    scale=None, causal=False, window=(-1, -1), alibi_slopes=None, threads: int = 1):
    """Attention of q (B, Sq, Hq, D) against a read-only KV cache (layouts as in
    :func:`gather_kvcache`).  Returns float64 O (B, Sq, Hq, D) and LSE (B, Hq, Sq); the
    mask and bias of sequence ``b`` use ``seqlen_k = cache_seqlens[b]``."""
    q = np.asarray(q)
    B, Sq, hq, D = q.shape
    hkv = k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, Sq, hq, D))
    lse = np.zeros((B, hq, Sq))
    kv = [gather_kvcache(k_cache, v_cache, b, cache_seqlens, cache_batch_idx, block_table) for b in range(B)]

    def one(bh):
        b, h = bh
        g = kv_head_of(h, hq, hkv)
        kb, vb = kv[b]
        o[b, :, h], lse[b, h] = head_forward(q[b, :, h], kb[:, g], vb[:, g], scale, causal, window,
                                             _slope(alibi_slopes, b, h))

    _run(one, [(b, h) for b in range(B) for h in range(hq)], threads)
    return o, lse


def _run(fn, work, threads):
    if threads <= 1 or len(work) <= 1:
        for w in work:
            fn(w)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, work))
