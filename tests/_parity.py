"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding, run the
oracle on the same seeded inputs, and compare element by element."""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from exact_tiled_attention_02_amd import synth
from oracle import attention_fp64 as orc

FWD_TOL = {"bf16": 1e-2, "fp16": 2e-3}  # max abs error of O
LSE_TOL = 1e-3  # max abs error of the LSE
# Relative Frobenius error of dQ, dK, dV.  The stated bar is for bf16 (unit roundoff
# 2^-8 of its 8-bit significand); fp16 carries 3 more significand bits, so the same
# margin over its unit roundoff (2^-11) is 5e-2 / 8.
GRAD_TOL = {"bf16": 5e-2, "fp16": 5e-2 / 8}

THREADS = min(16, os.cpu_count() or 1)
REPORT: list = []  # full-tensor errors, printed in the session's terminal summary
MANT_BITS = {"bf16": 8, "fp16": 11}  # significand bits including the implicit one


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash still shows what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def dev(x: dict) -> dict:
    return {k: v.cuda() for k, v in x.items()}


def run_forward(w: synth.Workload, x: dict, poison: bool = True):
    """HIP forward on device copies of ``x``; outputs pre-filled with NaN so that any
    element the kernel fails to write shows up."""
    from exact_tiled_attention_02_amd import fa
    d = dev(x)
    out = torch.full_like(d["q"], float("nan")) if poison else torch.empty_like(d["q"])
    lse = torch.full(fa.lse_shape(d["q"], d.get("cu_seqlens_q")), float("nan"), dtype=torch.float32, device="cuda")
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=d["cu_seqlens_q"], cu_seqlens_k=d["cu_seqlens_k"], max_seqlen_q=w.seqlen_q,
                  max_seqlen_k=w.seqlen_k)
    fa.fa_fwd(d["q"], d["k"], d["v"], out, lse, causal=w.causal, scale=w.softmax_scale, window_size=w.window,
              alibi_slopes=d.get("alibi_slopes"), **kw)
    torch.cuda.synchronize()
    return out, lse, d


def oracle_forward(w: synth.Workload, x: dict):
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=x["cu_seqlens_q"].numpy(), cu_seqlens_k=x["cu_seqlens_k"].numpy())
    slopes = x["alibi_slopes"].numpy() if "alibi_slopes" in x else None
    with threadpool_limits(1):  # the oracle threads over heads; BLAS one thread each
        return orc.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), scale=w.softmax_scale, causal=w.causal,
                           threads=THREADS, window=w.window, alibi_slopes=slopes, **kw)


def _slices(w: synth.Workload, x: dict):
    """(sequence, query head) -> (q rows, k rows, v rows) index data of every pair."""
    G = w.heads_q // w.heads_kv
    out = []
    for b in range(w.batch):
        if w.varlen:
            cq, ck = x["cu_seqlens_q"].tolist(), x["cu_seqlens_k"].tolist()
            q0, lq, k0, lk = cq[b], cq[b + 1] - cq[b], ck[b], ck[b + 1] - ck[b]
        else:
            q0, lq, k0, lk = b * w.seqlen_q, w.seqlen_q, b * w.seqlen_k, w.seqlen_k
        for h in range(w.heads_q):
            out.append((b, h, h // G, q0, lq, k0, lk))
    return out


def oracle_forward_all_rows(w: synth.Workload, x: dict, chunk: int = 1024):
    """The oracle's output and LSE for EVERY row of every (sequence, query head) pair,
    evaluated ``chunk`` query rows at a time with ``rows_forward`` (the same definition
    as ``forward``, pinned equal to it), so that memory stays bounded at long sequences.
    Threaded over (pair, chunk); BLAS one thread each.  Returns (O, LSE) in the layouts
    of the HIP path: O like q, LSE (B, Hq, Sq) or (Hq, total_q)."""
    q, k, v = x["q"], x["k"], x["v"]
    qf = f64(q).reshape((-1,) + tuple(q.shape[-2:]))
    kf = f64(k).reshape((-1,) + tuple(k.shape[-2:]))
    vf = f64(v).reshape((-1,) + tuple(v.shape[-2:]))
    o = np.full(qf.shape, np.nan)
    lse = np.full((w.heads_q, qf.shape[0]), np.nan)
    slopes = x["alibi_slopes"].numpy() if "alibi_slopes" in x else None
    work = []
    for (b, h, g, q0, lq, k0, lk) in _slices(w, x):
        for r0 in range(0, lq, chunk):
            work.append((b, h, g, q0, lq, k0, lk, r0, min(lq, r0 + chunk)))

    def one(item):
        b, h, g, q0, lq, k0, lk, r0, r1 = item
        slope = None if slopes is None else float(slopes[h] if slopes.ndim == 1 else slopes[b, h])
        rows = np.arange(r0, r1)
        ob, lb = orc.rows_forward(qf[q0 + r0:q0 + r1, h], rows, kf[k0:k0 + lk, g], vf[k0:k0 + lk, g],
                                  w.softmax_scale, w.causal, lq, window=w.window, alibi_slope=slope)
        o[q0 + r0:q0 + r1, h] = ob
        lse[h, q0 + r0:q0 + r1] = lb

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(one, work))
    if w.varlen:
        return o, lse
    return o.reshape(tuple(q.shape)), lse.reshape(w.heads_q, w.batch, w.seqlen_q).transpose(1, 0, 2).copy()


def excess_report(o: np.ndarray, o_ref: np.ndarray, tol: float, dtype: str) -> str:
    """Count of output elements over the bar, how many of them have |O_ref| >= 4 (where the
    16-bit rounding of the output alone can exceed a 1e-2 bar in bf16), and their distance
    in units in the last place of the output dtype."""
    err = np.abs(o - o_ref)
    bad = err > tol
    n = int(bad.sum())
    if n == 0:
        return "no element over the bar"
    big = bad & (np.abs(o_ref) >= 4)
    ref = np.abs(o_ref[bad])
    ulp = np.exp2(np.floor(np.log2(np.maximum(ref, 1e-300))) - (MANT_BITS[dtype] - 1))
    ulps = err[bad] / ulp
    return (f"{n} elements over {tol} ({int(big.sum())} with |O_ref| >= 4); distance {ulps.min():.2f}.."
            f"{ulps.max():.2f} ulp of {dtype}; first at {np.argwhere(bad)[:3].tolist()}")


def compare_forward(w: synth.Workload, o_gpu, lse_gpu, o_ref, lse_ref, where: str = ""):
    """Element-wise comparison at the stated tolerances; returns (max O err, max LSE err)."""
    o = f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lse = f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert np.isfinite(o).all(), f"{where}: non-finite output (unwritten or NaN) at {np.argwhere(~np.isfinite(o))[:5]}"
    err = float(np.abs(o - o_ref).max()) if o.size else 0.0
    inf_ref = np.isposinf(lse_ref)
    assert np.array_equal(np.isposinf(lse), inf_ref), f"{where}: +inf LSE rows differ"
    fin = ~inf_ref
    assert np.isfinite(lse[fin]).all(), f"{where}: non-finite LSE on a live row"
    lerr = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert err <= FWD_TOL[w.dtype], (f"{where}: max |O - O_ref| = {err:.3e} > {FWD_TOL[w.dtype]}: "
                                     f"{excess_report(o, o_ref, FWD_TOL[w.dtype], w.dtype)}")
    assert lerr <= LSE_TOL, f"{where}: max |LSE - LSE_ref| = {lerr:.3e} > {LSE_TOL}"
    return err, lerr


def sampled_rows(L: int, rng: np.random.Generator, n_random: int = 24, tiles=(64, 128)) -> np.ndarray:
    """Rows at the sequence ends, around tile boundaries and at random."""
    picks = {0, 1, L - 1, L - 2}
    for t in tiles:
        for m in (1, 2, (L // t) // 2, L // t - 1, L // t):
            for off in (-1, 0, 1):
                picks.add(m * t + off)
    picks.update(rng.integers(0, L, n_random).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < L))


def check_forward_sampled(w: synth.Workload, x: dict, o_gpu, lse_gpu, heads, seed: int = 0):
    """Compare sampled rows of the listed (sequence, query head) pairs with the
    row-by-row oracle."""
    rng = np.random.default_rng(seed)
    q, k, v = x["q"], x["k"], x["v"]
    G = w.heads_q // w.heads_kv
    o_all = o_gpu.cpu()
    l_all = lse_gpu.cpu()
    worst = (0.0, 0.0)
    for (b, h) in heads:
        if w.varlen:
            cq, ck = x["cu_seqlens_q"].tolist(), x["cu_seqlens_k"].tolist()
            q0, lq, k0, lk = cq[b], cq[b + 1] - cq[b], ck[b], ck[b + 1] - ck[b]
            qs, ks, vs = q[q0:q0 + lq, h], k[k0:k0 + lk, h // G], v[k0:k0 + lk, h // G]
            og, lg = o_all[q0:q0 + lq, h], l_all[h, q0:q0 + lq]
        else:
            lq, lk = w.seqlen_q, w.seqlen_k
            qs, ks, vs = q[b, :, h], k[b, :, h // G], v[b, :, h // G]
            og, lg = o_all[b, :, h], l_all[b, h]
        if lq == 0:
            continue
        rows = sampled_rows(lq, rng)
        slope = None
        if "alibi_slopes" in x:
            a = x["alibi_slopes"].numpy()
            slope = float(a[h] if a.ndim == 1 else a[b, h])
        o_ref, lse_ref = orc.rows_forward(f64(qs[rows]), rows, f64(ks), f64(vs), w.softmax_scale, w.causal, lq,
                                          window=w.window, alibi_slope=slope)
        e = compare_forward(w, og[rows], lg[rows], o_ref, lse_ref, where=f"{w.name} seq {b} head {h}")
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    return worst
