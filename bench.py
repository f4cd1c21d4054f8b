#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

A step is one forward (fa_fwd) plus one backward (fa_bwd with the workspace the binding
allocates by default, which holds the stored-dS area: preprocess, dK/dV main loop that
stores dS, dQ from the stored dS) over the causal MHA workload B=2, H=16, S=4096, D=128,
bf16 -- the reference workload that includes the backward.  Inputs are seeded synthetic
N(0,1) draws, resident in HBM before timing starts.

Prints ONE JSON line: throughput in algorithmic TFLOPS (forward 4*B*H*S*S*D/2 for causal,
backward 2.5x that; masked work and recomputation are not counted), the roofline of the
dominant kernel (the backward main loop) timed per launch with HIP events on the stream
it runs on, the fp64 CPU oracle timed on a bounded sample of the same workload, and
extra detail: the forward and backward of the causal GQA workload B=2, Hq=32, Hkv=8,
S=8192, D=128, the forwards of the other reference workloads, and the split-KV decode of
16 sequences against a 32k-position bf16 KV cache (GB/s).  The detail workloads run
before the headline steps, so that those are timed on a GPU already under load (its
clock takes tens of milliseconds of load to settle).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
# fp32 atomic adds complete at the memory side at ~2.1e10 64-byte requests per second for
# the whole chip (measured by `--atomic-rate`, whatever the lane layout or issuing XCD)
ATOMIC_REQ_PER_S = 2.1e10
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Case:
    """Device-resident inputs and outputs of one workload."""

    def __init__(self, n, with_bwd: bool):
        """``n``: a reference workload number, or a synth.Workload."""
        import torch
        from exact_tiled_attention_02_amd import fa, synth
        if isinstance(n, int):
            self.w, x = synth.draw_config(n)
        else:
            self.w, x = n, synth.make_inputs(n)
        self.w.backward = with_bwd
        d = {k: v.cuda() for k, v in x.items()}
        if with_bwd and "do" not in d:
            import numpy as np
            rng = np.random.default_rng(1000 + self.w.seed)
            d["do"] = synth._cast(rng.standard_normal(tuple(d["q"].shape), dtype=np.float32), self.w.dtype).cuda()
        self.d = d
        self.out = torch.empty_like(d["q"])
        self.lse = torch.empty(fa.lse_shape(d["q"], d.get("cu_seqlens_q")), dtype=torch.float32, device="cuda")
        if with_bwd:
            self.dq, self.dk, self.dv = (torch.empty_like(d[k]) for k in ("q", "k", "v"))
            # the binding's default workspace: with the stored-dS area (fa_bwd's fastest
            # route); its first fa_bwd_workspace_bytes serve the atomic route's stages too
            self.ws = fa.workspace_for(d["q"], k=d["k"], stored_ds=True)
        self.fwd_flops, self.bwd_flops = synth.flops(self.w)

    def fwd(self):
        from exact_tiled_attention_02_amd import fa
        if "cu_seqlens_q" in self.d:  # packed variable-length batch
            fa.fa_fwd(self.d["q"], self.d["k"], self.d["v"], self.out, self.lse, causal=self.w.causal,
                      scale=self.w.softmax_scale, cu_seqlens_q=self.d["cu_seqlens_q"],
                      cu_seqlens_k=self.d["cu_seqlens_k"], max_seqlen_q=self.w.seqlen_q, max_seqlen_k=self.w.seqlen_k)
            return
        fa.fa_fwd(self.d["q"], self.d["k"], self.d["v"], self.out, self.lse, causal=self.w.causal,
                  scale=self.w.softmax_scale)

    def bwd_stage(self, stage):
        from exact_tiled_attention_02_amd import fa
        fa.fa_bwd_stage(stage, self.d["do"], self.d["q"], self.d["k"], self.d["v"], self.out, self.lse, self.dq,
                        self.dk, self.dv, self.ws, causal=self.w.causal, scale=self.w.softmax_scale)

    def step(self):
        self.fwd()
        self.bwd_stage(0)


def time_launches(fn, n, pre=None, post=None, stats=None):
    """Average duration (s) of fn() over n launches, each bracketed by HIP events recorded
    on torch's current stream -- the stream the library launches on.  ``stats``, a dict,
    also receives the median and the minimum."""
    import torch
    total = 0.0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        if pre:
            pre()
        starts[i].record()
        fn()
        ends[i].record()
        if post:
            post()
    torch.cuda.synchronize()
    ts = sorted(s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends))
    total = sum(ts)
    if stats is not None:
        stats["median"] = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
        stats["min"] = ts[0]
    return total / n


def time_graph(fn, reps, n):
    """Device time (s) per call of fn(), from n replays of a HIP graph that holds reps
    calls.  For kernels of a few microseconds, where an event pair around one call from
    Python also times the host's launch path (argument checks, ctypes)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    t = time_launches(g.replay, n) / reps
    del g
    return t


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_main_fwdbwd_b2_h16_s4096_d128_bf16.json")
BWD_SOURCE = os.path.join(ROOT, "exact_tiled_attention_02_amd", "csrc", "fa_bwd.hip")


def measured_traffic():
    """HBM bytes per launch of the backward main loop from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's reading for a plain
    copy of known size), or None when the kernel source has changed since."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(BWD_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return 1024.0 * (rec["fetch_kib_per_launch"] * rec["copy_fetch_factor"] +
                     rec["write_kib_per_launch"] * rec["copy_write_factor"])


def copy_calibration(n_bytes: int = 512 << 20, reps: int = 3):
    """A plain device-to-device copy of known size, for scaling the byte counters."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n_bytes, "reps": reps}), flush=True)


def sweep(steps: int, warmup: int):
    """The benchmark grid of the FlashAttention README's A100 section ("Performance"):
    head dimension 64 or 128 with hidden size 2048 (32 or 16 heads), sequence lengths
    512 .. 16k, batch 16k / seqlen, forward + backward, causal and not; reproduced on one
    MI355X with synthetic bf16 inputs as a second workload.  Prints one JSON line per
    point: algorithmic TFLOPS of the forward, the backward and both, and their fractions
    of the dense bf16 MFMA peak (the pages' A100 figures are context, not a target; the
    correctness baseline is the fp64 oracle, which the parity tests run)."""
    import torch
    from exact_tiled_attention_02_amd import fa, synth
    for D in (64, 128):
        H = 2048 // D
        for causal in (False, True):
            for S in (512, 1024, 2048, 4096, 8192, 16384):
                B = 16384 // S
                w = synth.Workload(f"sweep_d{D}_s{S}", B, H, H, S, S, D, "bf16", causal, backward=True, seed=S + D)
                x = {k: v.cuda() for k, v in synth.make_inputs(w).items()}
                out = torch.empty_like(x["q"])
                lse = torch.empty(fa.lse_shape(x["q"]), dtype=torch.float32, device="cuda")
                dq, dk, dv = (torch.empty_like(x[k]) for k in ("q", "k", "v"))
                ws = fa.workspace_for(x["q"], k=x["k"], stored_ds=True)  # the binding's default route
                ws_base = fa.workspace_for(x["q"])                         # atomic route, for comparison
                fwd = lambda: fa.fa_fwd(x["q"], x["k"], x["v"], out, lse, causal=causal)
                bwd = lambda: fa.fa_bwd(x["do"], x["q"], x["k"], x["v"], out, lse, dq, dk, dv, ws, causal=causal)
                bwd_a = lambda: fa.fa_bwd(x["do"], x["q"], x["k"], x["v"], out, lse, dq, dk, dv, ws_base,
                                          causal=causal)
                for _ in range(warmup):
                    fwd()
                    bwd()
                tf = time_launches(fwd, steps)
                tb = time_launches(bwd, steps)
                ta = time_launches(bwd_a, steps)
                ff, fb = synth.flops(w)
                rec = {"workload": w.name, "batch": B, "heads": H, "seqlen": S, "headdim": D, "causal": causal,
                       "fwd_tflops": ff / tf / 1e12, "bwd_tflops": fb / tb / 1e12,
                       "fwdbwd_tflops": (ff + fb) / (tf + tb) / 1e12,
                       "fwd_pct_peak": 100 * ff / tf / 1e12 / PEAK_TFLOPS,
                       "bwd_pct_peak": 100 * fb / tb / 1e12 / PEAK_TFLOPS,
                       "fwdbwd_pct_peak": 100 * (ff + fb) / (tf + tb) / 1e12 / PEAK_TFLOPS,
                       "fwd_us": tf * 1e6, "bwd_us": tb * 1e6, "bwd_atomic_route_us": ta * 1e6}
                print(json.dumps(rec), flush=True)
                del x, out, lse, dq, dk, dv, ws, ws_base
                torch.cuda.empty_cache()


def decode_detail(steps: int, warmup: int):
    """Split-KV decode against a read-only KV cache (fa_fwd_kvcache, split kernel plus the
    merge kernel): 16 sequences with one new query row each, GQA 32:8 heads of 128, bf16
    cache of 32768 positions per sequence with lengths uniform in [1, 32768].  HBM-bound:
    reported as algorithmic bytes (every cached key and value row up to the length, q,
    out, LSE) per second of the whole call."""
    import torch
    from exact_tiled_attention_02_amd import fa, synth
    w = synth.decode_workload()
    d = {k: v.cuda() for k, v in synth.make_kvcache_inputs(w).items()}
    B, Sq, Hq, D = d["q"].shape
    out = torch.empty_like(d["q"])
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    ns = fa.kvcache_splits(d["q"], d["k_cache"])
    ws = torch.empty(fa.fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, ns), dtype=torch.uint8, device="cuda")
    run = lambda: fa.fa_fwd_kvcache(d["q"], d["k_cache"], d["v_cache"], out, lse, cache_seqlens=d["cache_seqlens"],
                                    causal=w.causal, scale=w.softmax_scale, workspace=ws)
    for _ in range(warmup):
        run()
    t = time_launches(run, steps)
    nbytes = synth.kvcache_bytes(w)
    return w.name, {"us": t * 1e6, "gbs": nbytes / t / 1e9, "pct_hbm_peak": 100 * nbytes / t / 1e9 / PEAK_HBM_GBS,
                    "bytes": nbytes, "cache_tokens": sum(w.cache_lengths()), "splits_max": ns}


def cpu_baseline(target_s: float = 12.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: whole
    (batch, head) slices of forward + backward, until about target_s seconds of work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from exact_tiled_attention_02_amd import synth
    from oracle import attention_fp64 as orc
    w, x = synth.draw_config(5)
    f = lambda t: t.to(dtype=__import__("torch").float64).numpy()
    q, k, v, do = (f(x[n]) for n in ("q", "k", "v", "do"))
    cores = min(16, os.cpu_count() or 1)
    heads_all = [(b, h) for b in range(w.batch) for h in range(w.heads_q)]
    per_head = synth.flops(w)
    per_head = (per_head[0] + per_head[1]) / len(heads_all)
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while done < len(heads_all) and time.perf_counter() - t0 < target_s:
            batch = heads_all[done:done + cores]
            orc.forward(q, k, v, causal=True, threads=cores, heads=batch)
            orc.backward(do, q, k, v, causal=True, threads=cores, heads=batch)
            done += len(batch)
    dt = time.perf_counter() - t0
    return {"value": per_head * done / dt / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle, forward+backward of {done} of {len(heads_all)} (batch, head) slices of "
                      f"B=2 H=16 S=4096 D=128 causal, {dt:.1f} s on {cores} threads (BLAS 1 thread each); "
                      f"value = algorithmic FLOPs of the sample / wall time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # ~70 ms of untimed steps: after 5 the timed steps still ran ~7 % slower than in steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-gqa", action="store_true",
                    help="skip the details of the other workloads (GQA S=8192 forward and backward, small S=128, "
                         "MHA S=2048, varlen D=256)")
    ap.add_argument("--skip-decode", action="store_true", help="skip the KV-cache decode detail")
    ap.add_argument("--copy-calibration", action="store_true", help="only run a 512 MiB device copy (counter scale)")
    ap.add_argument("--sweep", action="store_true", help="only run the head-dim / seqlen sweep (one JSON line each)")
    ap.add_argument("--atomic-rate", action="store_true",
                    help="only run the fp32 atomic-rate measurement program (one JSON line per variant)")
    ap.add_argument("--lds-rate", action="store_true",
                    help="only run the LDS read-rate measurement program (one JSON line per read form)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        sweep(args.steps, args.warmup)
        return
    if args.atomic_rate or args.lds_rate:
        import subprocess
        prog = os.path.join(ROOT, "exact_tiled_attention_02_amd", "atomic_rate" if args.atomic_rate else "lds_rate")
        sys.exit(subprocess.run([prog]).returncode)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path is single-GPU; "
              f"see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)
    import torch
    from exact_tiled_attention_02_amd import fa
    fa.lib()
    K, W = args.steps, args.warmup
    detail = {}

    # The other workloads run first, each with its own W untimed calls, so that the
    # headline steps (timed last) see the clock a GPU holds under sustained load.
    if not args.skip_gqa:
        # the long causal GQA workload (B=2, Hq=32, Hkv=8, S=8192, D=128): forward, and
        # the backward at the same shape (stages timed separately)
        c3 = Case(3, with_bwd=True)
        for _ in range(W):
            c3.fwd()
        st3 = {}
        t3 = time_launches(c3.fwd, K, stats=st3)
        n = max(3, K // 4)
        for _ in range(max(1, W // 4)):
            c3.bwd_stage(0)
        # the whole backward (fa_bwd, stored-dS route) per launch; its stages, and those of the
        # atomic route, per launch (milliseconds each; the main loops after a preprocess
        # that resets the key-block queue)
        t3b = time_launches(lambda: c3.bwd_stage(0), n)
        t3m = time_launches(lambda: c3.bwd_stage(4), n, pre=lambda: c3.bwd_stage(1))
        t3q = time_launches(lambda: c3.bwd_stage(5), n)
        t3a = time_launches(lambda: c3.bwd_stage(2), n, pre=lambda: c3.bwd_stage(1))
        detail[c3.w.name] = {
            "fwd_tflops": c3.fwd_flops / t3 / 1e12, "fwd_pct_peak": 100 * c3.fwd_flops / t3 / 1e12 / PEAK_TFLOPS,
            "fwd_us": t3 * 1e6, "fwd_us_median": st3["median"] * 1e6, "fwd_us_min": st3["min"] * 1e6,
            "bwd_tflops": c3.bwd_flops / t3b / 1e12, "bwd_pct_peak": 100 * c3.bwd_flops / t3b / 1e12 / PEAK_TFLOPS,
            "bwd_us": t3b * 1e6, "bwd_main_store_ds_us": t3m * 1e6, "bwd_dq_from_ds_us": t3q * 1e6,
            "bwd_main_atomic_route_us": t3a * 1e6,
        }
        log(f"[bench] GQA S=8192 forward {t3 * 1e6:.1f} us -> {detail[c3.w.name]['fwd_tflops']:.1f} TFLOPS; "
            f"backward {t3b * 1e6:.1f} us -> {detail[c3.w.name]['bwd_tflops']:.1f} TFLOPS "
            f"(main loop {t3m * 1e6:.1f} us, dQ from dS {t3q * 1e6:.1f} us; atomic main loop {t3a * 1e6:.1f} us)")
        del c3
        torch.cuda.empty_cache()

        # forwards of the small non-causal (B=1, H=2, S=128, D=64, fp16: launch/latency
        # bound, so also in GB/s of Q, K, V, O and LSE), the causal MHA (B=4, H=16, S=2048,
        # D=128, bf16) and the packed variable-length (16 sequences, H=8, D=256, fp16) workloads
        for n in (1, 2, 4):
            cn = Case(n, with_bwd=False)
            for _ in range(W):
                cn.fwd()
            tn = time_launches(cn.fwd, K)
            detail[cn.w.name] = {"fwd_tflops": cn.fwd_flops / tn / 1e12,
                                 "fwd_pct_peak": 100 * cn.fwd_flops / tn / 1e12 / PEAK_TFLOPS, "fwd_us": tn * 1e6}
            if n == 1:
                # A call this small is bound by the host (argument checks, ctypes): time K
                # launches captured in one HIP graph as well, which leaves the device time.
                tg = time_graph(cn.fwd, K, 5)
                nbytes = sum(t.numel() * t.element_size() for t in (cn.d["q"], cn.d["k"], cn.d["v"], cn.out, cn.lse))
                detail[cn.w.name].update({"fwd_us_graph": tg * 1e6, "bytes": nbytes, "gbs_graph": nbytes / tg / 1e9})
                log(f"[bench] {cn.w.name} forward in a graph {tg * 1e6:.2f} us per call, {nbytes / tg / 1e9:.1f} GB/s")
            log(f"[bench] {cn.w.name} forward {tn * 1e6:.1f} us -> {detail[cn.w.name]['fwd_tflops']:.1f} TFLOPS")
            del cn
        torch.cuda.empty_cache()

    if not args.skip_gqa:
        # head dimension 256 forward + backward: B=1, H=16, S=8192, causal, bf16
        from exact_tiled_attention_02_amd import synth
        c6 = Case(synth.Workload("fwdbwd_causal_b1_h16_s8192_d256_bf16", 1, 16, 16, 8192, 8192, 256, "bf16", True,
                                 backward=True, seed=6), with_bwd=True)
        for _ in range(max(1, W // 4)):
            c6.step()
        n = max(3, K // 4)
        t6f = time_launches(c6.fwd, n)
        t6b = time_launches(lambda: c6.bwd_stage(0), n)
        detail[c6.w.name] = {
            "fwd_tflops": c6.fwd_flops / t6f / 1e12, "fwd_pct_peak": 100 * c6.fwd_flops / t6f / 1e12 / PEAK_TFLOPS,
            "bwd_tflops": c6.bwd_flops / t6b / 1e12, "bwd_pct_peak": 100 * c6.bwd_flops / t6b / 1e12 / PEAK_TFLOPS,
            "fwd_us": t6f * 1e6, "bwd_us": t6b * 1e6,
        }
        log(f"[bench] D=256 S=8192 forward {t6f * 1e6:.1f} us -> {detail[c6.w.name]['fwd_tflops']:.1f} TFLOPS; "
            f"backward {t6b * 1e6:.1f} us -> {detail[c6.w.name]['bwd_tflops']:.1f} TFLOPS")
        del c6
        torch.cuda.empty_cache()

    if not args.skip_decode:
        name, dd = decode_detail(K, W)
        detail[name] = dd
        log(f"[bench] decode {dd['us']:.1f} us -> {dd['gbs']:.0f} GB/s ({dd['pct_hbm_peak']:.1f}% of HBM peak)")
        torch.cuda.empty_cache()

    # The headline: W untimed steps, then exactly K timed steps of forward + backward.
    c5 = Case(5, with_bwd=True)
    log(f"[bench] workload {c5.w.name}: warmup {W}, steps {K}")
    for _ in range(W):
        c5.step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K):
        c5.step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    step_flops = c5.fwd_flops + c5.bwd_flops
    value = step_flops / (ms * 1e-3) / 1e12
    log(f"[bench] step {ms:.3f} ms -> {value:.1f} TFLOPS")

    # per-kernel durations (HIP events on the launch stream).  The stored-dS route that the
    # step runs: preprocess (device time from a graph of 10 calls, ~15 us), the main loop
    # that stores dS (the dominant kernel), dQ from the stored dS.  Then the atomic route's
    # stages and the deterministic call with only the base workspace (recompute route).
    st_fwd, st_main = {}, {}
    t_fwd = time_launches(c5.fwd, K, stats=st_fwd)
    t_bwd = time_launches(lambda: c5.bwd_stage(0), K)
    t_main = time_launches(lambda: c5.bwd_stage(4), K, pre=lambda: c5.bwd_stage(1), post=lambda: c5.bwd_stage(5),
                           stats=st_main)
    t_dq = time_launches(lambda: c5.bwd_stage(5), K)
    t_pre = time_graph(lambda: c5.bwd_stage(1), 10, max(3, K // 4))
    t_amain = time_launches(lambda: c5.bwd_stage(2), K, pre=lambda: c5.bwd_stage(1), post=lambda: c5.bwd_stage(3))
    t_fin = time_graph(lambda: c5.bwd_stage(3), 10, max(3, K // 4))
    ws_full = c5.ws
    c5.ws = fa.workspace_for(c5.d["q"])  # base workspace only: fa_bwd takes the atomic route
    t_atomic = time_launches(lambda: c5.bwd_stage(0), max(3, K // 4))
    t_det = time_launches(lambda: c5.bwd_stage("deterministic"), max(3, K // 4))
    c5.ws = ws_full
    B, S, H, D = c5.w.batch, c5.w.seqlen_q, c5.w.heads_q, c5.w.headdim
    fin_bytes = B * S * H * D * (4 + 2)               # read fp32 acc, write dQ
    # the main loop of the stored-dS route does 4 of the 5 products (the dQ product is the
    # dQ pass's): its algorithmic FLOPs are 4/5 of the backward's
    main_flops = 0.8 * c5.bwd_flops
    main_tflops = main_flops / t_main / 1e12
    # stored dS: one 16-bit value per (query row, key) pair a 256-key block's step range
    # covers, written once by the main loop and read once by the dQ pass
    kb = 256
    ds_pairs = B * H * sum(S - min(S, j * kb) for j in range((S + kb - 1) // kb)) * kb
    # fp32 dQ atomics of the atomic route: one per (query row, head, column, 256-key block)
    n_atomics = B * H * D * sum(S - min(S, j * kb) for j in range((S + kb - 1) // kb))
    detail[c5.w.name] = {
        "fwd_tflops": c5.fwd_flops / t_fwd / 1e12,
        "fwd_pct_peak": 100 * c5.fwd_flops / t_fwd / 1e12 / PEAK_TFLOPS,
        "bwd_tflops": c5.bwd_flops / t_bwd / 1e12,
        "bwd_pct_peak": 100 * c5.bwd_flops / t_bwd / 1e12 / PEAK_TFLOPS,
        "fwd_us": t_fwd * 1e6, "bwd_us": t_bwd * 1e6,
        "bwd_pre_us": t_pre * 1e6, "bwd_main_us": t_main * 1e6, "bwd_dq_from_ds_us": t_dq * 1e6,
        "fwd_us_median": st_fwd["median"] * 1e6, "fwd_us_min": st_fwd["min"] * 1e6,
        "bwd_main_us_median": st_main["median"] * 1e6, "bwd_main_us_min": st_main["min"] * 1e6,
        "bwd_dq_from_ds_gbs": 2 * ds_pairs / t_dq / 1e9, "bwd_ds_bytes": 2 * ds_pairs,
        "bwd_atomic_route_us": t_atomic * 1e6, "bwd_atomic_route_tflops": c5.bwd_flops / t_atomic / 1e12,
        "bwd_atomic_main_us": t_amain * 1e6, "bwd_fin_us": t_fin * 1e6, "bwd_fin_gbs": fin_bytes / t_fin / 1e9,
        "bwd_deterministic_recompute_us": t_det * 1e6,
        "bwd_atomic_main_dq_atomics": n_atomics,
        # the atomic main loop against the time its atomics need at the chip's rate (16 adds per request)
        "bwd_atomic_main_floor_us": n_atomics / 16 / ATOMIC_REQ_PER_S * 1e6,
        "bwd_atomic_main_vs_floor": n_atomics / 16 / ATOMIC_REQ_PER_S / t_amain,
    }
    log(f"[bench] backward {t_bwd * 1e6:.1f} us (pre {t_pre * 1e6:.1f}, main {t_main * 1e6:.1f}, dQ from dS "
        f"{t_dq * 1e6:.1f}); atomic route {t_atomic * 1e6:.1f} us (main {t_amain * 1e6:.1f})")
    del c5
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a bounded sample")
        cpu = cpu_baseline()

    traffic = measured_traffic()
    rec = {
        "metric": "attention TFLOPS (fwd, fwd+bwd) & % of MI355X bf16 MFMA peak",
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fwdbwd_causal_mha_b2_h16_s4096_d128_bf16", "batch": 2, "heads_q": 16, "heads_kv": 16,
                   "seqlen_q": 4096, "seqlen_k": 4096, "headdim": 128, "causal": True, "pct_peak": 100 * value /
                   PEAK_TFLOPS},
        "roofline": {"bound": "mfma", "achieved": main_tflops, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": main_tflops / PEAK_TFLOPS, "traffic": traffic,
                     "traffic_note": ("HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE counter "
                                      "summary of this kernel source, scaled by a 512 MiB copy; not measured in "
                                      "this run") if traffic is not None else "no counter summary for this source",
                     "kernel": "bwd_main_k256_kernel<D=128, bf16, causal, padded, no dQ> storing dS "
                               "(4 of the backward's 5 products)"},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
