"""GPU parity of fa_bwd against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
from tests._parity import GRAD_TOL, REPORT, THREADS, dev, f64, say

pytestmark = pytest.mark.gpu


def rel_fro(got, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def run_fwd_bwd(w, x, poison=True, deterministic=False, stored_ds=False):
    """Forward, then the backward through the C ABI: with ``stored_ds`` the workspace holds
    the stored-dS area (fa_bwd takes that route), without it only the base workspace (the
    atomic route, or the recompute route when deterministic or above a 128-wide tile)."""
    d = dev(x)
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=d["cu_seqlens_q"], cu_seqlens_k=d["cu_seqlens_k"], max_seqlen_q=w.seqlen_q,
                  max_seqlen_k=w.seqlen_k)
    mk = dict(window_size=w.window, alibi_slopes=d.get("alibi_slopes"))
    out, lse = fa.forward(d["q"], d["k"], d["v"], causal=w.causal, scale=w.softmax_scale, **mk, **kw)
    if poison:
        dq = torch.full_like(d["q"], float("nan"))
        dk = torch.full_like(d["k"], float("nan"))
        dv = torch.full_like(d["v"], float("nan"))
    else:
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    ws = fa.workspace_for(d["q"], d.get("cu_seqlens_q"), w.seqlen_q if w.varlen else None, d["k"],
                          w.seqlen_k if w.varlen else None, stored_ds)
    if stored_ds:
        B = len(w.lengths_q) if w.varlen else w.batch
        assert ws.numel() > fa.fa_bwd_workspace_bytes(B, w.seqlen_q, w.heads_q, w.headdim), "no stored-dS area"
    ws.fill_(0xFF)  # the workspace's contents on entry must not matter (16-bit NaN in the dS area)
    run = fa.fa_bwd_deterministic if deterministic else fa.fa_bwd
    run(d["do"], d["q"], d["k"], d["v"], out, lse, dq, dk, dv, ws, causal=w.causal, scale=w.softmax_scale, **mk,
        **kw)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def check_grads(w, x, dq, dk, dv, heads=None):
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=x["cu_seqlens_q"].numpy(), cu_seqlens_k=x["cu_seqlens_k"].numpy())
    slopes = x["alibi_slopes"].numpy() if "alibi_slopes" in x else None
    with threadpool_limits(1):  # the oracle threads over heads; BLAS one thread each
        ref = orc.backward(f64(x["do"]), f64(x["q"]), f64(x["k"]), f64(x["v"]), scale=w.softmax_scale,
                           causal=w.causal, threads=THREADS, heads=heads, window=w.window, alibi_slopes=slopes,
                           **kw)
    got = [f64(t) for t in (dq, dk, dv)]
    for g, name in zip(got, ("dq", "dk", "dv")):
        assert np.isfinite(g).all(), f"{w.name}: non-finite {name} (unwritten or NaN)"
    if heads is not None:
        # padded MHA only: compare the listed (sequence, head) slices of dq, dk, dv
        assert not w.varlen and w.heads_q == w.heads_kv
        errs = []
        for i in range(3):
            g = np.concatenate([got[i][b, :, h].ravel() for b, h in heads])
            r = np.concatenate([ref[i][b, :, h].ravel() for b, h in heads])
            errs.append(rel_fro(g, r))
    else:
        errs = [rel_fro(g, r) for g, r in zip(got, ref)]
    tol = GRAD_TOL[w.dtype]
    assert max(errs) <= tol, f"{w.name}: rel Frobenius (dq, dk, dv) = {errs} > {tol}"
    return errs


def W(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=0, lengths=None, scale=None, window=(-1, -1), alibi=None):
    if lengths is not None:
        lq, lk = lengths
        return synth.Workload(name, len(lq), Hq, Hkv, max(max(lq), 1), max(max(lk), 1), D, dtype, causal,
                              backward=True, lengths_q=list(lq), lengths_k=list(lk), seed=seed, scale=scale,
                              window=window, alibi=alibi)
    return synth.Workload(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, backward=True, seed=seed, scale=scale,
                          window=window, alibi=alibi)


def _full(w, deterministic=False, stored_ds=False):
    x = synth.make_inputs(w)
    say(f"bwd{' det' if deterministic else ''}{' ds' if stored_ds else ''} {w.name} B={w.batch} Hq={w.heads_q} "
        f"Hkv={w.heads_kv} Sq={w.seqlen_q} Sk={w.seqlen_k} D={w.headdim} {w.dtype} causal={w.causal} "
        f"varlen={w.varlen}")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, deterministic=deterministic, stored_ds=stored_ds)
    return check_grads(w, x, dq, dk, dv)


# the two routes of fa_bwd: the workspace with the stored-dS area, and the base workspace
ROUTES = ["ds", "base"]


@pytest.mark.parametrize("route", ROUTES)
def test_workload5_full(route):
    """Workload 5 at full size: dQ, dK and dV of all 32 (sequence, head) pairs against the
    oracle's gradients, from the GPU's own forward outputs, on both routes."""
    w, x = synth.draw_config(5)
    say(f"bwd {w.name} (full tensor, route {route})")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, stored_ds=route == "ds")
    errs = check_grads(w, x, dq, dk, dv)
    msg = (f"workload 5 ({w.name}) backward, {'stored-dS' if route == 'ds' else 'atomic'} route: "
           f"rel-Frobenius (dq, dk, dv) = " + ", ".join(f"{e:.3e}" for e in errs))
    print(msg)
    REPORT.append(msg)


def test_workload3_backward_full():
    """The GQA workload at full size (B=2, Hq=32, Hkv=8, S=8192, causal, bf16) through the
    stored-dS route (8 GiB of dS tiles): dQ of all 64 (sequence, query head) pairs and dK,
    dV of all 16 (sequence, KV head) pairs, each summed over its four query heads, against
    the oracle's gradients, from the GPU's own forward outputs."""
    w = synth.config(3)
    w.backward = True  # the same q, k, v draws as the forward workload, then dO
    x = synth.make_inputs(w)
    say(f"bwd {w.name} (full tensor, stored-dS route)")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, stored_ds=True)
    errs = check_grads(w, x, dq, dk, dv)
    msg = (f"workload 3 ({w.name}) backward, stored-dS route: rel-Frobenius (dq, dk, dv) = "
           + ", ".join(f"{e:.3e}" for e in errs))
    print(msg)
    REPORT.append(msg)


def test_workload4_backward_full():
    """The packed variable-length workload at full size (16 sequences of 128..4096 tokens,
    H=8, D=256, fp16, causal) through the stored-dS route, whose D = 256 main loop holds 128
    keys per workgroup: dQ, dK, dV of every token and head against the oracle."""
    w, x = synth.draw_config(4)
    w.backward = True
    rng = np.random.default_rng(4000 + w.seed)  # dO, drawn after the workload's q, k, v
    x["do"] = synth._cast(rng.standard_normal(tuple(x["q"].shape), dtype=np.float32), w.dtype)
    say(f"bwd {w.name} (full tensor, stored-dS route)")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, stored_ds=True)
    errs = check_grads(w, x, dq, dk, dv)
    msg = (f"workload 4 ({w.name}) backward, stored-dS route: rel-Frobenius (dq, dk, dv) = "
           + ", ".join(f"{e:.3e}" for e in errs))
    print(msg)
    REPORT.append(msg)


def test_d256_s8192_backward_full():
    """The head-dimension-256 workload the benchmark times beside the five (B=1, H=16,
    S=8192, D=256, bf16, causal) at full size through the stored-dS route: dQ, dK, dV of
    every head against the oracle."""
    w = W("fwdbwd_causal_b1_h16_s8192_d256_bf16", 1, 16, 16, 8192, 8192, 256, "bf16", True, seed=6)
    x = synth.make_inputs(w)
    say(f"bwd {w.name} (full tensor, stored-dS route)")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, stored_ds=True)
    errs = check_grads(w, x, dq, dk, dv)
    msg = (f"D=256 S=8192 ({w.name}) backward, stored-dS route: rel-Frobenius (dq, dk, dv) = "
           + ", ".join(f"{e:.3e}" for e in errs))
    print(msg)
    REPORT.append(msg)


SHAPES = [
    (2, 2, 2, 300, 300),
    (1, 6, 2, 77, 500),
    (1, 4, 1, 500, 77),
    (2, 2, 2, 1, 129),
    (1, 2, 2, 129, 1),
]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sweep(D, dtype, causal, shape, route):
    B, Hq, Hkv, Sq, Sk = shape
    print(_full(W(f"bwd_{dtype}_d{D}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=D + Sq + 1),
                stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(D, causal, route):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    print(_full(W(f"bwd_varlen_d{D}_c{int(causal)}", None, 4, 2, None, None, D, "bf16", causal, seed=8,
                  lengths=(lq, lk)), stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ROUTES)
def test_gqa_long(route):
    print(_full(W("bwd_gqa_1k", 1, 8, 2, 1024, 1024, 128, "bf16", True, seed=9), stored_ds=route == "ds"))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_stored_ds_long_noncausal(D):
    """Several query blocks per workgroup row range and many key blocks per query block
    (S = 1100: five 256-key blocks, nine 128-row dQ workgroups, a ragged tail); the
    deterministic call, which takes the stored-dS route at every head dimension (fa_bwd
    keeps the atomic route at D <= 64)."""
    print(_full(W(f"bwd_ds_long_d{D}", 1, 4, 4, 1100, 1100, D, "bf16", False, seed=D + 40), deterministic=True,
                stored_ds=True))


def test_stored_ds_bitwise_repeatable_and_stages():
    """The stored-dS route has no atomics: two runs give bitwise the same gradients, and
    stages 1, 4, 5 through fa_bwd_stage give exactly what fa_bwd gives."""
    w = W("bwd_ds_repeat", 2, 8, 2, 1500, 1500, 128, "bf16", True, seed=34)
    x = synth.make_inputs(w)
    say("bwd ds bitwise repeat and stages 1, 4, 5")
    out, lse, dq, dk, dv = run_fwd_bwd(w, x, stored_ds=True)
    _, _, dq2, dk2, dv2 = run_fwd_bwd(w, x, stored_ds=True)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    check_grads(w, x, dq, dk, dv)
    d = dev(x)
    grads = [torch.full_like(d[k], float("nan")) for k in ("q", "k", "v")]
    ws = fa.workspace_for(d["q"], k=d["k"], stored_ds=True)
    ws.fill_(0xFF)
    args = (d["do"], d["q"], d["k"], d["v"], out, lse, *grads, ws)
    for stage in (1, 4, 5):
        fa.fa_bwd_stage(stage, *args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(grads[0], dq) and torch.equal(grads[1], dk) and torch.equal(grads[2], dv)
    # stages 4 and 5 refuse a workspace without the dS area
    small = fa.workspace_for(d["q"])
    with pytest.raises(RuntimeError, match="stored-dS"):
        fa.fa_bwd_stage(4, *args[:-1], small, causal=True)


# ---------------------------------------------------------------- deterministic backward

@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES[:3], ids=lambda s: "x".join(map(str, s)))
def test_deterministic_sweep(D, causal, shape, route):
    B, Hq, Hkv, Sq, Sk = shape
    print(_full(W(f"bwd_det_d{D}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, D, "bf16", causal, seed=D + Sq + 2),
                deterministic=True, stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("causal", [False, True])
def test_deterministic_varlen_fp16(causal, route):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    print(_full(W(f"bwd_det_varlen_c{int(causal)}", None, 4, 2, None, None, 128, "fp16", causal, seed=9,
                  lengths=(lq, lk)), deterministic=True, stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ROUTES)
def test_deterministic_is_bitwise_repeatable_and_matches_workload5(route):
    w, x = synth.draw_config(5)
    say(f"bwd det {w.name} route {route}")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, deterministic=True, stored_ds=route == "ds")
    _, _, dq2, dk2, dv2 = run_fwd_bwd(w, x, deterministic=True, stored_ds=route == "ds")
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    print("workload 5 deterministic full-tensor rel-Frobenius:", check_grads(w, x, dq, dk, dv))


def test_sweep_point_d64_s2048_sampled_heads():
    """A sweep point (hidden 2048 as 32 heads of 64, batch 16k / seqlen)."""
    w = W("sweep_d64_s2048", 8, 32, 32, 2048, 2048, 64, "bf16", True, seed=2112)
    x = synth.make_inputs(w)
    say(f"bwd {w.name}")
    _, _, dq, dk, dv = run_fwd_bwd(w, x)
    print(check_grads(w, x, dq, dk, dv, heads=[(0, 0), (7, 31)]))


# ---------------------------------------------------------------- the main loop's key-block queue

def _setup(w, stored_ds=False):
    x = synth.make_inputs(w)
    d = dev(x)
    out, lse = fa.forward(d["q"], d["k"], d["v"], causal=w.causal, scale=w.softmax_scale)
    grads = [torch.full_like(d[k], float("nan")) for k in ("q", "k", "v")]
    ws = fa.workspace_for(d["q"], k=d["k"], stored_ds=stored_ds)
    ws.fill_(0xFF)
    args = (d["do"], d["q"], d["k"], d["v"], out, lse, *grads, ws)
    return x, d, grads, args


@pytest.mark.parametrize("shape", [(3, 8, 4, 2100, 128), (4, 16, 16, 4200, 64)], ids=["108blocks", "1088blocks"])
def test_main_loop_repeated_alone(shape):
    """Stage 2 launched again on its own finds its key-block queue empty (the last
    workgroup empties it): dK/dV come out bitwise the same, dQ accumulates twice."""
    B, Hq, Hkv, S, D = shape
    w = W("queue_repeat", B, Hq, Hkv, S, S, D, "bf16", True, seed=31)
    say(f"bwd queue repeat B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    x, d, (dq, dk, dv), args = _setup(w)
    fa.fa_bwd(*args, causal=True)
    torch.cuda.synchronize()
    dq1, dk1, dv1 = dq.clone(), dk.clone(), dv.clone()
    assert torch.isfinite(dk1).all() and torch.isfinite(dv1).all() and torch.isfinite(dq1).all()
    dk.fill_(float("nan"))
    dv.fill_(float("nan"))
    for stage in (1, 2, 2, 3):
        fa.fa_bwd_stage(stage, *args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk1) and torch.equal(dv, dv1)
    err = rel_fro(f64(dq), 2.0 * f64(dq1))
    assert err <= 1e-2, f"dq after two main loops vs 2 x dq: rel Frobenius {err}"
    if B * Hq * S <= 3 * 8 * 2100:
        check_grads(w, x, dq1, dk1, dv1)


@pytest.mark.parametrize("D", [256, 192])
def test_staged_atomic_route_wide_heads(D):
    """Above a 128-wide tile fa_bwd takes the atomic-free route; stages 1, 2, 3 still run
    the main loop with dQ atomics there, and give the same gradients."""
    w = W(f"bwd_staged_d{D}", 2, 4, 2, 300, 333, D, "bf16", True, seed=33)
    say(f"bwd staged atomic route D={D}")
    x, d, (dq, dk, dv), args = _setup(w)
    for stage in (1, 2, 3):
        fa.fa_bwd_stage(stage, *args, causal=True)
    torch.cuda.synchronize()
    print(check_grads(w, x, dq, dk, dv))


@pytest.mark.parametrize("route", ROUTES)
def test_backward_graph_replays(route):
    """The whole backward captured in a HIP graph (no memset nodes; the queue counters are
    reset by the kernels themselves) and replayed several times, with eager work between
    the replays: every replay matches the eager result."""
    w = W("graph_bwd", 2, 8, 2, 1500, 1500, 128, "bf16", True, seed=32)
    say(f"bwd graph capture and replays, route {route}")
    x, d, (dq, dk, dv), args = _setup(w, stored_ds=route == "ds")
    fa.fa_bwd(*args, causal=True)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv)]
    check_grads(w, x, *ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fa_bwd(*args, causal=True)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_bwd(*args, causal=True)
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dk, ref[1]) and torch.equal(dv, ref[2]), f"replay {rep}: dk/dv differ"
        err = rel_fro(f64(dq), f64(ref[0]))
        assert err <= 1e-3, f"replay {rep}: dq rel Frobenius {err}"
        fa.fa_bwd(*args, causal=True)  # eager work between replays
        torch.cuda.synchronize()
