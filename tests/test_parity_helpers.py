"""CPU checks of the test helpers that evaluate the oracle for the GPU parity tests: the
chunked all-rows evaluation must give exactly the oracle's whole-head forward, and the
report of elements over the bar must count and measure them."""

import numpy as np
import torch

from exact_tiled_attention_02_amd import synth
from oracle import attention_fp64 as orc
from tests._parity import excess_report, f64, oracle_forward, oracle_forward_all_rows


def _same(a, b):
    assert a.shape == b.shape
    assert np.array_equal(np.isposinf(a), np.isposinf(b))
    fin = np.isfinite(b)
    assert np.allclose(a[fin], b[fin], rtol=0, atol=1e-12)


def test_all_rows_equals_forward_padded_gqa():
    w = synth.Workload("h", 2, 6, 2, 70, 90, 64, "bf16", True, seed=3)
    x = synth.make_inputs(w)
    o, lse = oracle_forward_all_rows(w, x, chunk=32)
    o_ref, lse_ref = oracle_forward(w, x)
    _same(o, o_ref)
    _same(lse, lse_ref)


def test_all_rows_equals_forward_varlen_window_alibi():
    w = synth.Workload("h", 3, 4, 2, 50, 60, 32, "fp16", True, lengths_q=[5, 0, 50], lengths_k=[9, 3, 60], seed=4,
                       window=(7, 0), alibi="head")
    x = synth.make_inputs(w)
    o, lse = oracle_forward_all_rows(w, x, chunk=16)
    o_ref, lse_ref = orc.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), scale=w.softmax_scale, causal=True,
                                 cu_seqlens_q=x["cu_seqlens_q"].numpy(), cu_seqlens_k=x["cu_seqlens_k"].numpy(),
                                 window=w.window, alibi_slopes=x["alibi_slopes"].numpy())
    _same(o, o_ref)
    _same(lse, lse_ref)


def test_excess_report_counts_and_ulps():
    ref = np.array([0.5, 5.0, 3.0, -6.0])
    got = ref + np.array([0.0, 0.03125, 0.0, -0.0625])  # 1 ulp at 5 (bf16: 2^-5), 2 ulp at 6 (2^-5 each)
    r = excess_report(got, ref, 1e-2, "bf16")
    assert r.startswith("2 elements over 0.01 (2 with |O_ref| >= 4)")
    assert "1.00..2.00 ulp" in r
    assert excess_report(ref, ref, 1e-2, "bf16") == "no element over the bar"


def test_lowp_baseline_formula_in_fp64():
    """The low-precision baseline's graph, run in fp64, is the oracle's definition: same
    mask alignment, GQA map, scale and gradients (so only its roundings differ)."""
    from tests._lowp_baseline import attention_lowp
    rng = np.random.default_rng(7)
    for (B, Hq, Hkv, Sq, Sk, D, causal) in [(2, 4, 2, 9, 6, 8, True), (1, 3, 1, 5, 11, 16, True),
                                            (1, 2, 2, 7, 7, 8, False)]:
        q = rng.standard_normal((B, Sq, Hq, D))
        k = rng.standard_normal((B, Sk, Hkv, D))
        v = rng.standard_normal((B, Sk, Hkv, D))
        do = rng.standard_normal((B, Sq, Hq, D))
        o, g = attention_lowp(*(torch.from_numpy(a) for a in (q, k, v, do)), causal=causal)
        o_ref, _ = orc.forward(q, k, v, causal=causal)
        g_ref = orc.backward(do, q, k, v, causal=causal)
        assert np.abs(o.numpy() - o_ref).max() < 1e-12
        for a, b in zip(g, g_ref):
            assert np.abs(a.numpy() - b).max() < 1e-11
