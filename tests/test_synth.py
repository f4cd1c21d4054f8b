"""The seeded generator reproduces the workloads' recipe (lengths, shapes, rounding)."""
import numpy as np
import torch

from exact_tiled_attention_02_amd import synth


def test_varlen_lengths_seed4():
    w = synth.config(4)
    assert w.lengths_q == [3011, 3870, 3626, 2157, 3860, 4002, 3979, 448, 1928, 2538, 1251, 1622,
                           2616, 3310, 2433, 820]
    assert sum(w.lengths_q) == 41471 and w.seqlen_q == 4002


def test_small_config_draws():
    w, x = synth.draw_config(1)
    assert x["q"].shape == (1, 128, 2, 64) and x["q"].dtype == torch.float16
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 128, 2, 64), dtype=np.float32).astype(np.float16)
    np.testing.assert_array_equal(x["q"].numpy(), q)


def test_varlen_cu_seqlens():
    w = synth.Workload("t", 3, 4, 2, 6, 6, 8, "bf16", True, lengths_q=[3, 1, 6], lengths_k=[5, 2, 6])
    x = synth.make_inputs(w)
    assert x["cu_seqlens_q"].tolist() == [0, 3, 4, 10]
    assert x["cu_seqlens_k"].tolist() == [0, 5, 7, 13]
    assert x["q"].shape == (10, 4, 8) and x["k"].shape == (13, 2, 8)


def test_flop_model():
    f, b = synth.flops(synth.config(3))
    assert abs(f - 4 * 2 * 32 * 8192 * 8192 * 128 / 2) < 1
    assert abs(b - 2.5 * f) < 1
