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


def test_device_draws_follow_their_recipe():
    # run on the CPU generator here: same seed -> same values; slices drawn in order, each
    # a float32 normal rounded once to the 16-bit dtype
    w = synth.Workload("dev", 2, 4, 2, 10, 13, 8, "bf16", True, backward=True, seed=5)
    a = synth.make_inputs_on_device(w, "cpu", chunk_rows=4)
    b = synth.make_inputs_on_device(w, "cpu", chunk_rows=4)
    assert [a[k].shape for k in ("q", "k", "v", "do")] == [(2, 10, 4, 8), (2, 13, 2, 8), (2, 13, 2, 8), (2, 10, 4, 8)]
    assert all(a[k].dtype == torch.bfloat16 and torch.equal(a[k], b[k]) for k in a)
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    q0 = torch.randn((2, 4, 4, 8), generator=g, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(a["q"][:, :4], q0)
    assert not torch.equal(a["k"][:, :10], a["q"][:, :, :2])


def test_device_kvcache_draws_follow_their_recipe():
    w = synth.KVCacheWorkload("devkv", 3, 2, 4, 2, 8, "fp16", 20, lengths=[20, 1, 7], batch_idx=[2, 0, 1], seed=9)
    a = synth.make_kvcache_inputs_on_device(w, "cpu", chunk_rows=8)
    b = synth.make_kvcache_inputs_on_device(w, "cpu", chunk_rows=8)
    assert a["q"].shape == (3, 2, 4, 8) and a["k_cache"].shape == (3, 20, 2, 8) and a["v_cache"].dtype == torch.float16
    assert all(torch.equal(a[k], b[k]) for k in a)
    assert a["cache_seqlens"].tolist() == [20, 1, 7] and a["cache_seqlens"].dtype == torch.int32
    assert a["cache_batch_idx"].tolist() == [2, 0, 1]
    g = torch.Generator(device="cpu")
    g.manual_seed(9)
    q = torch.randn((3, 2, 4, 8), generator=g, dtype=torch.float32).to(torch.float16)
    k0 = torch.randn((3, 8, 2, 8), generator=g, dtype=torch.float32).to(torch.float16)
    assert torch.equal(a["q"], q) and torch.equal(a["k_cache"][:, :8], k0)
