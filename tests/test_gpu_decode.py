"""GPU parity of fa_fwd_kvcache (split-KV decode against a read-only KV cache) with the
fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
from tests._parity import THREADS, compare_forward, f64, say

pytestmark = pytest.mark.gpu

KW = synth.KVCacheWorkload


def _host_checks(w, x):
    """Indices the kernel trusts are in range before anything is launched."""
    cap = w.capacity
    n_entries = x["k_cache"].shape[0]
    if "cache_seqlens" in x:
        L = x["cache_seqlens"]
        assert int(L.min()) >= 0 and int(L.max()) <= cap
    if "cache_batch_idx" in x:
        i = x["cache_batch_idx"]
        assert int(i.min()) >= 0 and int(i.max()) < n_entries
    if "block_table" in x:
        t = x["block_table"]
        assert t.shape == (w.batch, w.max_blocks) and int(t.min()) >= 0 and int(t.max()) < n_entries


def run_kvcache(w, x, num_splits=0):
    _host_checks(w, x)
    d = {k: v.cuda() for k, v in x.items()}
    B, Sq, Hq, D = d["q"].shape
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
    ns = fa.kvcache_splits(d["q"], d["k_cache"], d.get("block_table"), num_splits)
    n = fa.fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, ns)
    ns = num_splits  # 0: the library's own (window-aware) choice, within the workspace
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda") if n else None  # NaN-poisoned partials
    say(f"kvcache {w.name} B={B} Sq={Sq} Hq={Hq} Hkv={w.heads_kv} D={D} cap={w.capacity} page={w.page} "
        f"splits={ns} causal={w.causal} window={w.window} alibi={w.alibi}")
    fa.fa_fwd_kvcache(d["q"], d["k_cache"], d["v_cache"], out, lse, cache_seqlens=d.get("cache_seqlens"),
                      cache_batch_idx=d.get("cache_batch_idx"), block_table=d.get("block_table"), causal=w.causal,
                      scale=w.softmax_scale, window_size=w.window, alibi_slopes=d.get("alibi_slopes"),
                      num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, ns


def oracle_kvcache(w, x):
    g = lambda k: x[k].numpy() if k in x else None
    return orc.forward_kvcache(f64(x["q"]), f64(x["k_cache"]), f64(x["v_cache"]), cache_seqlens=g("cache_seqlens"),
                               cache_batch_idx=g("cache_batch_idx"), block_table=g("block_table"),
                               scale=w.softmax_scale, causal=w.causal, window=w.window,
                               alibi_slopes=g("alibi_slopes"), threads=THREADS)


def _check(w, num_splits=0):
    x = synth.make_kvcache_inputs(w)
    o, lse, ns = run_kvcache(w, x, num_splits)
    o_ref, lse_ref = oracle_kvcache(w, x)
    err = compare_forward(w, o, lse, o_ref, lse_ref, where=f"{w.name} splits={ns or 'auto'}")
    print(w.name, "splits", ns or "auto", "errors", err)
    return o, lse


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_basic_gqa_ragged_lengths(splits):
    _check(KW("basic", 3, 1, 8, 2, 128, "bf16", 1000, lengths=[1000, 517, 33], seed=1), splits)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_headdim_dtype_causal(D, dtype, causal):
    _check(KW(f"d{D}_{dtype}_c{int(causal)}", 2, 2, 4, 1, D, dtype, 700, causal=causal, lengths=[700, 301],
              seed=D + causal))


@pytest.mark.parametrize("splits", [0, 3])
def test_many_rows_several_row_groups(splits):
    # 16 queries x 8 heads per KV head = 128 packed rows = 4 row groups
    _check(KW("rows128", 2, 16, 16, 2, 128, "bf16", 600, lengths=[600, 129], seed=3), splits)


@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_and_empty_rows(causal):
    """Lengths 0, 1 and around the 32-key tile; under causal with Sq = 4 > length, the
    leading query rows keep no key (O = 0, LSE = +inf), and length 0 keeps nothing."""
    w = KW(f"edges_c{int(causal)}", 7, 4, 4, 2, 64, "fp16", 96, causal=causal, lengths=[0, 1, 2, 31, 32, 33, 96],
           seed=4)
    o, lse = _check(w, 3)
    assert (f64(o)[0] == 0).all() and np.isposinf(f64(lse)[0]).all()
    if causal:
        assert (f64(o)[1, :3] == 0).all() and np.isposinf(f64(lse)[1, :, :3]).all()


def test_cache_batch_index():
    _check(KW("batch_idx", 3, 2, 8, 4, 128, "bf16", 300, cache_batch=5, lengths=[300, 77, 150], batch_idx=[4, 0, 2],
              seed=5), 2)


@pytest.mark.parametrize("page", [32, 256])
@pytest.mark.parametrize("splits", [0, 1])
def test_paged_cache(page, splits):
    w = KW(f"paged{page}", 3, 3, 8, 2, 128, "bf16", 1024, lengths=[1024, 700, 31], page=page, seed=6)
    if splits == 1 and page == 32:
        splits = 0  # one split would need more than 64 pages of 32 keys
    _check(w, splits)


@pytest.mark.parametrize("causal,window", [(True, (100, -1)), (True, (0, -1)), (False, (50, 20)), (False, (-1, 5))])
def test_sliding_window(causal, window):
    _check(KW(f"window_{window[0]}_{window[1]}_c{int(causal)}", 2, 4, 8, 2, 128, "bf16", 900, causal=causal,
              lengths=[900, 333], window=window, seed=7), 4)


@pytest.mark.parametrize("splits", [0, 9])
def test_window_on_long_cache(splits):
    # the window reaches 1000 + Sq keys of an 8192-key cache: the splits cover that span
    _check(KW("window_long", 3, 4, 8, 2, 128, "bf16", 8192, causal=True, lengths=[8192, 5000, 700],
              window=(1000, -1), seed=13), splits)


@pytest.mark.parametrize("alibi", ["head", "batch_head"])
@pytest.mark.parametrize("causal", [False, True])
def test_alibi(alibi, causal):
    _check(KW(f"alibi_{alibi}_c{int(causal)}", 2, 3, 8, 2, 128, "bf16", 800, causal=causal, lengths=[800, 250],
              alibi=alibi, seed=8), 3)


def test_alibi_with_window_paged_fp16_d256():
    _check(KW("alibi_window_paged", 2, 2, 4, 2, 256, "fp16", 512, lengths=[512, 200], page=256, window=(64, -1),
              alibi="head", seed=9), 2)


def test_scale_zero_is_uniform_average():
    _check(KW("scale0", 1, 1, 4, 4, 64, "bf16", 200, scale=0.0, seed=10), 2)


def test_long_cache_128k():
    _check(KW("long128k", 1, 1, 8, 1, 128, "bf16", 131072, seed=11))


def test_bench_decode_workload_full():
    w = synth.decode_workload()
    o, lse = _check(w)


def test_decode_is_bitwise_deterministic():
    w = KW("det", 4, 2, 16, 4, 128, "bf16", 4096, lengths=[4096, 3000, 17, 2048], seed=12)
    x = synth.make_kvcache_inputs(w)
    o1, l1, _ = run_kvcache(w, x, 7)
    o2, l2, _ = run_kvcache(w, x, 7)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
