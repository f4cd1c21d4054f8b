"""fa_fwd_kvcache_noalloc (partials in the library's static scratch array) against
fa_fwd_kvcache with a caller workspace, through the C ABI: two calls in a row on one
device, the second with a smaller input, each bitwise equal to the workspace call and
within the oracle's bars."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
from tests._parity import FWD_TOL, LSE_TOL, f64, say

pytestmark = pytest.mark.gpu


def _run_both(w, num_splits=0):
    x = {k: v.cuda() for k, v in synth.make_kvcache_inputs(w).items()}
    B, Sq, Hq, D = x["q"].shape
    kw = dict(cache_seqlens=x.get("cache_seqlens"), block_table=x.get("block_table"), causal=w.causal,
              scale=w.softmax_scale, num_splits=num_splits)
    out_ref, lse_ref = fa.forward_kvcache(x["q"], x["k_cache"], x["v_cache"], **kw)
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    fa.fa_fwd_kvcache_noalloc(x["q"], x["k_cache"], x["v_cache"], out, lse, **kw)
    torch.cuda.synchronize()
    return x, out, lse, out_ref, lse_ref


def _check(w, x, out, lse, out_ref, lse_ref):
    assert torch.equal(out, out_ref), f"{w.name}: output differs from the workspace entry point"
    assert torch.equal(lse, lse_ref), f"{w.name}: LSE differs from the workspace entry point"
    cpu = {k: v.cpu() for k, v in x.items()}
    o_or, l_or = orc.forward_kvcache(f64(cpu["q"]), f64(cpu["k_cache"]), f64(cpu["v_cache"]),
                                     cache_seqlens=cpu["cache_seqlens"].numpy() if "cache_seqlens" in cpu else None,
                                     block_table=cpu["block_table"].numpy() if "block_table" in cpu else None,
                                     scale=w.softmax_scale, causal=w.causal, threads=8)
    assert float(np.abs(f64(out) - o_or).max()) <= FWD_TOL[w.dtype]
    fin = np.isfinite(l_or)
    assert float(np.abs(f64(lse)[fin] - l_or[fin]).max()) <= LSE_TOL


def test_noalloc_two_calls_second_smaller():
    big = synth.KVCacheWorkload("noalloc_big", 8, 2, 16, 4, 128, "bf16", 8192, lengths=[8192, 5000, 1, 7777, 300,
                                                                                      8192, 4096, 2500], seed=51)
    small = synth.KVCacheWorkload("noalloc_small", 3, 1, 8, 8, 64, "fp16", 2048, lengths=[100, 2048, 999], seed=52)
    say("noalloc kvcache: large call")
    x, out, lse, out_ref, lse_ref = _run_both(big)
    splits = fa.kvcache_splits(x["q"], x["k_cache"])
    assert splits > 1, "the large call must go through the scratch array"
    _check(big, x, out, lse, out_ref, lse_ref)
    say("noalloc kvcache: smaller call after it")
    x, out, lse, out_ref, lse_ref = _run_both(small)
    assert fa.kvcache_splits(x["q"], x["k_cache"]) > 1
    _check(small, x, out, lse, out_ref, lse_ref)


def test_noalloc_paged_and_oversized():
    w = synth.KVCacheWorkload("noalloc_paged", 4, 1, 32, 8, 128, "bf16", 4096, lengths=[4096, 17, 2049, 3000],
                              page=256, seed=53)
    say("noalloc kvcache: paged")
    x, out, lse, out_ref, lse_ref = _run_both(w)
    _check(w, x, out, lse, out_ref, lse_ref)
    # an explicit split count whose partials exceed the array is rejected before launch
    B, Sq, Hq, D = 64, 16, 64, 256
    assert fa.fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, 1024) > (64 << 20)
    q = torch.zeros(B, Sq, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, 64, 8, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, Sq, device="cuda")
    with pytest.raises(RuntimeError, match="static scratch"):
        fa.fa_fwd_kvcache_noalloc(q, kc, kc, out, lse, num_splits=1024)
