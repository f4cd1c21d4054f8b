"""Device-side argument checks (FA_DEBUG_CHECKS=1): cu_seqlens and KV-cache indices that
break the documented preconditions are caught on the device before any attention kernel
touches memory, every kernel then returns at once, and fa_debug_status() reports the
failure.  Every invalid input here is also chosen so that all addresses it could produce
stay inside the tensors' allocations."""

import os

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from tests._parity import compare_forward, oracle_forward, run_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_checks():
    old = os.environ.get("FA_DEBUG_CHECKS")
    os.environ["FA_DEBUG_CHECKS"] = "1"
    fa.fa_debug_status()  # start from a clear flag
    yield
    fa.fa_debug_status()
    if old is None:
        del os.environ["FA_DEBUG_CHECKS"]
    else:
        os.environ["FA_DEBUG_CHECKS"] = old


def _varlen(lq, lk, D=128, seed=41):
    w = synth.Workload("dbg", len(lq), 4, 2, max(lq), max(lk), D, "bf16", True, backward=True, lengths_q=lq,
                       lengths_k=lk, seed=seed)
    return w, synth.make_inputs(w)


def test_valid_varlen_passes(debug_checks):
    w, x = _varlen([100, 0, 257], [90, 5, 300])
    say("debug checks: valid varlen forward")
    o, lse, _ = run_forward(w, x)
    fa.fa_debug_status()
    compare_forward(w, o, lse, *oracle_forward(w, x), where="debug checks on")


def _expect_failure(match):
    with pytest.raises(ValueError, match=match):
        fa.fa_debug_status()
    fa.fa_debug_status()  # reported once, then clear


def test_sequence_longer_than_max_seqlen(debug_checks):
    w, x = _varlen([100, 200], [100, 200])
    d = {k: v.cuda() for k, v in x.items()}
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(fa.lse_shape(d["q"], d["cu_seqlens_q"]), float("nan"), device="cuda")
    say("debug checks: sequence longer than max_seqlen_q (forward)")
    # max_seqlen_q = 150 < 200, so the 300 packed rows exceed B * max_seqlen_q only through
    # the binding's own check; pass 160 rows' worth via a bound that the binding accepts
    fa.fa_fwd(d["q"], d["k"], d["v"], out, lse, causal=True, cu_seqlens_q=d["cu_seqlens_q"],
              cu_seqlens_k=d["cu_seqlens_k"], max_seqlen_q=150, max_seqlen_k=200)
    _expect_failure("longer than max_seqlen_q")
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all(), "a kernel ran after the failed check"


def test_decreasing_cu_seqlens_backward(debug_checks):
    w, x = _varlen([100, 150], [100, 150])
    d = {k: v.cuda() for k, v in x.items()}
    out, lse = fa.forward(d["q"], d["k"], d["v"], causal=True, cu_seqlens_q=d["cu_seqlens_q"],
                          cu_seqlens_k=d["cu_seqlens_k"], max_seqlen_q=150, max_seqlen_k=150)
    fa.fa_debug_status()
    bad = torch.tensor([0, 150, 100], dtype=torch.int32, device="cuda")  # sequence 1 has length -50
    dq, dk, dv = (torch.full_like(d[n], float("nan")) for n in ("q", "k", "v"))
    ws = fa.workspace_for(d["q"], bad, 150)
    say("debug checks: decreasing cu_seqlens (backward)")
    fa.fa_bwd(d["do"], d["q"], d["k"], d["v"], out, lse, dq, dk, dv, ws, causal=True, cu_seqlens_q=bad,
              cu_seqlens_k=bad, max_seqlen_q=150, max_seqlen_k=150)
    _expect_failure("decreases")
    torch.cuda.synchronize()
    assert torch.isnan(dq).all() and torch.isnan(dk).all() and torch.isnan(dv).all()
    # the flag is clear again: a valid call runs
    fa.fa_bwd(d["do"], d["q"], d["k"], d["v"], out, lse, dq, dk, dv, ws, causal=True, cu_seqlens_q=d["cu_seqlens_q"],
              cu_seqlens_k=d["cu_seqlens_k"], max_seqlen_q=150, max_seqlen_k=150)
    fa.fa_debug_status()
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_kvcache_block_table_out_of_range(debug_checks):
    w = synth.KVCacheWorkload("dbg_paged", 2, 1, 8, 2, 128, "bf16", 512, lengths=[300, 512], page=256, seed=42)
    x = {k: v.cuda() for k, v in synth.make_kvcache_inputs(w).items()}
    n_blocks = x["k_cache"].shape[0]
    table = x["block_table"].clone()
    table[1, 1] = n_blocks - 1  # the last block of the allocation: outside the pool passed below
    kc, vc = x["k_cache"][: n_blocks - 1], x["v_cache"][: n_blocks - 1]
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full((2, 8, 1), float("nan"), device="cuda")
    say("debug checks: block-table entry outside the pool")
    fa.fa_fwd_kvcache(x["q"], kc, vc, out, lse, cache_seqlens=x["cache_seqlens"], block_table=table, causal=True,
                      num_splits=1)
    _expect_failure("block-table entry")
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()


def test_checks_off_report_nothing():
    old = os.environ.pop("FA_DEBUG_CHECKS", None)
    try:
        fa.fa_debug_status()
    finally:
        if old is not None:
            os.environ["FA_DEBUG_CHECKS"] = old
