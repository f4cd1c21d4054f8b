"""GPU parity of the sliding-window and ALiBi variants (fa_fwd_ex, fa_bwd_ex) with the
fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from tests._parity import check_forward_sampled, compare_forward, f64, oracle_forward, run_forward, say
from tests.test_gpu_backward import W as WB, check_grads, run_fwd_bwd

pytestmark = pytest.mark.gpu


def WF(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=0, lengths=None, window=(-1, -1), alibi=None, scale=None):
    if lengths is not None:
        lq, lk = lengths
        return synth.Workload(name, len(lq), Hq, Hkv, max(max(lq), 1), max(max(lk), 1), D, dtype, causal,
                              lengths_q=list(lq), lengths_k=list(lk), seed=seed, window=window, alibi=alibi,
                              scale=scale)
    return synth.Workload(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=seed, window=window, alibi=alibi,
                          scale=scale)


def _fwd(w):
    x = synth.make_inputs(w)
    say(f"fwd {w.name} B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} Sq={w.seqlen_q} Sk={w.seqlen_k} D={w.headdim} "
        f"{w.dtype} causal={w.causal} window={w.window} alibi={w.alibi} varlen={w.varlen}")
    o, lse, _ = run_forward(w, x)
    o_ref, lse_ref = oracle_forward(w, x)
    return compare_forward(w, o, lse, o_ref, lse_ref, where=w.name), o, lse


def _bwd(w, deterministic=False, stored_ds=False):
    x = synth.make_inputs(w)
    say(f"bwd{' det' if deterministic else ''}{' ds' if stored_ds else ''} {w.name} B={w.batch} Hq={w.heads_q} "
        f"Hkv={w.heads_kv} Sq={w.seqlen_q} Sk={w.seqlen_k} D={w.headdim} {w.dtype} causal={w.causal} "
        f"window={w.window} alibi={w.alibi} varlen={w.varlen}")
    _, _, dq, dk, dv = run_fwd_bwd(w, x, deterministic=deterministic, stored_ds=stored_ds)
    return check_grads(w, x, dq, dk, dv)


SHAPES = [
    (2, 4, 2, 300, 300),   # several tiles and key blocks, ragged tail
    (1, 4, 1, 77, 500),    # Sq < Sk
    (1, 4, 2, 500, 77),    # Sq > Sk: leading rows keep nothing under causal/left windows
]
WINDOWS = [(0, 0), (5, 3), (100, -1), (-1, 40), (130, 70)]


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("window", WINDOWS, ids=lambda w: f"w{w[0]}_{w[1]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_window(window, causal, shape):
    B, Hq, Hkv, Sq, Sk = shape
    _fwd(WF(f"fwd_win{window}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, 128, "bf16", causal, seed=Sq + window[0],
            window=window))


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fwd_window_headdims(D, dtype):
    _fwd(WF(f"fwd_win_d{D}_{dtype}", 2, 4, 2, 333, 333, D, dtype, True, seed=D, window=(70, -1)))
    _fwd(WF(f"fwd_win2_d{D}_{dtype}", 1, 4, 4, 200, 260, D, dtype, False, seed=D + 1, window=(33, 17)))


@pytest.mark.parametrize("alibi", ["head", "batch_head"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_fwd_alibi(alibi, causal, D):
    _fwd(WF(f"fwd_alibi_{alibi}_c{int(causal)}_d{D}", 2, 4, 2, 300, 280, D, "bf16", causal, seed=D + 7,
            alibi=alibi))


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_alibi_with_window_varlen(causal):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    _fwd(WF(f"fwd_alibi_win_varlen_c{int(causal)}", None, 4, 2, None, None, 128, "fp16", causal, seed=21,
            lengths=(lq, lk), window=(48, 16), alibi="batch_head"))


def test_fwd_window_zero_zero_printed_5x2():
    """window (0, 0) with Sq = 5 > Sk = 2: rows 0-2 keep nothing (hand-written mask)."""
    (err, o, lse) = _fwd(WF("fwd_win00_5x2", 1, 1, 1, 5, 2, 64, "fp16", False, seed=22, window=(0, 0)))
    assert (f64(o)[0, :3] == 0).all() and np.isposinf(f64(lse)[0, 0, :3]).all()


def test_fwd_window_wider_than_sequence_is_no_window():
    """A window at least as long as the sequences is no limit: bitwise the plain result."""
    w = WF("fwd_wide", 2, 4, 2, 300, 300, 128, "bf16", True, seed=23)
    x = synth.make_inputs(w)
    say("fwd wide window vs plain")
    o1, l1, _ = run_forward(w, x)
    w.window = (300, 300)
    o2, l2, _ = run_forward(w, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_long_window_sampled():
    """Sliding window of 1024 on an 8192-token causal sequence (GQA), rows sampled."""
    w = WF("fwd_win1024_s8192", 1, 8, 2, 8192, 8192, 128, "bf16", True, seed=24, window=(1024, 0), alibi="head")
    x = synth.make_inputs(w)
    say(f"fwd {w.name}")
    o, lse, _ = run_forward(w, x)
    assert torch.isfinite(o).all().item()
    print(check_forward_sampled(w, x, o, lse, [(0, 0), (0, 7)], seed=24))


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("route", ["ds", "base"])
@pytest.mark.parametrize("window", WINDOWS, ids=lambda w: f"w{w[0]}_{w[1]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_window(window, causal, shape, route):
    B, Hq, Hkv, Sq, Sk = shape
    print(_bwd(WB(f"bwd_win{window}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, 128, "bf16", causal, seed=Sq + window[1],
                  window=window), stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ["ds", "base"])
@pytest.mark.parametrize("D", [64, 256])
def test_bwd_window_headdims(D, route):
    ds = route == "ds"
    print(_bwd(WB(f"bwd_win_d{D}", 2, 4, 2, 333, 333, D, "bf16", True, seed=D + 3, window=(70, -1)), stored_ds=ds))
    print(_bwd(WB(f"bwd_win2_d{D}", 1, 4, 4, 200, 260, D, "fp16", False, seed=D + 4, window=(33, 17)), stored_ds=ds))


@pytest.mark.parametrize("route", ["ds", "base"])
@pytest.mark.parametrize("alibi", ["head", "batch_head"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_alibi(alibi, causal, D, route):
    print(_bwd(WB(f"bwd_alibi_{alibi}_c{int(causal)}_d{D}", 2, 4, 2, 300, 280, D, "bf16", causal, seed=D + 9,
                  alibi=alibi), stored_ds=route == "ds"))


@pytest.mark.parametrize("route", ["ds", "base"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_alibi_with_window_varlen(causal, route):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    print(_bwd(WB(f"bwd_alibi_win_varlen_c{int(causal)}", None, 4, 2, None, None, 128, "bf16", causal, seed=25,
                  lengths=(lq, lk), window=(48, 16), alibi="head"), stored_ds=route == "ds"))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_deterministic_window_alibi(D):
    w = WB(f"bwd_det_win_alibi_d{D}", 2, 4, 2, 300, 300, D, "bf16", True, seed=D + 11, window=(90, -1),
           alibi="batch_head")
    print(_bwd(w, deterministic=True))
    x = synth.make_inputs(w)
    _, _, dq1, dk1, dv1 = run_fwd_bwd(w, x, deterministic=True)
    _, _, dq2, dk2, dv2 = run_fwd_bwd(w, x, deterministic=True)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
