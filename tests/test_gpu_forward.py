"""GPU parity of fa_fwd against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import synth
from tests._parity import (REPORT, check_forward_sampled, compare_forward, f64, oracle_forward,
                           oracle_forward_all_rows, run_forward, say)

pytestmark = pytest.mark.gpu


def W(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=0, lengths=None, scale=None):
    if lengths is not None:
        lq, lk = lengths
        return synth.Workload(name, len(lq), Hq, Hkv, max(max(lq), 1), max(max(lk), 1), D, dtype, causal,
                              lengths_q=list(lq), lengths_k=list(lk), seed=seed, scale=scale)
    return synth.Workload(name, B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=seed, scale=scale)


def _full_check(w):
    x = synth.make_inputs(w)
    say(f"fwd {w.name} B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} Sq={w.seqlen_q} Sk={w.seqlen_k} D={w.headdim} "
        f"{w.dtype} causal={w.causal} varlen={w.varlen}")
    o, lse, _ = run_forward(w, x)
    o_ref, lse_ref = oracle_forward(w, x)
    return compare_forward(w, o, lse, o_ref, lse_ref, where=w.name)


# ---------------------------------------------------------------- the reference workloads

def _workload_full(n):
    """Workload n at full size: every row of every (sequence, query head) pair of O and
    the LSE against the oracle (evaluated a chunk of rows at a time)."""
    w, x = synth.draw_config(n)
    say(f"fwd {w.name} (full tensor)")
    o, lse, _ = run_forward(w, x)
    o_ref, lse_ref = oracle_forward_all_rows(w, x)
    assert not np.isnan(o_ref).any() and not np.isnan(lse_ref).any(), "oracle left rows unevaluated"
    err = compare_forward(w, o, lse, o_ref, lse_ref, where=f"{w.name} full tensor")
    msg = (f"workload {n} ({w.name}) forward: max |O - O_ref| = {err[0]:.3e}, max |LSE - LSE_ref| = {err[1]:.3e} "
           f"over all {o_ref.size} outputs")
    print(msg)
    REPORT.append(msg)
    return err


def test_workload1_full():
    _workload_full(1)


def test_workload2_full():
    _workload_full(2)


def test_workload3_full():
    _workload_full(3)


def test_workload4_full():
    _workload_full(4)


def test_workload5_forward_full():
    _workload_full(5)


# ---------------------------------------------------------------- sweep: tiles + ragged tails

SHAPES = [
    # (B, Hq, Hkv, Sq, Sk)
    (2, 2, 2, 300, 300),   # several tiles, ragged tail
    (1, 6, 2, 77, 500),    # GQA 3:1, Sq < Sk (bottom-right causal keeps a wide band)
    (1, 4, 1, 500, 77),    # MQA, Sq > Sk: leading rows fully masked under causal
    (3, 2, 2, 1, 129),     # single query row
    (1, 2, 2, 129, 1),     # single key
]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sweep(D, dtype, causal, shape):
    B, Hq, Hkv, Sq, Sk = shape
    _full_check(W(f"sweep_{dtype}_d{D}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=D + Sq))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(D, causal):
    # includes an empty sequence, a length-1 sequence, Lq != Lk, and lengths off the tile grid
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    _full_check(W(f"varlen_d{D}_c{int(causal)}", None, 4, 2, None, None, D, "bf16", causal, seed=7,
                  lengths=(lq, lk)))


# Block order: with Hq a multiple of 8 each XCD takes Hq/8 query heads of every sequence
# and runs sequences longest first; these cases cover that mapping (equal lengths, an
# empty sequence, lengths off the block grid, GQA groups split over XCDs) and the
# fallback order above 64 packed sequences.
@pytest.mark.parametrize("D", [64, 128, 256])
def test_xcd_order_varlen(D):
    lq = [300, 0, 129, 300, 1, 513, 64, 300, 257]
    lk = [300, 5, 129, 300, 1, 513, 64, 310, 257]
    _full_check(W(f"xcd_varlen_d{D}", None, 8, 2, None, None, D, "bf16", True, seed=21, lengths=(lq, lk)))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_xcd_order_padded(D, causal):
    _full_check(W(f"xcd_padded_d{D}_c{int(causal)}", 2, 16, 4, 520, 520, D, "fp16", causal, seed=22))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_xcd_order_sequence_major_varlen(D):
    # At least four blocks per CU on every XCD (Hq = 8: one head per XCD), so the XCDs run
    # their sequences longest first, ranked on the device: equal lengths, an empty sequence
    # and lengths off the block grid. Non-causal: the order does not depend on the mask, and
    # rows that see hundreds of keys keep the bf16 bar on the kernel rather than on the
    # output rounding of rows that see one or two.
    rng = np.random.default_rng(25)
    lq = [int(x) for x in rng.integers(700, 1100, 40)]
    lq[3] = lq[7] = lq[11] = 900  # ties
    lq[5] = 0
    _full_check(W(f"xcd_seqmajor_varlen_d{D}", None, 8, 2, None, None, D, "bf16", False, seed=25, lengths=(lq, list(lq))))


def test_xcd_order_sequence_major_padded():
    _full_check(W("xcd_seqmajor_padded", 64, 8, 2, 520, 520, 128, "fp16", False, seed=26))


def test_xcd_order_sequence_major_boundary():
    # 15 sequences x 9 query blocks = 135 blocks per XCD, just past four per CU: the first
    # shape that runs sequence-major. Causal with Sk = 2 Sq (bottom-right aligned), so each
    # row sees more than 1,100 keys.
    _full_check(W("xcd_seqmajor_boundary", 15, 8, 2, 1100, 2200, 64, "fp16", True, seed=27))


def test_xcd_order_many_sequences():
    # Non-causal with at least 32 keys per sequence: every output row averages many values,
    # so |O| stays far below 2 and the bf16 bar measures the kernel, not the output
    # rounding of rows that see one or two keys.
    rng = np.random.default_rng(23)
    lq = [int(x) for x in rng.integers(32, 300, 70)]
    _full_check(W("xcd_varlen_70seq", None, 8, 8, None, None, 128, "bf16", False, seed=23, lengths=(lq, list(lq))))
    lq = [int(x) for x in rng.integers(32, 300, 64)]
    _full_check(W("xcd_varlen_64seq", None, 8, 8, None, None, 128, "bf16", False, seed=24, lengths=(lq, list(lq))))


def test_scale_argument():
    _full_check(W("scale_0.05", 1, 2, 2, 200, 333, 128, "bf16", True, seed=11, scale=0.05))
    _full_check(W("scale_0", 1, 2, 2, 65, 97, 64, "fp16", False, seed=12, scale=0.0))


def test_printed_5x2_mask_rows():
    """Sq=5, Sk=2 causal: rows 0-2 keep nothing (printed example) -> O = 0, LSE = +inf."""
    w = W("printed_5x2", 1, 1, 1, 5, 2, 64, "fp16", True, seed=13)
    x = synth.make_inputs(w)
    say("fwd printed 5x2 mask")
    o, lse, _ = run_forward(w, x)
    assert (f64(o)[0, :3] == 0).all()
    assert np.isposinf(f64(lse)[0, 0, :3]).all()
    _full_check(w)


def test_long_sequence_max_headdim():
    w = W("long_16k_d256", 1, 1, 1, 16384, 16384, 256, "bf16", True, seed=14)
    x = synth.make_inputs(w)
    say(f"fwd {w.name}")
    o, lse, _ = run_forward(w, x)
    assert torch.isfinite(o).all().item()
    check_forward_sampled(w, x, o, lse, [(0, 0)], seed=14)


def test_forward_is_bitwise_deterministic():
    w = W("det", 2, 4, 2, 700, 700, 128, "bf16", True, seed=15)
    x = synth.make_inputs(w)
    say("fwd determinism")
    o1, l1, _ = run_forward(w, x)
    o2, l2, _ = run_forward(w, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_sweep_point_d64_s16k_sampled():
    """The longest point of the head-dim / seqlen sweep: B=1, 32 heads, S=16384, D=64."""
    w = W("sweep_d64_s16k", 1, 32, 32, 16384, 16384, 64, "bf16", True, seed=16448)
    x = synth.make_inputs(w)
    say(f"fwd {w.name}")
    o, lse, _ = run_forward(w, x)
    assert torch.isfinite(o).all().item()
    check_forward_sampled(w, x, o, lse, [(0, 0), (0, 31)], seed=16)
