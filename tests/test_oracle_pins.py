"""Pins for the fp64 oracle: each checks it against something other than itself --
values the pages print, closed forms, invariants, finite differences, or an fp64
library routine -- so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle fails at least one test."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_fp64 as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------- masks

@pytest.mark.parametrize("name,lq,lk", [("causal_mask_sq2_sk5.txt", 2, 5), ("causal_mask_sq5_sk2.txt", 5, 2)])
def test_printed_causal_masks(name, lq, lk):
    want = _load_matrix(name).astype(bool)
    got = orc.causal_keep_mask(lq, lk, causal=True)
    np.testing.assert_array_equal(got, want)


def test_not_the_superseded_top_left_mask():
    old = _load_matrix("causal_mask_topleft_v20_sq2_sk5.txt").astype(bool)
    assert not np.array_equal(orc.causal_keep_mask(2, 5, True), old)


def test_noncausal_keeps_everything():
    assert orc.causal_keep_mask(3, 7, causal=False).all()


def test_printed_gqa_head_map():
    m = _load_matrix("gqa_head_map_6q_2kv.txt")
    for h, g in m:
        assert orc.kv_head_of(int(h), 6, 2) == g
    with pytest.raises(ValueError):
        orc.kv_head_of(0, 6, 4)


def test_printed_masks_drive_the_output():
    """The 5x2 printed mask: rows 0-2 keep nothing -> zero output (printed), LSE +inf
    (reading); row 3 keeps key 0 only -> O = v0; row 4 keeps both keys."""
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 5, 8), _rand(rng, 2, 8), _rand(rng, 2, 8)
    o, lse = orc.head_forward(q, k, v, 0.3, causal=True)
    np.testing.assert_array_equal(o[:3], 0.0)
    assert np.all(np.isposinf(lse[:3]))
    np.testing.assert_allclose(o[3], v[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[3], 0.3 * q[3] @ k[0], rtol=1e-14)
    s = 0.3 * k @ q[4]
    w = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    np.testing.assert_allclose(o[4], w @ v, rtol=1e-13)


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal,lq,lk", [(False, 6, 9), (True, 7, 7), (True, 4, 9)])
def test_identical_keys_give_mean_of_kept_values(causal, lq, lk):
    rng = np.random.default_rng(1)
    d = 16
    q = _rand(rng, lq, d)
    krow = _rand(rng, d)
    k = np.tile(krow, (lk, 1))
    v = _rand(rng, lk, d)
    scale = 0.7
    o, lse = orc.head_forward(q, k, v, scale, causal)
    for i in range(lq):
        n = (i + lk - lq + 1) if causal else lk
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=1e-12, atol=1e-14)
        # LSE is the natural log of the sum of exp(scale * q.k) over the n kept keys.
        np.testing.assert_allclose(lse[i], scale * q[i] @ krow + math.log(n), rtol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 5, 8), _rand(rng, 1, 8), _rand(rng, 1, 8)
    o, lse = orc.head_forward(q, k, v, 0.25, causal=False)
    np.testing.assert_allclose(o, np.tile(v[0], (5, 1)), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.25 * q @ k[0], rtol=1e-14)


def test_zero_query_or_zero_scale_is_uniform():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 6, 8), _rand(rng, 6, 8)
    o0, lse0 = orc.head_forward(np.zeros_like(q), k, v, 0.5, causal=False)
    o1, lse1 = orc.head_forward(q, k, v, 0.0, causal=False)
    for o, lse in ((o0, lse0), (o1, lse1)):
        np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (4, 1)), rtol=1e-13)
        np.testing.assert_allclose(lse, math.log(6), rtol=1e-14)


def test_causal_first_row_is_v0():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 9, 8), _rand(rng, 9, 8), _rand(rng, 9, 8)
    o, lse = orc.head_forward(q, k, v, 0.4, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-15)
    np.testing.assert_allclose(lse[0], 0.4 * q[0] @ k[0], rtol=1e-14)


# --------------------------------------------------------------------------- invariants

def test_probability_rows_sum_to_one_and_outputs_stay_in_hull():
    rng = np.random.default_rng(5)
    q, k, v = 3 * _rand(rng, 12, 16), _rand(rng, 20, 16), _rand(rng, 20, 16)
    for causal in (False, True):
        p, lse, keep = orc.head_probabilities(q, k, 0.25, causal)
        assert np.all(np.abs(p.sum(axis=1) - 1) < 1e-12)
        assert np.all(p[~keep] == 0)
        o, _ = orc.head_forward(q, k, v, 0.25, causal)
        for i in range(12):
            vv = v[keep[i]]
            assert np.all(o[i] >= vv.min(axis=0) - 1e-12) and np.all(o[i] <= vv.max(axis=0) + 1e-12)


def test_key_shift_moves_only_the_lse():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 11, 16), _rand(rng, 11, 16)
    u = _rand(rng, 16)
    for causal in (False, True):
        o, lse = orc.head_forward(q, k, v, 0.3, causal)
        o2, lse2 = orc.head_forward(q, k + u, v, 0.3, causal)
        np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + 0.3 * q @ u, rtol=1e-11)


def test_noncausal_key_permutation_invariance():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 13, 16), _rand(rng, 13, 16)
    perm = rng.permutation(13)
    o, lse = orc.head_forward(q, k, v, 0.3, False)
    o2, lse2 = orc.head_forward(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(8)
    B, S, Hq, Hkv, D = 2, 7, 6, 2, 8
    q, k, v = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    o, lse = orc.forward(q, k, v, causal=True)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    o2, lse2 = orc.forward(q, kr, vr, causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    do = _rand(rng, B, S, Hq, D)
    dq, dk, dv = orc.backward(do, q, k, v, causal=True)
    dq2, dkr, dvr = orc.backward(do, q, kr, vr, causal=True)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dkr.reshape(B, S, Hkv, Hq // Hkv, D).sum(axis=3), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dvr.reshape(B, S, Hkv, Hq // Hkv, D).sum(axis=3), rtol=1e-12, atol=1e-13)


def test_varlen_equals_independent_calls():
    rng = np.random.default_rng(9)
    lq, lk = [3, 1, 6], [5, 2, 6]
    Hq, Hkv, D = 4, 2, 8
    q, k, v = _rand(rng, sum(lq), Hq, D), _rand(rng, sum(lk), Hkv, D), _rand(rng, sum(lk), Hkv, D)
    do = _rand(rng, sum(lq), Hq, D)
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    o, lse = orc.forward(q, k, v, causal=True, cu_seqlens_q=cq, cu_seqlens_k=ck)
    dq, dk, dv = orc.backward(do, q, k, v, causal=True, cu_seqlens_q=cq, cu_seqlens_k=ck)
    assert lse.shape == (Hq, sum(lq))
    for b in range(3):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ob, lb = orc.forward(q[None, sq], k[None, sk], v[None, sk], causal=True)
        np.testing.assert_array_equal(o[sq], ob[0])
        np.testing.assert_array_equal(lse[:, sq], lb[0])
        gq, gk, gv = orc.backward(do[None, sq], q[None, sq], k[None, sk], v[None, sk], causal=True)
        np.testing.assert_allclose(dq[sq], gq[0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dk[sk], gk[0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dv[sk], gv[0], rtol=1e-14, atol=1e-15)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    q, k, v, do = (_rand(rng, 2, 9, 4, 8) for _ in range(4))
    a = orc.forward(q, k, v, causal=True, threads=1)
    b = orc.forward(q, k, v, causal=True, threads=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    a = orc.backward(do, q, k, v, causal=True, threads=1)
    b = orc.backward(do, q, k, v, causal=True, threads=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("causal,lq,lk", [(False, 17, 33), (False, 40, 5), (True, 29, 29)])
def test_matches_torch_sdpa_fp64(causal, lq, lk):
    """torch's fp64 CPU scaled_dot_product_attention (its causal flag is top-left
    aligned, so the causal case uses lq == lk, where both conventions agree)."""
    rng = np.random.default_rng(11)
    B, H, D = 2, 3, 32
    q, k, v = _rand(rng, B, lq, H, D), _rand(rng, B, lk, H, D), _rand(rng, B, lk, H, D)
    o, _ = orc.forward(q, k, v, scale=0.2, causal=causal)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=0.2)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- backward

def _fd_grads(f, arrays, h=1e-6):
    out = []
    for a in arrays:
        g = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = a[idx]
            a[idx] = old + h
            fp = f()
            a[idx] = old - h
            fm = f()
            a[idx] = old
            g[idx] = (fp - fm) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("varlen", [False, True])
def test_backward_matches_finite_differences(causal, varlen):
    rng = np.random.default_rng(12)
    Hq, Hkv, D = 4, 2, 4
    if varlen:
        lq, lk = [1, 3, 4], [2, 3, 5]
        cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
        q, k, v = _rand(rng, sum(lq), Hq, D), _rand(rng, sum(lk), Hkv, D), _rand(rng, sum(lk), Hkv, D)
        do = _rand(rng, sum(lq), Hq, D)
        kw = dict(cu_seqlens_q=cq, cu_seqlens_k=ck)
    else:
        q, k, v = _rand(rng, 1, 3, Hq, D), _rand(rng, 1, 5, Hkv, D), _rand(rng, 1, 5, Hkv, D)
        do = _rand(rng, 1, 3, Hq, D)
        kw = {}
    scale = 0.6

    def loss():
        o, _ = orc.forward(q, k, v, scale=scale, causal=causal, **kw)
        return float((o * do).sum())

    fq, fk, fv = _fd_grads(loss, [q, k, v])
    dq, dk, dv = orc.backward(do, q, k, v, scale=scale, causal=causal, **kw)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        assert err < 1e-6, err


def test_backward_invariants():
    rng = np.random.default_rng(13)
    lq, lk, D = 6, 9, 8
    q, k, v, do = _rand(rng, lq, D), _rand(rng, lk, D), _rand(rng, lk, D), _rand(rng, lq, D)
    for causal in (False, True):
        dq, dk, dv = orc.head_backward(q, k, v, do, 0.4, causal)
        # each row of dS sums to zero -> the key gradients sum to zero
        np.testing.assert_allclose(dk.sum(axis=0), 0, atol=1e-12)
        # every live row's probabilities sum to one -> value gradients sum to sum of dO
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
        # shifting every key by u leaves dQ unchanged
        u = _rand(rng, D)
        dq2, _, _ = orc.head_backward(q, k + u, v, do, 0.4, causal)
        np.testing.assert_allclose(dq2, dq, rtol=1e-10, atol=1e-12)
    # identical keys -> attention does not depend on q -> dQ = 0
    k1 = np.tile(k[0], (lk, 1))
    dq, _, _ = orc.head_backward(q, k1, v, do, 0.4, False)
    np.testing.assert_allclose(dq, 0, atol=1e-13)
    # fully masked rows contribute nothing
    dq, dk, dv = orc.head_backward(_rand(rng, 5, D), _rand(rng, 2, D), _rand(rng, 2, D), _rand(rng, 5, D), 0.4, True)
    np.testing.assert_array_equal(dq[:3], 0)


def test_dsum_identity():
    """Dsum_i = sum_d dO_id O_id equals sum_j P_ij dP_ij."""
    rng = np.random.default_rng(14)
    q, k, v, do = _rand(rng, 7, 8), _rand(rng, 10, 8), _rand(rng, 10, 8), _rand(rng, 7, 8)
    p, _, _ = orc.head_probabilities(q, k, 0.5, True)
    o = p @ v
    np.testing.assert_allclose((do * o).sum(axis=1), (p * (do @ v.T)).sum(axis=1), rtol=1e-12)


@pytest.mark.parametrize("causal,lq,lk", [(False, 9, 14), (True, 12, 12), (True, 10, 4), (True, 4, 10)])
def test_rows_forward_matches_whole_head(causal, lq, lk):
    """The row-sampled oracle equals the whole-head oracle on every row subset."""
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, lq, 8), _rand(rng, lk, 8), _rand(rng, lk, 8)
    o, lse = orc.head_forward(q, k, v, 0.35, causal)
    rows = rng.permutation(lq)[: max(1, lq // 2)]
    o2, lse2 = orc.rows_forward(q[rows], rows, k, v, 0.35, causal, lq)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(np.isinf(lse2), np.isinf(lse[rows]))
    fin = np.isfinite(lse2)
    np.testing.assert_allclose(lse2[fin], lse[rows][fin], rtol=1e-14)
