"""Pins for the oracle's sliding window, ALiBi bias and KV-cache gather.  As in
test_oracle_pins.py, each check compares the oracle with something other than itself:
masks written out by hand from the pages' rule, closed forms (geometric series of the
ALiBi weights), limits, an fp64 library routine with an explicit additive mask, finite
differences, and contiguous re-constructions of gathered and paged caches."""

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


# --------------------------------------------------------------------------- window

@pytest.mark.parametrize("name,lq,lk,causal,window", [
    ("window_mask_sq4_sk6_l1_r1.txt", 4, 6, False, (1, 1)),
    ("window_mask_sq4_sk6_l2_causal.txt", 4, 6, True, (2, -1)),
    ("window_mask_sq5_sk2_l0_r0.txt", 5, 2, False, (0, 0)),
])
def test_hand_written_window_masks(name, lq, lk, causal, window):
    want = _load_matrix(name).astype(bool)
    np.testing.assert_array_equal(orc.keep_mask(lq, lk, causal, window), want)


@pytest.mark.parametrize("lq,lk", [(7, 7), (3, 9), (9, 3)])
def test_window_special_cases(lq, lk):
    # (-1, -1) is no window; (-1, 0) is the bottom-right causal mask; a window wider than
    # the sequence changes nothing; causal ignores any right bound >= 0.
    np.testing.assert_array_equal(orc.keep_mask(lq, lk, False, (-1, -1)), np.ones((lq, lk), bool))
    np.testing.assert_array_equal(orc.keep_mask(lq, lk, False, (-1, 0)), orc.causal_keep_mask(lq, lk, True))
    big = lq + lk
    np.testing.assert_array_equal(orc.keep_mask(lq, lk, True, (big, big)), orc.causal_keep_mask(lq, lk, True))
    np.testing.assert_array_equal(orc.keep_mask(lq, lk, True, (2, 5)), orc.keep_mask(lq, lk, True, (2, -1)))
    # each row keeps at most left + right + 1 keys
    assert orc.keep_mask(lq, lk, False, (2, 1)).sum(axis=1).max() <= 4


def test_window_zero_zero_selects_one_value():
    """window (0, 0) with lq == lk: query i sees key i alone, so O_i = v_i and
    LSE_i = scale q_i . k_i exactly."""
    rng = np.random.default_rng(20)
    q, k, v = _rand(rng, 6, 8), _rand(rng, 6, 8), _rand(rng, 6, 8)
    o, lse = orc.head_forward(q, k, v, 0.3, False, window=(0, 0))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q * k).sum(axis=1), rtol=1e-14)


def test_window_identical_keys_mean_over_window():
    rng = np.random.default_rng(21)
    lq, lk, d, left = 5, 9, 8, 2
    q, v = _rand(rng, lq, d), _rand(rng, lk, d)
    k = np.tile(_rand(rng, d), (lk, 1))
    o, lse = orc.head_forward(q, k, v, 0.5, True, window=(left, -1))
    for i in range(lq):
        hi = i + lk - lq
        lo = max(0, hi - left)
        np.testing.assert_allclose(o[i], v[lo:hi + 1].mean(axis=0), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[i], 0.5 * q[i] @ k[0] + math.log(hi - lo + 1), rtol=1e-13)


# --------------------------------------------------------------------------- ALiBi

@pytest.mark.parametrize("slope", [0.25, 1.0])
def test_alibi_geometric_weights_single_query(slope):
    """lq = 1, q = 0: key j gets weight r^(lk-1-j), r = exp(-slope); the LSE is the log
    of the geometric sum (1 - r^lk) / (1 - r)."""
    rng = np.random.default_rng(22)
    lk, d = 11, 8
    q, k, v = np.zeros((1, d)), _rand(rng, lk, d), _rand(rng, lk, d)
    o, lse = orc.head_forward(q, k, v, 0.7, False, alibi_slope=slope)
    r = math.exp(-slope)
    w = r ** (lk - 1 - np.arange(lk))
    np.testing.assert_allclose(o[0], (w @ v) / w.sum(), rtol=1e-13)
    np.testing.assert_allclose(lse[0], math.log((1 - r ** lk) / (1 - r)), rtol=1e-13)


def test_alibi_two_sided_geometric_lse():
    """lq = lk = n, q = 0, not causal: row i weights r^|i-j|, so
    LSE_i = ln(sum_{m<=i} r^m + sum_{1<=m<=n-1-i} r^m)."""
    n, slope = 7, 0.4
    rng = np.random.default_rng(23)
    k, v = _rand(rng, n, 4), _rand(rng, n, 4)
    _, lse = orc.head_forward(np.zeros((n, 4)), k, v, 1.0, False, alibi_slope=slope)
    r = math.exp(-slope)
    g = lambda m: (1 - r ** m) / (1 - r)  # sum_{t<m} r^t
    want = [math.log(g(i + 1) + (g(n - i) - 1)) for i in range(n)]
    np.testing.assert_allclose(lse, want, rtol=1e-13)


def test_alibi_sign_and_alignment():
    """A steep slope leaves only the key on the aligned diagonal j = i + lk - lq; a zero
    slope is no bias."""
    rng = np.random.default_rng(24)
    lq, lk = 4, 9
    q, k, v = _rand(rng, lq, 8) * 0.1, _rand(rng, lk, 8) * 0.1, _rand(rng, lk, 8)
    o, _ = orc.head_forward(q, k, v, 0.5, False, alibi_slope=60.0)
    np.testing.assert_allclose(o, v[np.arange(lq) + lk - lq], atol=1e-20 + 1e-24, rtol=1e-20)
    a = orc.head_forward(q, k, v, 0.5, True, alibi_slope=0.0)
    b = orc.head_forward(q, k, v, 0.5, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("causal,window,lq,lk", [(False, (-1, -1), 13, 21), (True, (-1, -1), 17, 17),
                                                 (False, (3, 2), 15, 15), (True, (4, -1), 19, 19)])
def test_alibi_and_window_match_torch_sdpa_with_additive_mask(causal, window, lq, lk):
    """torch's fp64 scaled_dot_product_attention with a float attn_mask adds the mask to the
    scaled scores: give it the ALiBi matrix, with -inf outside the kept set, built here
    from the bias and window rule directly."""
    rng = np.random.default_rng(25)
    B, H, D = 2, 3, 16
    slopes = rng.uniform(0.05, 0.5, size=(B, H))
    q, k, v = _rand(rng, B, lq, H, D), _rand(rng, B, lk, H, D), _rand(rng, B, lk, H, D)
    o, lse = orc.forward(q, k, v, scale=0.25, causal=causal, window=window, alibi_slopes=slopes)
    i = np.arange(lq)[:, None] + lk - lq
    j = np.arange(lk)[None, :]
    keep = np.ones((lq, lk), bool)
    if causal:
        keep &= j <= i
    if window[0] >= 0:
        keep &= j >= i - window[0]
    if window[1] >= 0:
        keep &= j <= i + window[1]
    mask = np.where(keep[None, None], -slopes[:, :, None, None] * np.abs(i - j)[None, None], -np.inf)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask),
                                                           scale=0.25)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-13)
    s = 0.25 * np.einsum("bihd,bjhd->bhij", q, k) + mask
    want = np.log(np.exp(s).sum(axis=-1))
    np.testing.assert_allclose(lse, want, rtol=1e-12)


def test_alibi_slopes_per_head_and_per_sequence():
    """(Hq,) slopes equal the same slopes broadcast to (B, Hq); a (B, Hq) array applies
    row b to sequence b (checked against single-sequence calls)."""
    rng = np.random.default_rng(26)
    B, L, Hq, Hkv, D = 3, 10, 4, 2, 8
    q, k, v = _rand(rng, B, L, Hq, D), _rand(rng, B, L, Hkv, D), _rand(rng, B, L, Hkv, D)
    s1 = rng.uniform(0.1, 1.0, Hq)
    a = orc.forward(q, k, v, causal=True, alibi_slopes=s1)
    b = orc.forward(q, k, v, causal=True, alibi_slopes=np.tile(s1, (B, 1)))
    np.testing.assert_array_equal(a[0], b[0])
    s2 = rng.uniform(0.1, 1.0, (B, Hq))
    o, lse = orc.forward(q, k, v, causal=True, alibi_slopes=s2)
    for bi in range(B):
        ob, lb = orc.forward(q[bi:bi + 1], k[bi:bi + 1], v[bi:bi + 1], causal=True, alibi_slopes=s2[bi])
        np.testing.assert_array_equal(o[bi], ob[0])
        np.testing.assert_array_equal(lse[bi], lb[0])


@pytest.mark.parametrize("causal,window,alibi", [(False, (2, 1), False), (True, (1, -1), True),
                                                 (False, (-1, -1), True)])
def test_backward_with_window_and_alibi_matches_finite_differences(causal, window, alibi):
    rng = np.random.default_rng(27)
    Hq, Hkv, D = 4, 2, 4
    q, k, v = _rand(rng, 1, 4, Hq, D), _rand(rng, 1, 6, Hkv, D), _rand(rng, 1, 6, Hkv, D)
    do = _rand(rng, 1, 4, Hq, D)
    slopes = rng.uniform(0.1, 0.8, Hq) if alibi else None
    kw = dict(scale=0.6, causal=causal, window=window, alibi_slopes=slopes)

    def loss():
        o, _ = orc.forward(q, k, v, **kw)
        return float((o * do).sum())

    grads = []
    for a in (q, k, v):
        g = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = a[idx]
            a[idx] = old + 1e-6
            fp = loss()
            a[idx] = old - 1e-6
            fm = loss()
            a[idx] = old
            g[idx] = (fp - fm) / 2e-6
        grads.append(g)
    got = orc.backward(do, q, k, v, **kw)
    for x, want in zip(got, grads):
        assert np.linalg.norm(x - want) / np.linalg.norm(want) < 1e-6


@pytest.mark.parametrize("causal,lq,lk", [(False, 9, 14), (True, 12, 12), (True, 10, 4)])
def test_rows_forward_with_window_and_alibi_matches_whole_head(causal, lq, lk):
    rng = np.random.default_rng(28)
    q, k, v = _rand(rng, lq, 8), _rand(rng, lk, 8), _rand(rng, lk, 8)
    o, lse = orc.head_forward(q, k, v, 0.35, causal, window=(3, 2), alibi_slope=0.3)
    rows = rng.permutation(lq)[: max(1, lq // 2)]
    o2, lse2 = orc.rows_forward(q[rows], rows, k, v, 0.35, causal, lq, window=(3, 2), alibi_slope=0.3)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(np.isinf(lse2), np.isinf(lse[rows]))
    fin = np.isfinite(lse2)
    np.testing.assert_allclose(lse2[fin], lse[rows][fin], rtol=1e-14)


# --------------------------------------------------------------------------- KV cache

def _cache(rng, Bc, Sc, Hkv, D):
    return _rand(rng, Bc, Sc, Hkv, D), _rand(rng, Bc, Sc, Hkv, D)


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_full_cache_equals_plain_forward(causal):
    rng = np.random.default_rng(30)
    B, Sq, Sc, Hq, Hkv, D = 2, 3, 17, 4, 2, 8
    q = _rand(rng, B, Sq, Hq, D)
    kc, vc = _cache(rng, B, Sc, Hkv, D)
    o, lse = orc.forward_kvcache(q, kc, vc, causal=causal)
    o2, lse2 = orc.forward(q, kc, vc, causal=causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (4, -1))])
def test_kvcache_lengths_and_batch_index(causal, window):
    """Sequence b attends the first cache_seqlens[b] rows of cache entry
    cache_batch_idx[b]; the causal/window alignment uses that length."""
    rng = np.random.default_rng(31)
    B, Sq, Bc, Sc, Hq, Hkv, D = 3, 2, 5, 20, 4, 1, 8
    q = _rand(rng, B, Sq, Hq, D)
    kc, vc = _cache(rng, Bc, Sc, Hkv, D)
    lens = np.array([20, 7, 1], dtype=np.int32)
    idx = np.array([4, 0, 2], dtype=np.int32)
    slopes = rng.uniform(0.1, 0.5, Hq)
    o, lse = orc.forward_kvcache(q, kc, vc, cache_seqlens=lens, cache_batch_idx=idx, causal=causal, window=window,
                                 alibi_slopes=slopes)
    for b in range(B):
        L, e = int(lens[b]), int(idx[b])
        ob, lb = orc.forward(q[b:b + 1], kc[e:e + 1, :L].copy(), vc[e:e + 1, :L].copy(), causal=causal, window=window,
                             alibi_slopes=slopes)
        np.testing.assert_array_equal(o[b], ob[0])
        np.testing.assert_array_equal(lse[b], lb[0])
    # Sq = 2 > L = 1 under causal: query row 0 keeps no key -> zero output, +inf LSE
    if causal:
        np.testing.assert_array_equal(o[2, 0], 0)
        assert np.isposinf(lse[2, :, 0]).all()


def test_kvcache_paged_equals_contiguous():
    """Cut contiguous caches into pages, scatter the pages over a shuffled pool and
    address them through a block table: the result must not change."""
    rng = np.random.default_rng(32)
    B, Sq, Hq, Hkv, D, page, nblk = 3, 4, 4, 2, 8, 8, 5
    cap = page * nblk
    q = _rand(rng, B, Sq, Hq, D)
    kc, vc = _cache(rng, B, cap, Hkv, D)
    lens = np.array([cap, 13, 8], dtype=np.int32)
    pool = B * nblk + 3
    perm = rng.permutation(pool)[: B * nblk].reshape(B, nblk)
    kp, vp = _rand(rng, pool, page, Hkv, D), _rand(rng, pool, page, Hkv, D)
    for b in range(B):
        for t in range(nblk):
            kp[perm[b, t]] = kc[b, t * page:(t + 1) * page]
            vp[perm[b, t]] = vc[b, t * page:(t + 1) * page]
    a = orc.forward_kvcache(q, kc, vc, cache_seqlens=lens, causal=True)
    p = orc.forward_kvcache(q, kp, vp, cache_seqlens=lens, block_table=perm.astype(np.int32), causal=True)
    np.testing.assert_array_equal(a[0], p[0])
    np.testing.assert_array_equal(a[1], p[1])
    with pytest.raises(ValueError):
        orc.forward_kvcache(q, kp, vp, cache_seqlens=np.array([cap + 1, 1, 1]), block_table=perm)


def test_lse_merge_of_key_chunks_equals_whole():
    """Attention over disjoint key chunks merges exactly with the natural-log LSE:
    LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.  (An empty chunk has
    LSE -inf and weight 0.)  This fixes the units the split-key decode relies on."""
    rng = np.random.default_rng(33)
    lq, lk, d = 3, 50, 16
    q, k, v = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d)
    o, lse = orc.head_forward(q, k, v, 0.3, False, alibi_slope=0.05)
    cuts = [0, 7, 7, 31, 50]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b == a:
            parts.append((np.zeros((lq, d)), np.full(lq, -np.inf)))
            continue
        # the chunk's bias is that of its keys' positions in the whole sequence
        bias = orc.alibi_bias(lq, lk, 0.05)[:, a:b]
        s = 0.3 * q @ k[a:b].T + bias
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        parts.append(((e @ v[a:b]) / e.sum(axis=1)[:, None], m + np.log(e.sum(axis=1))))
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    O = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(L, lse, rtol=1e-14)
    np.testing.assert_allclose(O, o, rtol=1e-12, atol=1e-14)
