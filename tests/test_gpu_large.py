"""Tensors past 4 GiB: K and V of one sequence of 65,536 keys whose K/V rows span 64 KiB
(128 heads of dimension 256, or 256 heads of dimension 128), 4 GiB each in bf16, so byte
offsets into them need more than 32 bits.  The forward then runs its generic kernel,
which forms every tile's base address in 64 bits (the ping-pong and key-split kernels
address a sequence's K/V with 32-bit offsets and are not used); the backward runs
unchanged (its buffer resources start at each key block).  Forward and backward through
the C ABI, checked against the fp64 oracle on whole heads (all 256 query rows against all
65,536 keys) of three of the heads.  Likewise a decode call against KV caches of 4 GiB.
The inputs are drawn on the GPU (synth's device recipes) and read back for the oracle."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
from tests import test_gpu_decode as td
from tests._parity import FWD_TOL, GRAD_TOL, LSE_TOL, REPORT, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H, D", [(128, 256), (256, 128)], ids=["h128_d256", "h256_d128"])
def test_kv_past_4gib_forward_backward(H, D):
    w = synth.Workload(f"kv_past_4gib_b1_h{H}_sq256_sk65536_d{D}_bf16_causal", 1, H, H, 256, 65536, D, "bf16", True,
                       backward=True, seed=40 + D)
    assert w.seqlen_k * w.heads_kv * D * 2 >= 1 << 32
    say(w.name)
    d = synth.make_inputs_on_device(w)
    out, lse = fa.forward(d["q"], d["k"], d["v"], causal=True)
    dq, dk, dv = fa.backward(d["do"], d["q"], d["k"], d["v"], out, lse, causal=True)
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0]
    for h in (0, H // 2 + 13, H - 1):
        sl = lambda t: f64(t[:, :, h:h + 1])  # noqa: E731  (batch, seq, this head, D)
        q, k, v, do = (sl(d[n]) for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = orc.forward(q, k, v, causal=True)
        e_o = float(np.abs(sl(out) - o_ref).max())
        e_l = float(np.abs(f64(lse[:, h:h + 1]) - lse_ref).max())
        g_ref = orc.backward(do, q, k, v, causal=True)
        e_g = max(float(np.linalg.norm(sl(g) - r) / np.linalg.norm(r)) for g, r in zip((dq, dk, dv), g_ref))
        print(f"{w.name} head {h}: max|O-O_ref| {e_o:.3e}, max|LSE-LSE_ref| {e_l:.3e}, "
              f"max rel_fro(dq,dk,dv) {e_g:.3e}", flush=True)
        assert e_o <= FWD_TOL["bf16"] and e_l <= LSE_TOL and e_g <= GRAD_TOL["bf16"], (w.name, h, e_o, e_l, e_g)
        worst = [max(a, b) for a, b in zip(worst, (e_o, e_l, e_g))]
    REPORT.append(f"{w.name} (3 whole heads): max |O - O_ref| = {worst[0]:.3e}, max |LSE - LSE_ref| = {worst[1]:.3e}, "
                  f"max rel_fro(dq, dk, dv) = {worst[2]:.3e}")


def test_kvcache_past_4gib():
    # 16 cache entries of 131,072 positions x 8 KV heads x 128 (4 GiB per cache in bf16);
    # sequence b reads entry 15 - b, so the long sequences read the last GiB of each cache.
    lens = [131072, 1, 65537, 131071, 777, 131072, 40000, 4096, 131072, 99999, 8192, 12345, 100, 2, 131072, 70001]
    w = synth.KVCacheWorkload("kvcache_past_4gib_b16_hq32_hkv8_d128_bf16_cache131072", 16, 1, 32, 8, 128, "bf16",
                              131072, causal=True, lengths=lens, batch_idx=[15 - b for b in range(16)], seed=77)
    assert w.capacity * 16 * w.heads_kv * w.headdim * 2 >= 1 << 32
    x = synth.make_kvcache_inputs_on_device(w)
    o, lse, _ = td.run_kvcache(w, x)
    worst = [0.0, 0.0]
    for b in (0, 3, 5, 8, 14, 15):
        e, L = 15 - b, lens[b]
        o_ref, lse_ref = orc.forward_kvcache(f64(x["q"][b:b + 1]), f64(x["k_cache"][e:e + 1, :L]),
                                             f64(x["v_cache"][e:e + 1, :L]), cache_seqlens=np.array([L]),
                                             scale=w.softmax_scale, causal=True)
        e_o = float(np.abs(f64(o[b:b + 1]) - o_ref).max())
        e_l = float(np.abs(f64(lse[b:b + 1]) - lse_ref).max())
        print(f"{w.name} sequence {b} (entry {e}, {L} keys): max|O-O_ref| {e_o:.3e}, max|LSE-LSE_ref| {e_l:.3e}",
              flush=True)
        assert e_o <= FWD_TOL["bf16"] and e_l <= LSE_TOL, (w.name, b, e_o, e_l)
        worst = [max(worst[0], e_o), max(worst[1], e_l)]
    REPORT.append(f"{w.name} (6 whole sequences): max |O - O_ref| = {worst[0]:.3e}, "
                  f"max |LSE - LSE_ref| = {worst[1]:.3e}")
