"""Tensors past 4 GiB: K and V of one sequence of 65,536 keys whose K/V rows span 64 KiB
(128 heads of dimension 256, or 256 heads of dimension 128), 4 GiB each in bf16, so byte
offsets into them need more than 32 bits.  The forward then runs its generic kernel,
which forms every tile's base address in 64 bits (the ping-pong and key-split kernels
address a sequence's K/V with 32-bit offsets and are not used); the backward runs
unchanged (its buffer resources start at each key block).  Forward and backward through
the C ABI, checked against the fp64 oracle on whole heads (all 256 query rows against all
65,536 keys) of three of the heads.  The inputs are drawn on the GPU (synth's device
recipe) and read back for the oracle."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
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
