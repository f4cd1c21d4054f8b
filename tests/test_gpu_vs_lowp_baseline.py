"""The README's test criterion ("Tests" section of the FlashAttention README): outputs and
gradients match a reference within numerical tolerance, with a maximum numerical error at
most twice that of a baseline.  The reference here is the fp64 oracle; the baseline is
plain attention computed the way a framework computes it in the 16-bit dtype itself
(tests/_lowp_baseline.py: 16-bit products, fp32 softmax, every intermediate rounded to
the input dtype), on the CPU.  The HIP path's error against the oracle must stay within
twice the baseline's, for O (max abs) and for dQ, dK, dV (relative Frobenius)."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_02_amd import fa, synth
from oracle import attention_fp64 as orc
from tests._lowp_baseline import attention_lowp
from tests._parity import dev, f64, say

pytestmark = pytest.mark.gpu


def _rel(g, r):
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, dtype, causal
    (2, 4, 2, 300, 300, 128, "bf16", True),
    (1, 4, 4, 257, 500, 64, "bf16", False),
    (1, 6, 2, 500, 300, 128, "fp16", True),
    (2, 2, 1, 384, 384, 256, "bf16", True),
    (1, 4, 2, 200, 333, 96, "fp16", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Sk{}_D{}_{}_c{}".format(*c))
def test_error_within_twice_the_lowp_baseline(case):
    B, Hq, Hkv, Sq, Sk, D, dtype, causal = case
    w = synth.Workload("lowp_" + "_".join(map(str, case)), B, Hq, Hkv, Sq, Sk, D, dtype, causal, backward=True,
                       seed=Sq + Sk + D)
    x = synth.make_inputs(w)
    say(f"lowp baseline criterion {w.name}")
    d = dev(x)
    out, lse = fa.forward(d["q"], d["k"], d["v"], causal=causal)
    dq, dk, dv = fa.backward(d["do"], d["q"], d["k"], d["v"], out, lse, causal=causal)
    torch.cuda.synchronize()

    o_ref, _ = orc.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), causal=causal)
    g_ref = orc.backward(f64(x["do"]), f64(x["q"]), f64(x["k"]), f64(x["v"]), causal=causal)
    o_b, g_b = attention_lowp(x["q"], x["k"], x["v"], x["do"], causal=causal)

    e_gpu = float(np.abs(f64(out) - o_ref).max())
    e_base = float(np.abs(f64(o_b) - o_ref).max())
    msg = [f"O max abs: kernel {e_gpu:.3e}, baseline {e_base:.3e}"]
    ok = e_gpu <= 2.0 * e_base
    for name, g, gb, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_b, g_ref):
        eg, eb = _rel(f64(g), r), _rel(f64(gb), r)
        msg.append(f"{name} rel Frobenius: kernel {eg:.3e}, baseline {eb:.3e}")
        ok = ok and eg <= 2.0 * eb
    print("; ".join(msg))
    assert ok, f"{w.name}: error above twice the 16-bit baseline's: " + "; ".join(msg)
