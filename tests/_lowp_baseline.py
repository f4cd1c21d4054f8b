"""Plain attention in the 16-bit input dtype on the CPU: the low-precision baseline of the
README's test criterion (an implementation's error may be at most twice this baseline's).

It is what a framework computes when it runs the textbook formula in bf16/fp16 without
a fused kernel: the score product, the probabilities and the output product are each
rounded to the input dtype (torch's CPU matmul accumulates in fp32 and rounds its result
once); the softmax runs in fp32 on the rounded scores.  Gradients come from torch
autograd through the same rounded graph.  Test infrastructure only: it shares nothing
with the HIP path, and the fp64 oracle stays the reference both are measured against.
"""

from __future__ import annotations

import torch


def attention_lowp(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, causal: bool,
                   scale: float | None = None):
    """q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D], dout like q, all in one 16-bit dtype on the
    CPU (fp64 inputs run the same graph in fp64, which is how its formula is pinned).
    Returns (out, (dq, dk, dv)) in that dtype.  Causal masking is aligned to the
    bottom-right corner (key j kept for query i iff j <= i + Sk - Sq); a query row that
    keeps no key outputs zeros."""
    dt = q.dtype
    acc = torch.float64 if dt == torch.float64 else torch.float32  # the softmax's precision
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = D ** -0.5
    qh = q.detach().permute(0, 2, 1, 3).contiguous().requires_grad_(True)  # [B, Hq, Sq, D]
    kh = k.detach().permute(0, 2, 1, 3).contiguous().requires_grad_(True)  # [B, Hkv, Sk, D]
    vh = v.detach().permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kx = kh.repeat_interleave(G, dim=1)  # query head h reads KV head h // G
    vx = vh.repeat_interleave(G, dim=1)
    s = torch.matmul(qh, kx.transpose(-1, -2).contiguous())  # rounded to dt
    s = s.to(acc) * scale
    keep = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        i = torch.arange(Sq).unsqueeze(1)
        j = torch.arange(Sk).unsqueeze(0)
        keep = j <= i + (Sk - Sq)
    s = s.masked_fill(~keep, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)  # rows that keep no key
    o = torch.matmul(p.to(dt), vx)  # rounded to dt
    loss = (o.to(acc) * dout.detach().permute(0, 2, 1, 3).to(acc)).sum()
    loss.backward()
    out = o.detach().permute(0, 2, 1, 3).contiguous()
    grads = tuple(t.grad.permute(0, 2, 1, 3).contiguous() for t in (qh, kh, vh))
    return out, grads
