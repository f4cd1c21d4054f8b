"""The C-ABI library loads, exports every function include/fa.h declares, and rejects
every invalid argument on the host with the documented status before launching
anything (these calls return before any HIP call, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

from exact_tiled_attention_02_amd import build, fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        build.build()
    return fa.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "fa_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libfa.so does not export {n}"


def test_status_strings(L):
    assert L.fa_status_string(0) == b"FA_OK"
    assert L.fa_status_string(1) == b"FA_ERR_INVALID_ARGUMENT"
    assert L.fa_status_string(4) == b"FA_ERR_HIP"
    assert L.fa_status_string(99) == b"unknown fa_status"


P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced by these calls


def _fwd(L, **over):
    a = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Sq=128, Sk=128, Hq=4, Hkv=2, D=128, scale=0.1, causal=1,
             cu_q=None, cu_k=None, dtype=1, stream=None)
    a.update(over)
    return L.fa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"],
                    a["scale"], a["causal"], a["cu_q"], a["cu_k"], a["dtype"], a["stream"])


def _bwd(L, **over):
    a = dict(do=P, q=P, k=P, v=P, out=P, lse=P, dq=P, dk=P, dv=P, B=1, Sq=128, Sk=128, Hq=4, Hkv=2, D=128,
             scale=0.1, causal=1, cu_q=None, cu_k=None, dtype=1, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(over)
    return L.fa_bwd(a["do"], a["q"], a["k"], a["v"], a["out"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["Sq"],
                    a["Sk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["cu_q"], a["cu_k"], a["dtype"],
                    a["ws"], a["ws_bytes"], a["stream"])


INVALID = [
    (dict(Hq=6, Hkv=4), 1),                # heads not divisible
    (dict(D=100), 2),                      # head dimension not a multiple of 8
    (dict(D=264), 2),                      # head dimension above 256
    (dict(D=512), 2),
    (dict(D=0), 1),
    (dict(dtype=7), 2),                    # unknown dtype
    (dict(B=0), 1),
    (dict(Sq=-1), 1),
    (dict(Sk=0), 1),
    (dict(Hkv=0), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(scale=-0.5), 1),
    (dict(cu_q=P, cu_k=None), 1),         # only one cu_seqlens
    (dict(cu_q=None, cu_k=P), 1),
    (dict(cu_q=P + 2, cu_k=P), 1),         # misaligned cu_seqlens
    (dict(q=None), 1),
    (dict(v=P + 8), 1),                    # misaligned tensor
    (dict(lse=None), 1),
]


@pytest.mark.parametrize("over,status", INVALID, ids=lambda x: str(x))
def test_fwd_rejects(L, over, status):
    assert _fwd(L, **over) == status
    assert L.fa_last_error() != b""


@pytest.mark.parametrize("over,status", INVALID + [
    (dict(dq=None), 1), (dict(dk=P + 4), 1), (dict(do=None), 1),
    (dict(ws=None), 3), (dict(ws_bytes=16), 3), (dict(ws=P + 8), 3),
], ids=lambda x: str(x))
def test_bwd_rejects(L, over, status):
    assert _bwd(L, **over) == status


def test_workspace_bytes(L):
    n = L.fa_bwd_workspace_bytes(2, 4096, 16, 128)
    assert n >= 2 * 4096 * 16 * 128 * 4 + 2 * 4096 * 16 * 4
    assert n % 256 == 0
    assert L.fa_bwd_workspace_bytes(0, 1, 1, 1) == 0
    # documented layout: fp32 dQ accumulator, -Dsum and LSE*log2(e) per (row, head), each
    # 256-byte aligned, then 256 bytes of queue counters
    al = lambda x: (x + 255) // 256 * 256
    for B, S, H, D in ((2, 4096, 16, 128), (3, 77, 6, 64), (1, 1, 1, 256)):
        rows = B * S
        assert L.fa_bwd_workspace_bytes(B, S, H, D) == al(rows * H * D * 4) + 2 * al(rows * H * 4) + 256


def test_python_status_mapping(L):
    fa.check(0)
    for st, exc in ((1, ValueError), (2, ValueError), (3, RuntimeError), (4, RuntimeError)):
        with pytest.raises(exc):
            fa.check(st)


def test_binding_rejects_host_tensors(L):
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q, q.clone(), torch.zeros(1, 2, 8), causal=False)


@pytest.mark.parametrize("stage", [0, 6, -1])
def test_bwd_stage_rejects_bad_stage(L, stage):
    args = [P] * 9 + [1, 128, 128, 4, 2, 128, 0.1, 1, None, None, 1, P, 1 << 40, None]
    assert L.fa_bwd_stage(stage, *args) == 1


def test_ds_workspace_bytes(L):
    """The stored-dS area: B * Hq * ceil(Sq / 32) * ceil(Sk / KB) tiles of 32 x KB 16-bit
    values (KB = 256 keys up to a 128-wide tile, 128 above), 256-byte rounded; 0 for invalid
    sizes and above the 32 GiB cap."""
    for B, Sq, Sk, H, D, kb in ((2, 4096, 4096, 16, 128, 256), (3, 77, 500, 6, 64, 256), (1, 1, 1, 1, 256, 128),
                                (2, 300, 333, 4, 192, 128), (16, 2048, 2048, 8, 40, 256)):
        n = B * H * -(-Sq // 32) * -(-Sk // kb) * 32 * kb * 2
        assert L.fa_bwd_ds_workspace_bytes(B, Sq, Sk, H, D) == (n + 255) // 256 * 256
    assert L.fa_bwd_ds_workspace_bytes(2, 4096, 4096, 16, 128) == 2 * 16 * 4096 * 4096 * 2
    assert L.fa_bwd_ds_workspace_bytes(0, 1, 1, 1, 128) == 0
    assert L.fa_bwd_ds_workspace_bytes(1, 1, 0, 1, 128) == 0
    assert L.fa_bwd_ds_workspace_bytes(1, 1, 1, 1, 100) == 0
    # 1 x 32 x 32768^2 x 2 bytes = 64 GiB: beyond the cap, the route is not offered
    assert L.fa_bwd_ds_workspace_bytes(1, 32768, 32768, 32, 128) == 0
    assert L.fa_bwd_ds_workspace_bytes(1, 32768, 32768, 16, 128) == 32 << 30


@pytest.mark.parametrize("stage", [4, 5])
def test_stored_ds_stages_need_the_area(L, stage):
    """Stages 4 and 5 with only the base workspace return FA_ERR_WORKSPACE before any launch."""
    base = L.fa_bwd_workspace_bytes(1, 128, 4, 128)
    args = [P] * 9 + [1, 128, 128, 4, 2, 128, 0.1, 1, None, None, 1, P, base, None]
    assert L.fa_bwd_stage(stage, *args) == 3
    assert b"stored-dS" in L.fa_last_error()


def test_bwd_stage_validates_like_fa_bwd(L):
    args = [P] * 9 + [1, 128, 128, 6, 4, 128, 0.1, 1, None, None, 1, P, 1 << 40, None]
    assert L.fa_bwd_stage(2, *args) == 1


# ---------------------------------------------------------------------------- KV-cache decode

def _kvc(L, **over):
    a = dict(q=P, k=P, v=P, out=P, lse=P, B=2, Sq=1, Hq=8, Hkv=2, D=128, cache_batch=2, cache_seqlen=4096,
             seqlens=None, batch_idx=None, table=None, max_blocks=0, scale=0.1, causal=1, wl=-1, wr=-1,
             alibi=None, alibi_stride=0, splits=1, dtype=1, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return L.fa_fwd_kvcache(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"],
                            a["cache_batch"], a["cache_seqlen"], a["seqlens"], a["batch_idx"], a["table"],
                            a["max_blocks"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"],
                            a["alibi_stride"], a["splits"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


KVC_INVALID = [
    (dict(Hq=6, Hkv=4), 1),
    (dict(D=84), 2),
    (dict(dtype=3), 2),
    (dict(B=0), 1),
    (dict(Sq=0), 1),
    (dict(cache_seqlen=0), 1),
    (dict(cache_batch=0), 1),
    (dict(scale=float("nan")), 1),
    (dict(q=None), 1),
    (dict(k=P + 8), 1),
    (dict(lse=None), 1),
    (dict(wl=-2), 1),
    (dict(wr=-5), 1),
    (dict(alibi=P, alibi_stride=3), 1),             # neither per-head nor per-(sequence, head)
    (dict(alibi=P + 2), 1),                          # misaligned slopes
    (dict(seqlens=P + 1), 1),
    (dict(table=P, max_blocks=0), 1),                # paged without a block count
    (dict(table=P, max_blocks=4, cache_seqlen=48), 1),  # page size not a multiple of 32
    (dict(table=P, max_blocks=4, cache_seqlen=256, batch_idx=P), 1),  # batch index with pages
    (dict(table=P, max_blocks=4096, cache_seqlen=256, splits=1), 1),  # too many pages per split
    (dict(splits=-1), 1),
    (dict(splits=4, ws=None), 3),                    # several splits need a workspace
    (dict(splits=4, ws=P, ws_bytes=64), 3),
    (dict(splits=4, ws=P + 8, ws_bytes=1 << 40), 3),
]


@pytest.mark.parametrize("over,status", KVC_INVALID, ids=lambda x: str(x))
def test_kvcache_rejects(L, over, status):
    assert _kvc(L, **over) == status
    assert L.fa_last_error() != b""


def test_kvcache_split_heuristic_and_workspace(L):
    # few (sequence, KV head) units and a long cache: many splits, at least 256 keys each
    assert L.fa_fwd_kvcache_num_splits(1, 1, 8, 1, 128, 1 << 17, 0) == 512
    assert L.fa_fwd_kvcache_num_splits(1, 1, 8, 1, 128, 1 << 20, 0) == 1024
    # enough units to fill the GPU by themselves: one split
    assert L.fa_fwd_kvcache_num_splits(512, 1, 64, 8, 128, 8192, 0) == 1
    assert L.fa_fwd_kvcache_num_splits(128, 1, 64, 8, 128, 8192, 0) == 4
    # short cache: at least 256 keys per split
    assert L.fa_fwd_kvcache_num_splits(1, 1, 8, 8, 128, 1024, 0) == 4
    # paged: never more than 64 pages in a split
    for cap, page in ((1 << 17, 256), (1 << 17, 32), (4096, 32)):
        s = L.fa_fwd_kvcache_num_splits(64, 1, 8, 8, 128, cap, page)
        tps = -(-(-(-cap // 32)) // s)
        assert -(-tps * 32 // page) + 1 <= 64
    assert L.fa_fwd_kvcache_workspace_bytes(2, 1, 8, 128, 1) == 0
    n = L.fa_fwd_kvcache_workspace_bytes(2, 3, 8, 128, 5)
    assert n >= 5 * 2 * 3 * 8 * (128 + 1) * 4 and n % 256 == 0


# ---------------------------------------------------------------------------- window / ALiBi entry points

def _fwd_ex(L, **over):
    a = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Sq=128, Sk=128, Hq=4, Hkv=2, D=128, scale=0.1, causal=1, wl=-1,
             wr=-1, alibi=None, stride=0, cu_q=None, cu_k=None, dtype=1, stream=None)
    a.update(over)
    return L.fa_fwd_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"],
                       a["D"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["stride"], a["cu_q"],
                       a["cu_k"], a["dtype"], a["stream"])


def _bwd_ex(L, **over):
    a = dict(do=P, q=P, k=P, v=P, out=P, lse=P, dq=P, dk=P, dv=P, B=1, Sq=128, Sk=128, Hq=4, Hkv=2, D=128,
             scale=0.1, causal=1, wl=-1, wr=-1, alibi=None, stride=0, cu_q=None, cu_k=None, dtype=1, det=0, ws=P,
             ws_bytes=1 << 40, stream=None)
    a.update(over)
    return L.fa_bwd_ex(a["do"], a["q"], a["k"], a["v"], a["out"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                       a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["wl"], a["wr"],
                       a["alibi"], a["stride"], a["cu_q"], a["cu_k"], a["dtype"], a["det"], a["ws"], a["ws_bytes"],
                       a["stream"])


EX_INVALID = INVALID + [
    (dict(wl=-2), 1),
    (dict(wr=-7), 1),
    (dict(alibi=P, stride=3), 1),   # stride must be 0 or Hq
    (dict(alibi=P + 2), 1),         # misaligned slopes
]


@pytest.mark.parametrize("over,status", EX_INVALID, ids=lambda x: str(x))
def test_fwd_ex_rejects(L, over, status):
    assert _fwd_ex(L, **over) == status


@pytest.mark.parametrize("over,status", EX_INVALID + [(dict(ws=None), 3), (dict(ws_bytes=16), 3)],
                         ids=lambda x: str(x))
def test_bwd_ex_rejects(L, over, status):
    assert _bwd_ex(L, **over) == status


# ---------------------------------------------------------------------------- binding shape checks
# The C ABI sees only pointers, so the binding checks every tensor's shape before a call;
# these errors come before any device check, so host tensors exercise them.

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def _fwd_tensors(B=2, Sq=8, Sk=12, Hq=4, Hkv=2, D=64):
    import torch
    q, k, v = _t(B, Sq, Hq, D), _t(B, Sk, Hkv, D), _t(B, Sk, Hkv, D)
    return dict(q=q, k=k, v=v, out=_t(B, Sq, Hq, D), lse=torch.zeros(B, Hq, Sq))


@pytest.mark.parametrize("bad", ["k_batch", "k_dim", "v", "out", "lse"])
def test_binding_forward_shapes(bad):
    import torch
    t = _fwd_tensors()
    if bad == "k_batch":
        t["k"] = t["v"] = _t(3, 12, 2, 64)
    elif bad == "k_dim":
        t["k"] = t["v"] = _t(2, 12, 2, 32)
    elif bad == "v":
        t["v"] = _t(2, 13, 2, 64)
    elif bad == "out":
        t["out"] = _t(2, 8, 4, 32)
    else:
        t["lse"] = torch.zeros(2, 8, 4)  # (B, Sq, Hq) instead of (B, Hq, Sq)
    with pytest.raises(ValueError, match="shape"):
        fa.fa_fwd(t["q"], t["k"], t["v"], t["out"], t["lse"], causal=True)


@pytest.mark.parametrize("bad", ["dout", "dq", "dk", "dv", "lse"])
def test_binding_backward_shapes(bad):
    import torch
    t = _fwd_tensors()
    g = dict(dout=_t(2, 8, 4, 64), dq=_t(2, 8, 4, 64), dk=_t(2, 12, 2, 64), dv=_t(2, 12, 2, 64))
    if bad == "lse":
        t["lse"] = torch.zeros(2, 4, 9)
    else:
        g[bad] = _t(2, 8, 2, 64) if bad in ("dout", "dq") else _t(2, 8, 2, 64)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        fa.fa_bwd(g["dout"], t["q"], t["k"], t["v"], t["out"], t["lse"], g["dq"], g["dk"], g["dv"], ws, causal=True)


def test_binding_varlen_shapes():
    import torch
    q, k = _t(20, 4, 64), _t(30, 2, 64)
    cu = torch.tensor([0, 10, 20], dtype=torch.int32)
    cuk = torch.tensor([0, 15, 30], dtype=torch.int32)
    lse = torch.zeros(4, 20)
    kw = dict(cu_seqlens_q=cu, cu_seqlens_k=cuk, max_seqlen_q=10, max_seqlen_k=15)
    with pytest.raises(ValueError, match="shape"):   # lse is (Hq, total_q)
        fa.fa_fwd(q, k, k.clone(), q.clone(), torch.zeros(20, 4), **kw)
    with pytest.raises(ValueError, match="head dimension"):
        fa.fa_fwd(q, _t(30, 2, 32), _t(30, 2, 32), q.clone(), lse, **kw)
    with pytest.raises(ValueError, match="more rows"):  # 20 packed rows > 2 sequences of at most 8
        fa.fa_fwd(q, k, k.clone(), q.clone(), lse, **dict(kw, max_seqlen_q=8))


def test_binding_kvcache_shapes():
    import torch
    q, kc = _t(2, 1, 8, 64), _t(2, 256, 2, 64)
    with pytest.raises(ValueError, match="shape"):
        fa.fa_fwd_kvcache(q, kc, kc.clone(), _t(2, 1, 8, 32), torch.zeros(2, 8, 1))
    with pytest.raises(ValueError, match="shape"):
        fa.fa_fwd_kvcache(q, kc, kc.clone(), _t(2, 1, 8, 64), torch.zeros(2, 1, 8))
