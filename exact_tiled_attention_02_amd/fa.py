"""Python binding of libfa.so (ctypes).  Argument marshalling only: every step of the
attention computation runs in the HIP kernels behind the C ABI of include/fa.h.
PyTorch supplies device memory and the current stream.

The low-level entry points keep the C names (``fa_fwd``, ``fa_bwd``,
``fa_bwd_workspace_bytes``, ``fa_fwd_kvcache`` ...); ``forward``/``backward``/
``forward_kvcache`` additionally allocate their outputs.
There is no fallback: if libfa.so is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_DTYPE_FP16, FA_DTYPE_BF16 = 0, 1
_DTYPE_CODE = {torch.float16: FA_DTYPE_FP16, torch.bfloat16: FA_DTYPE_BF16}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_tiled_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, i, vp]
        L.fa_fwd.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_bwd_ds_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_bwd_ds_workspace_bytes.restype = sz
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, i, vp, sz, vp]
        L.fa_bwd.restype = i
        L.fa_bwd_deterministic.argtypes = L.fa_bwd.argtypes
        L.fa_bwd_deterministic.restype = i
        L.fa_bwd_stage.argtypes = [i] + L.fa_bwd.argtypes
        L.fa_bwd_stage.restype = i
        L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, i, vp, vp, i, vp]
        L.fa_fwd_ex.restype = i
        L.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, i, vp, vp, i, i,
                                vp, sz, vp]
        L.fa_bwd_ex.restype = i
        L.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp, i, f, i, i, i, vp, i, i, i,
                                     vp, sz, vp]
        L.fa_fwd_kvcache.restype = i
        L.fa_fwd_kvcache_noalloc.argtypes = L.fa_fwd_kvcache.argtypes[:-3] + [vp]
        L.fa_fwd_kvcache_noalloc.restype = i
        L.fa_fwd_kvcache_num_splits.argtypes = [i, i, i, i, i, i, i]
        L.fa_fwd_kvcache_num_splits.restype = i
        L.fa_fwd_kvcache_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_fwd_kvcache_workspace_bytes.restype = sz
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_last_error.argtypes = []
        L.fa_last_error.restype = ctypes.c_char_p
        L.fa_debug_status.argtypes = [vp]
        L.fa_debug_status.restype = i
        _lib = L
    return _lib


def check(status: int) -> None:
    """Map an fa_status to a Python exception (1, 2 -> ValueError; 3, 4 -> RuntimeError)."""
    if status == FA_OK:
        return
    L = lib()
    msg = f"{L.fa_status_string(status).decode()}: {L.fa_last_error().decode()}"
    if status in (FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED):
        raise ValueError(msg)
    raise RuntimeError(msg)


def fa_debug_status(stream=None) -> None:
    """Report the device-side argument checks that FA_DEBUG_CHECKS=1 enables: synchronises
    ``stream`` and raises ValueError naming the failed checks (and clears them), if any."""
    check(lib().fa_debug_status(_stream(stream)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, shape, name):
    """The C ABI cannot see tensor sizes: every tensor's shape is checked here, before a
    pointer reaches a kernel that would read or write past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _geometry(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k):
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    if cu_seqlens_q is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("padded q/k/v are (batch, seqlen, heads, headdim)")
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
        if k.shape[0] != B or k.shape[3] != D:
            raise ValueError(f"k has shape {tuple(k.shape)}: batch and head dimension must match q {tuple(q.shape)}")
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("varlen q/k/v are (total, heads, headdim)")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen calls need max_seqlen_q and max_seqlen_k")
        for c in (cu_seqlens_q, cu_seqlens_k):
            if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
                raise ValueError("cu_seqlens must be contiguous 1-D int32 GPU tensors")
        B = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        Sq, Sk = int(max_seqlen_q), int(max_seqlen_k)
        Hq, D = q.shape[1], q.shape[2]
        Hkv = k.shape[1]
        if k.shape[2] != D:
            raise ValueError(f"k has shape {tuple(k.shape)}: head dimension must match q {tuple(q.shape)}")
        # Each sequence is at most max_seqlen long, so B * max_seqlen bounds the packed rows
        # the kernels may address; more rows than that cannot be covered by the launch.
        if q.shape[0] > B * Sq or k.shape[0] > B * Sk:
            raise ValueError("packed q/k hold more rows than batch * max_seqlen")
    if q.device != k.device:
        raise ValueError("q and k live on different devices")
    return B, Sq, Sk, Hq, Hkv, D


def _dtype(*ts):
    d = ts[0].dtype
    if d not in _DTYPE_CODE:
        raise ValueError(f"dtype {d} is not float16/bfloat16")
    for t in ts:
        if t.dtype != d:
            raise ValueError("q, k, v (and dout, out) must share one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
    return _DTYPE_CODE[d]


def _same_device(q, *ts):
    for t in ts:
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise ValueError(f"a tensor lives on {t.device}, q on {q.device}")


def _check_shapes(q, k, lse, cu_seqlens_q, **like):
    """v and dk/dv must have k's shape; out, dout and dq q's; lse the shape lse_shape()
    gives; every tensor on q's device."""
    _expect(lse, lse_shape(q, cu_seqlens_q), "lse")
    for name, t in like.items():
        _expect(t, k.shape if name in ("v", "dk", "dv") else q.shape, name)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 GPU tensor")
    for name, t in list(like.items()) + [("lse", lse)]:
        if t.device != q.device:
            raise ValueError(f"{name} lives on {t.device}, q on {q.device}")


def _alibi_stride(alibi_slopes, B, Hq):
    """Batch stride of an ALiBi slope tensor: (Hq,) -> 0, (B, Hq) -> Hq."""
    if alibi_slopes is None:
        return 0
    if alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_contiguous() or not alibi_slopes.is_cuda:
        raise ValueError("alibi_slopes must be a contiguous float32 GPU tensor")
    if tuple(alibi_slopes.shape) == (Hq,):
        return 0
    if tuple(alibi_slopes.shape) == (B, Hq):
        return Hq
    raise ValueError("alibi_slopes is (nheads,) or (batch, nheads)")


def _plain(window_size, alibi_slopes) -> bool:
    return alibi_slopes is None and tuple(window_size) == (-1, -1)


def fa_fwd(q, k, v, out, lse, causal: bool = False, scale: float | None = None, cu_seqlens_q=None,
           cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, stream=None, window_size=(-1, -1),
           alibi_slopes=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream); writes out, lse.
    ``window_size`` = (left, right) sliding window (-1: unbounded); ``alibi_slopes`` fp32
    (Hq,) or (B, Hq).  Without either this is the C ``fa_fwd``, else ``fa_fwd_ex``."""
    B, Sq, Sk, Hq, Hkv, D = _geometry(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    _check_shapes(q, k, lse, cu_seqlens_q, v=v, out=out)
    dt = _dtype(q, k, v, out)
    _same_device(q, cu_seqlens_q, cu_seqlens_k, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if _plain(window_size, alibi_slopes):
        check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, float(scale),
                           int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), dt, _stream(stream)))
        return
    stride = _alibi_stride(alibi_slopes, B, Hq)
    check(lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, float(scale),
                          int(bool(causal)), int(window_size[0]), int(window_size[1]), _ptr(alibi_slopes), stride,
                          _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), dt, _stream(stream)))


def fa_bwd_workspace_bytes(B: int, Sq: int, Hq: int, D: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, Sq, Hq, D))


def fa_bwd_ds_workspace_bytes(B: int, Sq: int, Sk: int, Hq: int, D: int) -> int:
    """Extra workspace of the stored-dS backward route (0: not available at this size)."""
    return int(lib().fa_bwd_ds_workspace_bytes(B, Sq, Sk, Hq, D))


def fa_bwd(dout, q, k, v, out, lse, dq, dk, dv, workspace, causal: bool = False, scale: float | None = None,
           cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, stream=None,
           window_size=(-1, -1), alibi_slopes=None) -> None:
    """Enqueue the backward; writes dq, dk, dv.  ``workspace``: a uint8 device tensor of
    at least fa_bwd_workspace_bytes(B, Sq, Hq, D) bytes (plus fa_bwd_ds_workspace_bytes
    for the stored-dS route; :func:`workspace_for`).  With a window or ALiBi this is the
    C ``fa_bwd_ex``."""
    if _plain(window_size, alibi_slopes):
        fa_bwd_stage(0, dout, q, k, v, out, lse, dq, dk, dv, workspace, causal, scale, cu_seqlens_q, cu_seqlens_k,
                     max_seqlen_q, max_seqlen_k, stream)
    else:
        _bwd_ex(False, dout, q, k, v, out, lse, dq, dk, dv, workspace, causal, scale, cu_seqlens_q, cu_seqlens_k,
                max_seqlen_q, max_seqlen_k, stream, window_size, alibi_slopes)


def _bwd_args(dout, q, k, v, out, lse, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
              max_seqlen_k):
    B, Sq, Sk, Hq, Hkv, D = _geometry(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    _check_shapes(q, k, lse, cu_seqlens_q, v=v, out=out, dout=dout, dq=dq, dk=dk, dv=dv)
    dt = _dtype(q, k, v, out, dout, dq, dk, dv)
    _same_device(q, cu_seqlens_q, cu_seqlens_k)
    if not workspace.is_cuda or workspace.device != q.device:
        raise ValueError("workspace must live in GPU memory on q's device")
    return B, Sq, Sk, Hq, Hkv, D, dt


def _bwd_ex(deterministic, dout, q, k, v, out, lse, dq, dk, dv, workspace, causal, scale, cu_seqlens_q,
            cu_seqlens_k, max_seqlen_q, max_seqlen_k, stream, window_size, alibi_slopes):
    B, Sq, Sk, Hq, Hkv, D, dt = _bwd_args(dout, q, k, v, out, lse, dq, dk, dv, workspace, cu_seqlens_q,
                                          cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stride = _alibi_stride(alibi_slopes, B, Hq)
    check(lib().fa_bwd_ex(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                          B, Sq, Sk, Hq, Hkv, D, float(scale), int(bool(causal)), int(window_size[0]),
                          int(window_size[1]), _ptr(alibi_slopes), stride, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                          dt, int(bool(deterministic)), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)))


def fa_bwd_stage(stage, dout, q, k, v, out, lse, dq, dk, dv, workspace, causal: bool = False,
                 scale: float | None = None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                 max_seqlen_k=None, stream=None) -> None:
    """Enqueue one backward stage (1 preprocess, 2 main loop with dQ atomics, 3 finalize,
    4 main loop storing dS, 5 dQ from the stored dS); stage 0 runs the whole backward
    (``fa_bwd``)."""
    B, Sq, Sk, Hq, Hkv, D, dt = _bwd_args(dout, q, k, v, out, lse, dq, dk, dv, workspace, cu_seqlens_q,
                                          cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = (_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, Sq, Sk,
            Hq, Hkv, D, float(scale), int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), dt, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if stage == 0:
        check(lib().fa_bwd(*args))
    elif stage == "deterministic":
        check(lib().fa_bwd_deterministic(*args))
    else:
        check(lib().fa_bwd_stage(int(stage), *args))


def fa_bwd_deterministic(dout, q, k, v, out, lse, dq, dk, dv, workspace, causal: bool = False,
                         scale: float | None = None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                         max_seqlen_k=None, stream=None, window_size=(-1, -1), alibi_slopes=None) -> None:
    """Enqueue the deterministic backward (dQ by a separate pass, no atomics)."""
    if _plain(window_size, alibi_slopes):
        fa_bwd_stage("deterministic", dout, q, k, v, out, lse, dq, dk, dv, workspace, causal, scale, cu_seqlens_q,
                     cu_seqlens_k, max_seqlen_q, max_seqlen_k, stream)
    else:
        _bwd_ex(True, dout, q, k, v, out, lse, dq, dk, dv, workspace, causal, scale, cu_seqlens_q, cu_seqlens_k,
                max_seqlen_q, max_seqlen_k, stream, window_size, alibi_slopes)


def lse_shape(q, cu_seqlens_q=None):
    if cu_seqlens_q is None:
        B, Sq, Hq, _ = q.shape
        return (B, Hq, Sq)
    return (q.shape[1], q.shape[0])


def forward(q, k, v, causal: bool = False, scale: float | None = None, cu_seqlens_q=None, cu_seqlens_k=None,
            max_seqlen_q=None, max_seqlen_k=None, stream=None, window_size=(-1, -1), alibi_slopes=None):
    """Allocate (out, lse) and run :func:`fa_fwd`."""
    out = torch.empty_like(q)
    lse = torch.empty(lse_shape(q, cu_seqlens_q), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, out, lse, causal, scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, stream,
           window_size, alibi_slopes)
    return out, lse


def workspace_for(q, cu_seqlens_q=None, max_seqlen_q=None, k=None, max_seqlen_k=None, stored_ds: bool = False):
    """Backward workspace for q; with ``stored_ds`` (and k) also the stored-dS area when
    that route is available at this size (fa_bwd then takes it)."""
    if cu_seqlens_q is None:
        B, Sq, Hq, D = q.shape
    else:
        # every sequence is at most max_seqlen_q long, so B * max_seqlen_q >= total_q
        B, Sq, Hq, D = cu_seqlens_q.numel() - 1, int(max_seqlen_q), q.shape[1], q.shape[2]
    n = fa_bwd_workspace_bytes(B, Sq, Hq, D)
    if stored_ds:
        if k is None:
            raise ValueError("the stored-dS area needs k (its key length)")
        Sk = k.shape[1] if cu_seqlens_q is None else int(max_seqlen_k)
        ds = fa_bwd_ds_workspace_bytes(B, Sq, Sk, Hq, D)
        if ds:
            n = (n + 255) // 256 * 256 + ds
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def backward(dout, q, k, v, out, lse, causal: bool = False, scale: float | None = None, cu_seqlens_q=None,
             cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, stream=None, deterministic: bool = False,
             window_size=(-1, -1), alibi_slopes=None, stored_ds: bool = True):
    """Allocate (dq, dk, dv) and the workspace, and run :func:`fa_bwd` (or
    :func:`fa_bwd_deterministic`).  ``stored_ds`` gives the workspace the stored-dS area
    when the call will take that route (D > 64, or deterministic) and it is available at
    this size: the fastest route there, and deterministic; without it the backward takes
    the atomic route (or, deterministic or D > 128, the recompute route)."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    use_ds = stored_ds and (deterministic or q.shape[-1] > 64)
    ws = workspace_for(q, cu_seqlens_q, max_seqlen_q, k, max_seqlen_k, use_ds)
    run = fa_bwd_deterministic if deterministic else fa_bwd
    run(dout, q, k, v, out, lse, dq, dk, dv, ws, causal, scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
        max_seqlen_k, stream, window_size, alibi_slopes)
    return dq, dk, dv


# ---------------------------------------------------------------------------- KV-cache decode

def _int32_vec(t, n, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor of {n} entries")
    return t


def _kvcache_geometry(q, k_cache, block_table):
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q is (batch, seqlen_q, heads, headdim); the caches are 4-D")
    B, Sq, Hq, D = q.shape
    cache_batch, cache_seqlen, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[3] != D:
        raise ValueError("q and the caches differ in head dimension")
    max_blocks = 0
    if block_table is not None:
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table is (batch, max_blocks_per_seq)")
        if block_table.dtype != torch.int32 or not block_table.is_contiguous() or not block_table.is_cuda:
            raise ValueError("block_table must be a contiguous int32 GPU tensor")
        max_blocks = block_table.shape[1]
    return B, Sq, Hq, Hkv, D, cache_batch, cache_seqlen, max_blocks


def fa_fwd_kvcache_num_splits(B: int, Sq: int, Hq: int, Hkv: int, D: int, seqlen_k: int,
                              page_block_size: int = 0) -> int:
    return int(lib().fa_fwd_kvcache_num_splits(B, Sq, Hq, Hkv, D, seqlen_k, page_block_size))


def fa_fwd_kvcache_workspace_bytes(B: int, Sq: int, Hq: int, D: int, num_splits: int) -> int:
    return int(lib().fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, num_splits))


def kvcache_splits(q, k_cache, block_table=None, num_splits: int = 0) -> int:
    """Split count fa_fwd_kvcache uses for these tensors (``num_splits`` 0 = heuristic)."""
    B, Sq, Hq, Hkv, D, _, cache_seqlen, max_blocks = _kvcache_geometry(q, k_cache, block_table)
    if num_splits:
        return int(num_splits)
    cap = max_blocks * cache_seqlen if block_table is not None else cache_seqlen
    return fa_fwd_kvcache_num_splits(B, Sq, Hq, Hkv, D, cap, cache_seqlen if block_table is not None else 0)


def fa_fwd_kvcache(q, k_cache, v_cache, out, lse, cache_seqlens=None, cache_batch_idx=None, block_table=None,
                   causal: bool = False, scale: float | None = None, window_size=(-1, -1), alibi_slopes=None,
                   num_splits: int = 0, workspace=None, stream=None) -> None:
    """Enqueue attention of q (B, Sq, Hq, D) against a read-only KV cache; writes out and
    lse (B, Hq, Sq).  Caches are (cache_batch, cache_seqlen, Hkv, D), or pages
    (num_blocks, page_block_size, Hkv, D) addressed through ``block_table``
    (B, max_blocks_per_seq).  ``cache_seqlens`` / ``cache_batch_idx``: int32 (B,) GPU
    tensors or None.  ``alibi_slopes``: fp32 (Hq,) or (B, Hq).  With more than one split
    ``workspace`` (uint8 GPU tensor) must hold fa_fwd_kvcache_workspace_bytes(...)."""
    B, Sq, Hq, Hkv, D, cache_batch, cache_seqlen, max_blocks = _kvcache_geometry(q, k_cache, block_table)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache differ in shape")
    _expect(out, q.shape, "out")
    _expect(lse, (B, Hq, Sq), "lse")
    dt = _dtype(q, k_cache, v_cache, out)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 GPU tensor")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("out", out), ("lse", lse)):
        if t.device != q.device:
            raise ValueError(f"{name} lives on {t.device}, q on {q.device}")
    _int32_vec(cache_seqlens, B, "cache_seqlens")
    _int32_vec(cache_batch_idx, B, "cache_batch_idx")
    stride = _alibi_stride(alibi_slopes, B, Hq)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wl, wr = (int(window_size[0]), int(window_size[1]))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must live in GPU memory")
    check(lib().fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, Sq, Hq, Hkv, D,
                               cache_batch, cache_seqlen, _ptr(cache_seqlens), _ptr(cache_batch_idx),
                               _ptr(block_table), max_blocks, float(scale), int(bool(causal)), wl, wr,
                               _ptr(alibi_slopes), stride, int(num_splits), dt, _ptr(workspace), ws_bytes,
                               _stream(stream)))


def fa_fwd_kvcache_noalloc(q, k_cache, v_cache, out, lse, cache_seqlens=None, cache_batch_idx=None,
                           block_table=None, causal: bool = False, scale: float | None = None, window_size=(-1, -1),
                           alibi_slopes=None, num_splits: int = 0, stream=None) -> None:
    """:func:`fa_fwd_kvcache` without a workspace (the C ``fa_fwd_kvcache_noalloc``): the
    split partials go to the library's static per-device scratch array, so neither the
    library nor this call allocates; calls that overlap on one GPU must not be issued."""
    B, Sq, Hq, Hkv, D, cache_batch, cache_seqlen, max_blocks = _kvcache_geometry(q, k_cache, block_table)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache differ in shape")
    _expect(out, q.shape, "out")
    _expect(lse, (B, Hq, Sq), "lse")
    dt = _dtype(q, k_cache, v_cache, out)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 GPU tensor")
    _int32_vec(cache_seqlens, B, "cache_seqlens")
    _int32_vec(cache_batch_idx, B, "cache_batch_idx")
    _same_device(q, k_cache, v_cache, out, lse, cache_seqlens, cache_batch_idx, block_table, alibi_slopes)
    stride = _alibi_stride(alibi_slopes, B, Hq)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    check(lib().fa_fwd_kvcache_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, Sq, Hq, Hkv,
                                       D, cache_batch, cache_seqlen, _ptr(cache_seqlens), _ptr(cache_batch_idx),
                                       _ptr(block_table), max_blocks, float(scale), int(bool(causal)),
                                       int(window_size[0]), int(window_size[1]), _ptr(alibi_slopes), stride,
                                       int(num_splits), dt, _stream(stream)))


def forward_kvcache(q, k_cache, v_cache, cache_seqlens=None, cache_batch_idx=None, block_table=None,
                    causal: bool = False, scale: float | None = None, window_size=(-1, -1), alibi_slopes=None,
                    num_splits: int = 0, stream=None):
    """Allocate (out, lse) and the workspace and run :func:`fa_fwd_kvcache`.
    ``cache_seqlens`` may also be a Python int (the same length for every sequence)."""
    B, Sq, Hq, _, D, _, _, _ = _kvcache_geometry(q, k_cache, block_table)
    if isinstance(cache_seqlens, int):
        cache_seqlens = torch.full((B,), cache_seqlens, dtype=torch.int32, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    n = fa_fwd_kvcache_workspace_bytes(B, Sq, Hq, D, kvcache_splits(q, k_cache, block_table, num_splits))
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    fa_fwd_kvcache(q, k_cache, v_cache, out, lse, cache_seqlens, cache_batch_idx, block_table, causal, scale,
                   window_size, alibi_slopes, num_splits, ws, stream)
    return out, lse
