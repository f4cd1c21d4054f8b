"""GPU parity for head dimensions that are not a tile width (any multiple of 8 up to 256):
forward, backward (atomic and deterministic dQ), decode, window and ALiBi, against the fp64
oracle through the C ABI.  The kernels run such a head dimension in the next tile width
(64, 128 or 256) with the padding masked; these cases cover one head dimension just above
each smaller tile width, ones inside each, the smallest (8) and one in the last 16-wide
slice of a tile (248), at ragged shapes that span several tiles."""

import pytest

from exact_tiled_attention_02_amd import synth
from tests import test_gpu_backward as tb
from tests import test_gpu_decode as td
from tests import test_gpu_forward as tf

pytestmark = pytest.mark.gpu

DIMS = [8, 32, 40, 72, 96, 112, 160, 192, 200, 248]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 300, 300), (1, 2, 2, 100, 200), (1, 6, 2, 129, 77)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward(D, causal, shape):
    B, Hq, Hkv, Sq, Sk = shape
    dtype = "bf16" if D % 16 else "fp16"
    tf._full_check(tf.W(f"hd_fwd_d{D}_c{int(causal)}", B, Hq, Hkv, Sq, Sk, D, dtype, causal, seed=D * 7 + Sq))


@pytest.mark.parametrize("D", [32, 96, 160, 192])
def test_forward_varlen(D):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    tf._full_check(tf.W(f"hd_fwd_varlen_d{D}", None, 4, 2, None, None, D, "bf16", True, seed=D + 3, lengths=(lq, lk)))


@pytest.mark.parametrize("route", tb.ROUTES)
@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_backward(D, causal, route):
    dtype = "fp16" if D % 16 else "bf16"
    print(tb._full(tb.W(f"hd_bwd_d{D}_c{int(causal)}", 2, 4, 2, 300, 300, D, dtype, causal, seed=D * 11),
                   stored_ds=route == "ds"))


@pytest.mark.parametrize("route", tb.ROUTES)
@pytest.mark.parametrize("D", [32, 96, 160, 192])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_gqa(D, causal, route):
    lq = [1, 129, 0, 300, 64, 17]
    lk = [5, 129, 3, 250, 64, 200]
    print(tb._full(tb.W(f"hd_bwd_varlen_d{D}_c{int(causal)}", None, 6, 2, None, None, D, "bf16", causal, seed=D + 5,
                        lengths=(lq, lk)), stored_ds=route == "ds"))


@pytest.mark.parametrize("D", [32, 96, 160, 192])
def test_backward_deterministic(D):
    print(tb._full(tb.W(f"hd_bwd_det_d{D}", 1, 6, 2, 77, 500, D, "bf16", True, seed=D + 9), deterministic=True))


@pytest.mark.parametrize("D", [96, 200])
def test_window_alibi(D):
    w = tb.W(f"hd_local_d{D}", 2, 4, 2, 300, 280, D, "bf16", True, seed=D + 13, window=(70, 0), alibi="head")
    print(tb._full(w))
    print(tb._full(w, deterministic=True))
    print(tb._full(w, stored_ds=True))


@pytest.mark.parametrize("D", [32, 96, 160, 192])
@pytest.mark.parametrize("splits", [0, 1])
def test_decode(D, splits):
    td._check(td.KW(f"hd_dec_d{D}", 3, 2, 8, 2, D, "bf16", 1000, lengths=[1000, 517, 33], seed=D + 17), splits)


@pytest.mark.parametrize("D", [40, 160])
def test_decode_paged(D):
    td._check(td.KW(f"hd_dec_paged_d{D}", 4, 1, 8, 2, D, "fp16", 1024, lengths=[1024, 1, 700, 256], page=256,
                    seed=D + 19))
