"""Parity of the fp32 master weight -> FP8 cast.

The distributed optimizer keeps fp32 master weights and, with
--fp8-param-gather, casts them straight to FP8 instead of keeping a bf16 copy
("How to reduce cuda memory usage of fp8?", the answer naming
cast_master_weights_to_fp8; "Low-Precision Training Guide", knob
--fp8-param-gather).  The single-GPU part of that is one quantizer call on
fp32 input that writes both FP8 copies and their scales.

W2 [14336 x 4096] fp32 ~N(0, 0.02) (the larger weight of the 4096-hidden
Linear), every recipe, both copies -- every byte and scale bit-exact against
the oracle:
* tensorwise: amax, scale, scale_inv, Q and Q^T (E4M3);
* delayed: three steps of the master weights after small updates, cast with
  the history's scale while the amax is fused into the cast, then the
  history update (amax, scale and bytes of every step);
* MXFP8: row- and column-wise codes and E8M0 scales;
* blockwise 128x128: Q, Q^T and both scale grids.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import to_dev

pytestmark = pytest.mark.gpu

R, C = 14336, 4096


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


@pytest.fixture(scope="module")
def master():
    return workloads.normal([70, 0], (R, C), 0.02, "f32")


def u8(shape):
    import torch

    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def bits(v):
    return np.float32(v).view(np.uint32)


def test_tensorwise(q, master):
    import torch

    x = to_dev(master)
    qq, qt = u8((R, C)), u8((C, R))
    s = torch.zeros(3, device="cuda")
    q.qsg_quantize(x, q.TENSORWISE, q.E4M3, q=qq, s=s, qt=qt)
    rq, rqt, ra, rs, rsi = oracle.quantize_tensorwise(master, "e4m3")
    got = s.cpu().numpy()
    assert [bits(v) for v in got] == [bits(ra), bits(rs), bits(rsi)]
    assert np.array_equal(qq.cpu().numpy(), rq)
    assert np.array_equal(qt.cpu().numpy(), rqt)


def test_delayed_three_steps(q, master):
    import torch

    L = 16
    state = oracle.DelayedState(L, "e4m3")
    hist = torch.zeros(L, device="cuda")
    scale = torch.ones(1, device="cuda")
    sinv = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    w = master
    for t in range(3):
        if t:  # an optimizer step moves the master weights a little
            w = (w + workloads.normal([70, 1, t], (R, C), 1e-3, "f32")).astype(np.float32)
        x = to_dev(w)
        qq, qt = u8((R, C)), u8((C, R))
        q.qsg_cast_transpose(x, q.E4M3, scale, qq, qt, amax)
        q.qsg_amax_update(hist, t, amax, q.E4M3, 0, scale, sinv)
        rq, rqt, ra, _, _ = state.step(w, t)
        assert bits(amax.item()) == bits(ra), t
        assert bits(scale.item()) == bits(state.scale) and bits(sinv.item()) == bits(state.scale_inv), t
        assert np.array_equal(qq.cpu().numpy(), rq), t
        assert np.array_equal(qt.cpu().numpy(), rqt), t


def test_mxfp8(q, master):
    x = to_dev(master)
    qq, s, qt, st = u8((R, C)), u8((R, C // 32)), u8((C, R)), u8((C, R // 32))
    q.qsg_quantize(x, q.MXFP8, q.E4M3, q=qq, s=s, qt=qt, st=st)
    ref = oracle.mx_quantize(master, "e4m3")
    for name, t in (("q", qq), ("s", s), ("qt", qt), ("st", st)):
        assert np.array_equal(t.cpu().numpy(), ref[name]), name


def test_blockwise_128x128(q, master):
    import torch

    x = to_dev(master)
    qq, qt = u8((R, C)), u8((C, R))
    s = torch.empty((R // 128, C // 128), device="cuda")
    st = torch.empty((C // 128, R // 128), device="cuda")
    q.qsg_quantize(x, q.BLOCK_128X128, q.E4M3, q=qq, s=s, qt=qt, st=st)
    ref = oracle.block_quantize_128x128(master, "e4m3")
    assert np.array_equal(qq.cpu().numpy(), ref["q"])
    assert np.array_equal(qt.cpu().numpy(), ref["qt"])
    assert np.array_equal(s.cpu().numpy().view(np.uint32), np.asarray(ref["s"], np.float32).view(np.uint32))
    assert np.array_equal(st.cpu().numpy().view(np.uint32), np.asarray(ref["st"], np.float32).view(np.uint32))
