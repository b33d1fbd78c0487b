"""Quantizers on a tensor with more 128 x 128 tiles than the grid holds.

Without atomics the quantizers launch one workgroup per tile up to 128 per CU
and walk further tiles with a grid stride; this tensor (4096 rows, enough
columns for the grid plus two tile-columns per tile-row) makes the workgroups
of the last tile-row's end run a second tile.  Two 128-row bands are checked
bit-exactly against the oracle: the first tile-row (first tiles of the grid)
and the last one (which holds the second-stride tiles).  Each band's row-wise
copy depends only on its rows, and its 128 rows hold whole column blocks, so
the oracle runs on the band alone.  NVFP4 takes its tensor scale from the
maximum |x| of the whole tensor (an exact reduction, taken with torch).
"""

import numpy as np
import pytest

import oracle
from helpers import to_np

pytestmark = pytest.mark.gpu

ROWS = 4096
BAND = 128


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


@pytest.fixture(scope="module")
def big():
    """A seeded bf16 tensor ROWS x cols with ntiles > 128 x CUs; returns the
    device tensor and the two bands as float32 host arrays."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = 128 * cus
    tiles_c = grid // (ROWS // 128) + 2
    cols = tiles_c * 128
    assert (ROWS // 128) * tiles_c > grid
    g = torch.Generator(device="cuda")
    g.manual_seed(71)
    x = torch.randn((ROWS, cols), device="cuda", generator=g)
    x.mul_(torch.exp(torch.empty((ROWS, 1), device="cuda").uniform_(-6, 6, generator=g)))
    x = x.to(torch.bfloat16)
    bands = {r0: x[r0:r0 + BAND].float().cpu().numpy() for r0 in (0, ROWS - BAND)}
    return x, bands


def _empty(shape, dtype=None):
    import torch

    return torch.empty(shape, dtype=dtype or torch.uint8, device="cuda")


def test_tensorwise_cast_grid_stride(q, big):
    import torch

    x, bands = big
    R, C = x.shape
    qq, qt = _empty((R, C)), _empty((C, R))
    scale = np.float32(24.0)
    q.qsg_cast_transpose(x, q.E4M3, torch.tensor([scale], device="cuda"), qq, qt)
    torch.cuda.synchronize()
    for r0, xb in bands.items():
        ref_q, ref_qt = oracle.cast_transpose(xb, scale, "e4m3")
        assert np.array_equal(to_np(qq[r0:r0 + BAND]), ref_q), r0
        assert np.array_equal(to_np(qt[:, r0:r0 + BAND]), ref_qt), r0
    del qq, qt


def test_mxfp8_grid_stride(q, big):
    import torch

    x, bands = big
    R, C = x.shape
    qq, s, qt, st = _empty((R, C)), _empty((R, C // 32)), _empty((C, R)), _empty((C, R // 32))
    q.qsg_quantize(x, q.MXFP8, q.E4M3, q=qq, s=s, qt=qt, st=st)
    torch.cuda.synchronize()
    for r0, xb in bands.items():
        ref = oracle.mx_quantize(xb, "e4m3", "ceil")
        assert np.array_equal(to_np(qq[r0:r0 + BAND]), ref["q"]), r0
        assert np.array_equal(to_np(s[r0:r0 + BAND]), ref["s"]), r0
        assert np.array_equal(to_np(qt[:, r0:r0 + BAND]), ref["qt"]), r0
        assert np.array_equal(to_np(st[:, r0 // 32:(r0 + BAND) // 32]), ref["st"]), r0
    del qq, s, qt, st


def test_block_1x128_grid_stride(q, big):
    import torch

    x, bands = big
    R, C = x.shape
    qq, qt = _empty((R, C)), _empty((C, R))
    s = _empty((R, C // 128), torch.float32)
    st = _empty((C, R // 128), torch.float32)
    q.qsg_quantize(x, q.BLOCK_1X128, q.E4M3, q=qq, s=s, qt=qt, st=st)
    torch.cuda.synchronize()
    for r0, xb in bands.items():
        ref = oracle.block_quantize_1x128(xb, "e4m3")
        assert np.array_equal(to_np(qq[r0:r0 + BAND]), ref["q"]), r0
        assert np.array_equal(to_np(s[r0:r0 + BAND]).view(np.uint32), ref["s"].view(np.uint32)), r0
        assert np.array_equal(to_np(qt[:, r0:r0 + BAND]), ref["qt"]), r0
        assert np.array_equal(to_np(st[:, r0 // 128:r0 // 128 + 1]).view(np.uint32), ref["st"].view(np.uint32)), r0
    del qq, s, qt, st


def test_nvfp4_grid_stride(q, big):
    import torch

    x, bands = big
    R, C = x.shape
    ts = torch.empty(3, device="cuda")
    qq, s = _empty((R, C // 2)), _empty((R, C // 16))
    qt, st = _empty((C, R // 2)), _empty((C, R // 16))
    q.qsg_quantize_nvfp4(x, ts, qq, s, qt, st)
    torch.cuda.synchronize()
    amax = np.float32(x.abs().max().float().item())
    s_enc, s_dec = oracle.nvfp4.tensor_scale(amax)
    got_ts = to_np(ts)
    assert got_ts[0] == amax
    assert got_ts[1].view(np.uint32) == np.float32(s_enc).view(np.uint32)
    assert got_ts[2].view(np.uint32) == np.float32(s_dec).view(np.uint32)
    for r0, xb in bands.items():
        ref_q, ref_s = oracle.nvfp4.quantize_rows(xb, s_enc)
        assert np.array_equal(to_np(qq[r0:r0 + BAND]), ref_q), r0
        assert np.array_equal(to_np(s[r0:r0 + BAND]), ref_s), r0
        ref_qt, ref_st = oracle.nvfp4.quantize_rows(np.ascontiguousarray(xb.T), s_enc)
        assert np.array_equal(to_np(qt[:, r0 // 2:(r0 + BAND) // 2]), ref_qt), r0
        assert np.array_equal(to_np(st[:, r0 // 16:(r0 + BAND) // 16]), ref_st), r0
    del qq, s, qt, st
