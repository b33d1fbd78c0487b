"""Parity at the full sizes of the benchmarked 4096-hidden Linear step
(X 32768x4096, W 4096x4096, W2 14336x4096, dY 32768x4096, dY2 32768x14336,
tensorwise hybrid), in the launch configuration bench.py times.

Quantized bytes and scales are compared in full (bit-exact).  GEMM outputs
are compared on a seeded sample of 256 output rows x 256 output columns,
each element computed by the oracle as an fp64 dot product of the
dequantized row and column.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_bits_to_f32, to_dev_bf16

pytestmark = pytest.mark.gpu

M, H, F = 32768, 4096, 14336


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


@pytest.fixture(scope="module")
def linear(q):
    """Inputs and library-quantized copies of the full Linear."""
    import torch

    host = workloads.linear_4096(M, H, F)
    out = {}
    for name, fmt, code in (("X", "e4m3", q.E4M3), ("W", "e4m3", q.E4M3), ("W2", "e4m3", q.E4M3),
                            ("dY", "e5m2", q.E5M2), ("dY2", "e5m2", q.E5M2)):
        bits = host[name]
        R, C = bits.shape
        xd = to_dev_bf16(bits)
        qq = torch.empty((R, C), dtype=torch.uint8, device="cuda")
        qt = torch.empty((C, R), dtype=torch.uint8, device="cuda")
        s = torch.zeros(3, device="cuda")
        q.qsg_quantize(xd, q.TENSORWISE, code, q=qq, s=s, qt=qt)
        out[name] = dict(bits=bits, fmt=fmt, code=code, q=qq, qt=qt, s=s)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["X", "W", "W2", "dY", "dY2"])
def test_fullsize_tensorwise_quantize_bit_exact(linear, name):
    t = linear[name]
    xf = bf16_bits_to_f32(t["bits"])
    a = oracle.amax(xf)
    s, si = oracle.tensorwise_scale(a, t["fmt"])
    got = t["s"].cpu().numpy()
    assert got.view(np.uint32).tolist() == np.float32([a, s, si]).view(np.uint32).tolist()
    rq, _ = oracle.cast_transpose(xf, s, t["fmt"])
    gq = t["q"].cpu().numpy()
    assert np.array_equal(gq, rq)
    assert np.array_equal(t["qt"].cpu().numpy(), np.ascontiguousarray(rq.T))


GEMMS = {
    # name: (A key, A copy, B key, B copy, M, N, K)
    "fprop_W": ("X", "q", "W", "q"),
    "fprop_W2": ("X", "q", "W2", "q"),
    "dgrad_W": ("dY", "q", "W", "qt"),
    "dgrad_W2": ("dY2", "q", "W2", "qt"),
    "wgrad_W": ("dY", "qt", "X", "qt"),
    "wgrad_W2": ("dY2", "qt", "X", "qt"),
}


@pytest.mark.parametrize("gname", list(GEMMS))
def test_fullsize_gemm_sampled(q, linear, gname):
    import torch

    ak, ac, bk, bc = GEMMS[gname]
    A, B = linear[ak], linear[bk]
    qa, qb = A[ac], B[bc]
    Mo, K = qa.shape
    No = qb.shape[0]
    c = torch.empty((Mo, No), dtype=torch.bfloat16, device="cuda")
    q.qsg_scaled_gemm(qa, A["code"], q.TENSORWISE, A["s"][2:3], qb, B["code"], q.TENSORWISE, B["s"][2:3], c)
    torch.cuda.synchronize()
    g = workloads.generator(50, len(gname))
    rows = np.sort(g.choice(Mo, 256, replace=False))
    cols = np.sort(g.choice(No, 256, replace=False))
    ra = qa[torch.from_numpy(rows).cuda()].cpu().numpy()
    rb = qb[torch.from_numpy(cols).cuda()].cpu().numpy()
    sai = A["s"][2].item()
    sbi = B["s"][2].item()
    ref = oracle.gemm_per_tensor(ra, A["fmt"], np.float32(sai), rb, B["fmt"], np.float32(sbi))
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    ok, info = oracle.tolerance_check(got, ref)
    assert ok, info
    # the full output must hold no NaN / inf
    assert torch.isfinite(c).all().item()
