"""GPU parity of the FP8-stored MLP activation input (GeLU) against the oracle.

* forward: the stored FP8 bytes and the fused amax bit-exact; bf16 gelu(h)
  within the elementwise rule |a - ref| <= 2^-8 |ref| + 2^-126;
* backward: bf16 dh within |dh - ref| <= 2^-8 |ref| + 2^-20 |da| + 2^-126,
  the reference recovering h' = fp32(dec(q) * scale_inv) from the same bytes;
* shapes: vector path, columns not a multiple of 8 (element path), a strided
  input, an empty tensor; E4M3 and E5M2;
* h ~ N(0, 1.28) (the spread of X W2^T in the 4096-hidden Linear's workload),
  da ~ N(0, 1e-3), the per-tensor scale from the tensor's amax;
* at 8192 x 14336 (a quarter of that Linear's FC1 output) the bytes in full
  and a seeded sample of 2^20 outputs.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_bits_to_f32, to_dev, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu
FMTS = {0: "e4m3", 1: "e5m2"}


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def fscal(v):
    import torch

    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run_case(q, fmt, hb, dab, h_dev=None, sample=None):
    """hb, dab: bf16 bit patterns (numpy); h_dev overrides the device input (a strided view)."""
    import torch

    R, C = hb.shape
    hf = bf16_bits_to_f32(hb)
    s, si = oracle.tensorwise_scale(oracle.amax(hf), FMTS[fmt])
    hd = to_dev_bf16(hb) if h_dev is None else h_dev
    a = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    qq = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    amax = torch.zeros(1, device="cuda")
    q.qsg_act_fp8_store_fwd(hd, fmt, fscal(s), a, qq, amax)
    dh = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    q.qsg_act_fp8_store_bwd(to_dev_bf16(dab), fmt, qq, fscal(si), dh)
    torch.cuda.synchronize()
    aref, qref = oracle.act_fp8_store_fwd(hf, s, FMTS[fmt])
    assert np.array_equal(to_np(qq), qref)
    assert np.float32(amax.item()).view(np.uint32) == np.float32(oracle.amax(hf)).view(np.uint32)
    daf = bf16_bits_to_f32(dab)
    got_a, got_dh = to_np(a), to_np(dh)
    if sample is not None:
        idx = sample
        aref = aref.reshape(-1)[idx]
        got_a = got_a.reshape(-1)[idx]
        got_dh = got_dh.reshape(-1)[idx]
        dref = oracle.act_fp8_store_bwd(daf.reshape(-1)[idx], qref.reshape(-1)[idx], FMTS[fmt], si)
        gain = daf.reshape(-1)[idx]
    else:
        dref = oracle.act_fp8_store_bwd(daf, qref, FMTS[fmt], si)
        gain = daf
    ok, info = oracle.elementwise_check(got_a, aref)
    assert ok, ("forward", info)
    ok, info = oracle.elementwise_check(got_dh, dref, gain=gain)
    assert ok, ("backward", info)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("R,C", [(256, 1024), (130, 77), (1, 8), (33, 4097)])
def test_act_small(q, fmt, R, C):
    hb = workloads.normal([90, fmt, R, C, 0], (R, C), 1.28)
    dab = workloads.normal([90, fmt, R, C, 1], (R, C), 1e-3)
    run_case(q, fmt, hb, dab)


def test_act_extreme_inputs(q):
    """Large negative inputs (gelu tiny, kept relative through erfc), values
    around the derivative's root, zeros and signed zeros, the E4M3 range."""
    vals = np.concatenate([np.linspace(-12, 12, 4001), [-0.7517915, -0.75, 0.0, -0.0, 400.0, -400.0]])
    vals = np.resize(vals.astype(np.float32), 4096).reshape(8, 512)
    hb = (vals.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 patterns
    dab = workloads.normal([91, 1], (8, 512), 1.0)
    run_case(q, 0, hb, dab)


def test_act_strided_input(q):
    big = workloads.normal([92, 0], (96, 300), 1.28)
    hb = np.ascontiguousarray(big[:, 10:10 + 256])
    dab = workloads.normal([92, 1], (96, 256), 1e-3)
    hdev = to_dev_bf16(big)[:, 10:10 + 256]
    run_case(q, 0, hb, dab, h_dev=hdev)


def test_act_empty(q):
    import torch

    h = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    qq = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    amax = torch.full((1,), 7.0, device="cuda")
    q.qsg_act_fp8_store_fwd(h, 0, fscal(1.0), a, qq, amax)
    assert amax.item() == 0.0


def test_act_fc1_quarter_sampled(q):
    R, C = 8192, 14336
    hb = workloads.normal([93, 0], (R, C), 1.28)
    dab = workloads.normal([93, 1], (R, C), 1e-3)
    g = workloads.generator(93)
    idx = g.integers(0, R * C, 1 << 20)
    run_case(q, 0, hb, dab, sample=idx)
