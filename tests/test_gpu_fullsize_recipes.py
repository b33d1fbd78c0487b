"""Parity at full size for the delayed, MXFP8 and blockwise workloads.

* delayed_4096: 64 steps of X_t [8192 x 4096] (E4M3, 41 outlier columns x50)
  with amax_history_len 1024, compute_algo max, margin 0 — the amax, scale and
  scale_inv of every step bit-exact, the FP8 bytes of steps 0, 1 and 63
  bit-exact in full; dY_t [8192 x 4096] (E5M2) for 8 steps likewise; the
  three GEMMs of step 1 (fprop, dgrad, wgrad, 8192 x 4096 x 4096 and
  4096 x 4096 x 8192) against the oracle on every output element.
* mxfp8_4096: X [16384 x 4096], W [14336 x 4096] and dY [16384 x 14336],
  row- and column-wise MXFP8 (bytes and E8M0 scales bit-exact in full); the
  MX fprop, dgrad (A = Q(dY), B = Q(W)^T) and wgrad (A = Q(dY)^T,
  B = Q(X)^T) GEMMs, fed the library's own row- and column-wise copies, on a
  seeded sample of 256 output rows x 256 output columns.
* blockwise_7168: X [16384 x 7168] and dY [16384 x 18432] 1x128 (row +
  column copies), W [18432 x 7168] 128x128, bit-exact in full; the blockwise
  fprop (1x128 x 128x128), dgrad (1x128 dY against the transposed 128x128
  grid of W) and wgrad (1x128 x 1x128 along the tokens) GEMMs on a seeded
  256 x 256 sample of outputs.

GEMM samples are compared with the R10 acceptance rule of oracle.gemm.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_bits_to_f32, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def bits32(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def sample_idx(seed, n, k=256):
    return np.sort(workloads.generator(60, seed).choice(n, k, replace=False))


@pytest.mark.parametrize("tensor,fmt,steps,check", [("X", "e4m3", 64, (0, 1, 63)), ("dY", "e5m2", 8, (7,))])
def test_delayed_4096_trajectory(q, tensor, fmt, steps, check):
    import torch

    L = 1024
    code = q.FMT[fmt]
    R, C = 8192, 4096
    hist = torch.zeros(L, device="cuda")
    scale = torch.ones(1, device="cuda")
    scale_inv = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    qq = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    qt = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    st = oracle.DelayedState(L, fmt, margin=0)
    for t in range(steps):
        xb = workloads.delayed_4096_step(t, R, C, C)[tensor]
        q.qsg_cast_transpose(to_dev_bf16(xb), code, scale, qq, qt, amax)
        q.qsg_amax_update(hist, t, amax, code, 0, scale, scale_inv)
        xf = bf16_bits_to_f32(xb)
        used = st.scale
        a = oracle.amax(xf)
        if t in check:
            rq, _ = oracle.cast_transpose(xf, used, fmt)
            assert np.array_equal(qq.cpu().numpy(), rq), t
            assert np.array_equal(qt.cpu().numpy(), np.ascontiguousarray(rq.T)), t
        st.scale, st.scale_inv = oracle.amax_update(st.history, t, a, fmt, 0, st.scale, st.scale_inv)
        assert bits32(amax.cpu().numpy())[0] == bits32(a)[()], t
        assert bits32(scale.cpu().numpy())[0] == bits32(st.scale)[()], t
        assert bits32(scale_inv.cpu().numpy())[0] == bits32(st.scale_inv)[()], t
    assert np.array_equal(bits32(hist.cpu().numpy()), bits32(st.history))


def test_delayed_4096_gemms_full_output(q):
    """The three GEMMs of a delayed-scaling step (step 1: every tensor's scale
    comes from the amax history of step 0), E4M3 X and W, E5M2 dY, bf16 out,
    checked on every output element against the oracle on the same FP8 bytes
    and the scale_inv each tensor was quantized with."""
    import torch

    L, R, C = 1024, 8192, 4096
    wbits = workloads.delayed_4096_weight()
    st = {}
    for name, code in (("X", q.E4M3), ("W", q.E4M3), ("dY", q.E5M2)):
        rows, cols = (C, C) if name == "W" else (R, C)
        st[name] = dict(code=code, hist=torch.zeros(L, device="cuda"), scale=torch.ones(1, device="cuda"),
                        sinv=torch.ones(1, device="cuda"), amax=torch.zeros(1, device="cuda"),
                        q=torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                        qt=torch.empty((cols, rows), dtype=torch.uint8, device="cuda"))
    for t in (0, 1):
        step = workloads.delayed_4096_step(t, R, C, C)
        for name, bits in (("X", step["X"]), ("W", wbits), ("dY", step["dY"])):
            b = st[name]
            b["used"] = b["sinv"].clone()  # scale_inv of the bytes written at this step
            q.qsg_cast_transpose(to_dev_bf16(bits), b["code"], b["scale"], b["q"], b["qt"], b["amax"])
            q.qsg_amax_update(b["hist"], t, b["amax"], b["code"], 0, b["scale"], b["sinv"])
    torch.cuda.synchronize()
    x, w, dy = st["X"], st["W"], st["dY"]
    assert x["used"].item() != 1.0 and dy["used"].item() != 1.0  # step 1 runs on history scales
    cases = {
        "fprop": (x["q"], "e4m3", x["used"], w["q"], "e4m3", w["used"]),
        "dgrad": (dy["q"], "e5m2", dy["used"], w["qt"], "e4m3", w["used"]),
        "wgrad": (dy["qt"], "e5m2", dy["used"], x["qt"], "e4m3", x["used"]),
    }
    for label, (qa, fa, sa, qb, fb, sb) in cases.items():
        c = torch.empty((qa.shape[0], qb.shape[0]), dtype=torch.bfloat16, device="cuda")
        q.qsg_scaled_gemm(qa, q.FMT[fa], q.DELAYED, sa, qb, q.FMT[fb], q.DELAYED, sb, c)
        got = c.float().cpu().numpy()
        ref = oracle.gemm_per_tensor(qa.cpu().numpy(), fa, np.float32(sa.item()), qb.cpu().numpy(), fb,
                                     np.float32(sb.item()))
        ok, info = oracle.tolerance_check(got, ref)
        assert ok, (label, info)
        del c, got, ref


@pytest.fixture(scope="module")
def mx_inputs():
    return workloads.mxfp8_4096(with_dy=True)


def run_mx(q, bits):
    import torch

    R, C = bits.shape
    out = dict(q=torch.empty((R, C), dtype=torch.uint8, device="cuda"),
               s=torch.empty((R, C // 32), dtype=torch.uint8, device="cuda"),
               qt=torch.empty((C, R), dtype=torch.uint8, device="cuda"),
               st=torch.empty((C, R // 32), dtype=torch.uint8, device="cuda"))
    q.qsg_quantize(to_dev_bf16(bits), q.MXFP8, q.E4M3, **out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["X", "W", "dY"])
def test_mxfp8_4096_quantize_bit_exact(q, mx_inputs, name):
    bits = mx_inputs[name]
    got = run_mx(q, bits)
    ref = oracle.mx_quantize(bf16_bits_to_f32(bits), "e4m3", "ceil")
    for k in ("s", "q", "st", "qt"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


def test_mxfp8_4096_fprop_sampled(q, mx_inputs):
    import torch

    gx = run_mx(q, mx_inputs["X"])
    gw = run_mx(q, mx_inputs["W"])
    M, K = mx_inputs["X"].shape
    N = mx_inputs["W"].shape[0]
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qsg_scaled_gemm(gx["q"], q.E4M3, q.MXFP8, gx["s"], gw["q"], q.E4M3, q.MXFP8, gw["s"], c)
    torch.cuda.synchronize()
    rows, cols = sample_idx(1, M), sample_idx(2, N)
    rr, cc = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref = oracle.gemm_mx(gx["q"][rr].cpu().numpy(), "e4m3", gx["s"][rr].cpu().numpy(),
                         gw["q"][cc].cpu().numpy(), "e4m3", gw["s"][cc].cpu().numpy())
    got = c[rr][:, cc].float().cpu().numpy()
    ok, info = oracle.tolerance_check(got, ref)
    assert ok, info
    assert torch.isfinite(c).all().item()


@pytest.mark.parametrize("which", ["dgrad", "wgrad"])
def test_mxfp8_4096_backward_sampled(q, mx_inputs, which):
    """MX dgrad dX = dY W (A = Q(dY) with its row-wise E8M0 scales, B = the
    column-wise copy Q(W)^T with its scales: K = 14336) and wgrad dW = dY^T X
    (A = Q(dY)^T, B = Q(X)^T, both column-wise copies: K = 16384 tokens), each
    fed what qsg_quantize wrote, on a 256 x 256 sample of outputs."""
    import torch

    if which == "dgrad":
        ga = run_mx(q, mx_inputs["dY"])
        gb = run_mx(q, mx_inputs["W"])
        qa, sa, qb, sb = ga["q"], ga["s"], gb["qt"], gb["st"]
    else:
        ga = run_mx(q, mx_inputs["dY"])
        gb = run_mx(q, mx_inputs["X"])
        qa, sa, qb, sb = ga["qt"], ga["st"], gb["qt"], gb["st"]
    M, N = qa.shape[0], qb.shape[0]
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qsg_scaled_gemm(qa, q.E4M3, q.MXFP8, sa, qb, q.E4M3, q.MXFP8, sb, c)
    torch.cuda.synchronize()
    rows, cols = sample_idx(5 if which == "dgrad" else 7, M), sample_idx(6 if which == "dgrad" else 8, N)
    rr, cc = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref = oracle.gemm_mx(qa[rr].cpu().numpy(), "e4m3", sa[rr].cpu().numpy(),
                         qb[cc].cpu().numpy(), "e4m3", sb[cc].cpu().numpy())
    got = c[rr][:, cc].float().cpu().numpy()
    ok, info = oracle.tolerance_check(got, ref)
    assert ok, info
    assert torch.isfinite(c).all().item()


@pytest.fixture(scope="module")
def block_inputs():
    return workloads.blockwise_7168(with_dy=True)


def run_block_act(q, bits):
    import torch

    R, C = bits.shape
    out = dict(q=torch.empty((R, C), dtype=torch.uint8, device="cuda"),
               s=torch.empty((R, C // 128), device="cuda"),
               qt=torch.empty((C, R), dtype=torch.uint8, device="cuda"),
               st=torch.empty((C, R // 128), device="cuda"))
    q.qsg_quantize(to_dev_bf16(bits), q.BLOCK_1X128, q.E4M3, **out)
    torch.cuda.synchronize()
    return out


def run_block_w(q, bits):
    import torch

    R, C = bits.shape
    out = dict(q=torch.empty((R, C), dtype=torch.uint8, device="cuda"),
               s=torch.empty((R // 128, C // 128), device="cuda"),
               qt=torch.empty((C, R), dtype=torch.uint8, device="cuda"),
               st=torch.empty((C // 128, R // 128), device="cuda"))
    q.qsg_quantize(to_dev_bf16(bits), q.BLOCK_128X128, q.E4M3, **out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["X", "dY"])
def test_blockwise_7168_activation_bit_exact(q, block_inputs, name):
    bits = block_inputs[name]
    got = run_block_act(q, bits)
    ref = oracle.block_quantize_1x128(bf16_bits_to_f32(bits), "e4m3")
    for k in ("s", "st"):
        assert np.array_equal(bits32(got[k].cpu().numpy()), bits32(ref[k])), k
    for k in ("q", "qt"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


def test_blockwise_7168_weight_bit_exact(q, block_inputs):
    bits = block_inputs["W"]
    got = run_block_w(q, bits)
    ref = oracle.block_quantize_128x128(bf16_bits_to_f32(bits), "e4m3")
    for k in ("s", "st"):
        assert np.array_equal(bits32(got[k].cpu().numpy()), bits32(ref[k])), k
    for k in ("q", "qt"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


def test_blockwise_7168_fprop_sampled(q, block_inputs):
    import torch

    gx = run_block_act(q, block_inputs["X"])
    gw = run_block_w(q, block_inputs["W"])
    M, K = block_inputs["X"].shape
    N = block_inputs["W"].shape[0]
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qsg_scaled_gemm(gx["q"], q.E4M3, q.BLOCK_1X128, gx["s"], gw["q"], q.E4M3, q.BLOCK_128X128, gw["s"], c)
    torch.cuda.synchronize()
    rows, cols = sample_idx(3, M), sample_idx(4, N)
    rr, cc = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    sb = gw["s"].cpu().numpy()[cols // 128]  # the 128x128 scale rows of the sampled columns
    ref = oracle.gemm_block(gx["q"][rr].cpu().numpy(), "e4m3", gx["s"][rr].cpu().numpy(),
                            gw["q"][cc].cpu().numpy(), "e4m3", sb, "1x128")
    got = c[rr][:, cc].float().cpu().numpy()
    ok, info = oracle.tolerance_check(got, ref)
    assert ok, info
    assert torch.isfinite(c).all().item()


@pytest.mark.parametrize("which", ["dgrad", "wgrad"])
def test_blockwise_7168_backward_sampled(q, block_inputs, which):
    """Blockwise dgrad dX = dY W: A = Q(dY) with 1x128 scales along the 18432
    output features, B = Q(W)^T with the transposed 128x128 grid (7168 x 18432,
    56 x 144 blocks).  Blockwise wgrad dW = dY^T X: A = Q(dY)^T and B = Q(X)^T,
    the column-wise copies with 1x128 scales along the 16384 tokens.  Both fed
    what qsg_quantize wrote, on a 256 x 256 sample of outputs."""
    import torch

    gy = run_block_act(q, block_inputs["dY"])
    if which == "dgrad":
        gw = run_block_w(q, block_inputs["W"])
        qa, sa, qb, sb, kb, lay = gy["q"], gy["s"], gw["qt"], gw["st"], q.BLOCK_128X128, "128x128"
    else:
        gx = run_block_act(q, block_inputs["X"])
        qa, sa, qb, sb, kb, lay = gy["qt"], gy["st"], gx["qt"], gx["st"], q.BLOCK_1X128, "1x128"
    M, N = qa.shape[0], qb.shape[0]
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qsg_scaled_gemm(qa, q.E4M3, q.BLOCK_1X128, sa, qb, q.E4M3, kb, sb, c)
    torch.cuda.synchronize()
    rows, cols = sample_idx(9 if which == "dgrad" else 11, M), sample_idx(10 if which == "dgrad" else 12, N)
    rr, cc = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    if lay == "128x128":
        sbr = sb.cpu().numpy()[cols // 128]  # the 128x128 scale row of each sampled column
    else:
        sbr = sb[cc].cpu().numpy()
    # sbr now holds one scale row per sampled column of B: a 1x128 grid
    ref = oracle.gemm_block(qa[rr].cpu().numpy(), "e4m3", sa[rr].cpu().numpy(), qb[cc].cpu().numpy(), "e4m3", sbr,
                            "1x128")
    got = c[rr][:, cc].float().cpu().numpy()
    ok, info = oracle.tolerance_check(got, ref)
    assert ok, info
    assert torch.isfinite(c).all().item()
