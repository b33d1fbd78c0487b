"""GPU parity of the NVFP4 entry points (qsg_quantize_nvfp4, qsg_gemm_nvfp4)
against the CPU oracle (oracle.nvfp4).

Quantization: packed E2M1 codes, E4M3 block-scale bytes and the three tensor
scale floats must be bit-exact, for row-wise and column-wise copies, bf16 and
fp32 inputs, ragged tiles, strided views and the degenerate cases (empty,
all zero, infinities, blocks whose scale underflows to zero or to an E4M3
subnormal).  GEMM: integer-valued products with exact sums must be bit-exact;
everything else meets |y - ref| <= 1e-2 |ref| + 1e-3 rms(ref) against the
fp64 oracle on the same bytes.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_bits_to_f32, f32_to_bf16_rne_f64, to_dev, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu

nv = oracle.nvfp4


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def mixture(key, shape, lo=-34, hi=4):
    """Student-t (nu = 3) samples, each 16 x 16 patch multiplied by its own
    power of two 2^U[lo, hi) (so some blocks' scales are E4M3 subnormals or
    underflow to zero), with about 2 % of the patches zeroed."""
    g = workloads.generator(70, *key)
    R, C = shape
    x = g.standard_t(3.0, shape).astype(np.float32)
    pr, pc = (R + 15) // 16, (C + 15) // 16
    e = g.integers(lo, hi, (pr, pc)).astype(np.float32)
    e[g.random((pr, pc)) < 0.02] = -np.inf
    f = np.repeat(np.repeat(np.exp2(e), 16, 0), 16, 1)[:R, :C]
    return (x * f).astype(np.float32)


def as_input(x, dtype):
    """(device tensor, the float32 values it holds)."""
    if dtype == "bf16":
        b = workloads.f32_to_bf16_bits(x)
        return to_dev_bf16(b), bf16_bits_to_f32(b)
    return to_dev(x), x


def run_quant(q, xd, row=True, col=True):
    import torch

    rows, cols = xd.shape
    ts = torch.full((3,), float("nan"), device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    qd = torch.full((rows, cols // 2), 0xEE, **u8) if row else None
    sd = torch.full((rows, cols // 16), 0xEE, **u8) if row else None
    qtd = torch.full((cols, rows // 2), 0xEE, **u8) if col else None
    std = torch.full((cols, rows // 16), 0xEE, **u8) if col else None
    q.qsg_quantize_nvfp4(xd, ts, qd, sd, qtd, std)
    torch.cuda.synchronize()
    return {"ts": to_np(ts), "q": to_np(qd) if row else None, "s": to_np(sd) if row else None,
            "qt": to_np(qtd) if col else None, "st": to_np(std) if col else None}


def f32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_quant(got, xf, row=True, col=True):
    ref = nv.quantize(xf, rowwise=row, colwise=col)
    want_ts = np.array([ref["amax"], ref["s_enc"], ref["s_dec"]], dtype=np.float32)
    assert np.array_equal(f32bits(got["ts"]), f32bits(want_ts)), (got["ts"], want_ts)
    for k in (("q", "s") if row else ()) + (("qt", "st") if col else ()):
        bad = np.nonzero(got[k] != ref[k])
        assert bad[0].size == 0, (k, bad[0][:5], bad[1][:5], got[k][bad][:5], ref[k][bad][:5])
    return ref


SHAPES = [(256, 512), (272, 400), (16, 16), (1008, 48), (48, 1008), (128, 128), (400, 2064)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_quantize_bit_exact(q, dtype, rows, cols):
    xd, xf = as_input(mixture([1, rows, cols], (rows, cols)), dtype)
    check_quant(run_quant(q, xd), xf)


@pytest.mark.parametrize("rows,cols,row,col", [(37, 64, True, False), (64, 37, False, True),
                                               (130, 272, True, False), (272, 130, False, True)])
def test_quantize_one_copy_ragged(q, rows, cols, row, col):
    xd, xf = as_input(mixture([2, rows, cols], (rows, cols)), "bf16")
    check_quant(run_quant(q, xd, row, col), xf, row, col)


@pytest.mark.parametrize("dtype,extra", [("bf16", 3), ("bf16", 8), ("f32", 5), ("f32", 4)])
def test_quantize_strided_view(q, dtype, extra):
    rows, cols = 144, 160
    big = mixture([3, extra], (rows, cols + extra))
    xd, xf = as_input(big, dtype)
    check_quant(run_quant(q, xd[:, extra:]), np.ascontiguousarray(xf[:, extra:]))


def test_quantize_special_values(q):
    rows, cols = 64, 64
    x = mixture([4], (rows, cols), lo=-4, hi=2)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, 3] = np.inf
    x[5, 40] = -np.inf
    x[7, :] = np.float32(1e-38)  # scale underflows to zero: the codes keep the sign of zero
    x[8, :] *= -1
    xd, xf = as_input(x, "f32")
    check_quant(run_quant(q, xd), xf)


def test_quantize_all_zero_and_empty(q):
    import torch

    x = np.zeros((32, 48), dtype=np.float32)
    x[3, 5] = -0.0
    xd, xf = as_input(x, "f32")
    check_quant(run_quant(q, xd), xf)
    ts = torch.full((3,), float("nan"), device="cuda")
    e = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    q.qsg_quantize_nvfp4(e, ts)
    assert np.array_equal(to_np(ts), np.array([0.0, 1.0, 1.0], dtype=np.float32))


def test_quantize_rejects_bad_shapes(q):
    import torch

    ts = torch.zeros(3, device="cuda")
    x = torch.zeros((32, 40), dtype=torch.bfloat16, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QsgError):  # cols % 16 != 0 for the row-wise copy
        q.qsg_quantize_nvfp4(x, ts, torch.empty((32, 20), **u8), torch.empty((32, 2), **u8))
    with pytest.raises(q.QsgError):  # neither copy requested
        q.qsg_quantize_nvfp4(x, ts)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def gemm(q, qa, sa, ta, qb, sb, tb, out="f32"):
    import torch

    M, N = qa.shape[0], qb.shape[0]
    c = torch.full((M, N), float("nan"), device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    q.qsg_gemm_nvfp4(qa, sa, ta, qb, sb, tb, c)
    return to_np(c).astype(np.float64)


def r10_ok(y, ref):
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    lim = 1e-2 * np.abs(ref) + 1e-3 * rms
    return bool(np.all(err <= lim)), float(np.max(err / np.maximum(lim, 1e-300))) if ref.size else 0.0


def tscale(s_dec):
    import torch

    return torch.tensor([0.0, 1.0 / s_dec, s_dec], dtype=torch.float32, device="cuda")


GEMM_SHAPES = [(128, 128, 128), (256, 384, 512), (130, 250, 304), (1, 1, 16), (37, 300, 1008),
               (512, 256, 4096), (64, 64, 16), (100, 200, 48), (257, 129, 80),
               # at least 128 tiles of 256 x 256 and K % 512 == 0: the persistent kernel
               (4096, 2048, 512), (3968, 2176, 1024)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_integer_exact(q, M, N, K):
    """Codes of every magnitude, block scales 1 and 1.5 (E4M3 0x38, 0x3C),
    tensor scales 4 and 1/8: each product is a multiple of 1/16 below 82 and
    every partial sum is exact in binary32, so C is exact."""
    g = workloads.generator(71, M, N, K)
    ca = g.integers(0, 16, (M, K)).astype(np.uint8)
    cb = g.integers(0, 16, (N, K)).astype(np.uint8)
    sa = np.where(g.random((M, K // 16)) < 0.5, 0x38, 0x3C).astype(np.uint8)
    sb = np.where(g.random((N, K // 16)) < 0.5, 0x38, 0x3C).astype(np.uint8)
    qa, qb = nv.pack(ca), nv.pack(cb)
    exact = nv.gemm(qa, sa, 4.0, qb, sb, 0.125)
    args = (to_dev(qa), to_dev(sa), tscale(4.0), to_dev(qb), to_dev(sb), tscale(0.125))
    assert np.array_equal(gemm(q, *args, out="f32"), exact)
    assert np.array_equal(gemm(q, *args, out="bf16"), f32_to_bf16_rne_f64(exact))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (130, 250, 304), (77, 129, 1024), (300, 200, 48),
                                   (4000, 2100, 1536)])
def test_gemm_random_codes_wide_scales(q, M, N, K):
    """Any code, any finite non-negative E4M3 block scale (subnormals
    included), tensor scales not powers of two."""
    g = workloads.generator(72, M, N, K)
    qa = nv.pack(g.integers(0, 16, (M, K)).astype(np.uint8))
    qb = nv.pack(g.integers(0, 16, (N, K)).astype(np.uint8))
    sa = g.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    sb = g.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    ta, tb = np.float32(0.37), np.float32(3.1e-3)
    ref = nv.gemm(qa, sa, ta, qb, sb, tb)
    for out in ("f32", "bf16"):
        y = gemm(q, to_dev(qa), to_dev(sa), tscale(float(ta)), to_dev(qb), to_dev(sb), tscale(float(tb)), out)
        ok, worst = r10_ok(y, ref)
        assert ok, (out, worst)


def test_gemm_strided_operands_and_k_zero(q):
    import torch

    g = workloads.generator(73)
    M, N, K = 96, 80, 112  # K % 32 == 16: the last staged piece holds one block
    pad = 7
    qa = nv.pack(g.integers(0, 16, (M, K + 2 * pad)).astype(np.uint8))
    qb = nv.pack(g.integers(0, 16, (N, K + 2 * pad)).astype(np.uint8))
    sa = g.integers(0x30, 0x40, (M, K // 16)).astype(np.uint8)
    sb = g.integers(0x30, 0x40, (N, K // 16)).astype(np.uint8)
    ref = nv.gemm(qa[:, : K // 2], sa, 1.0, qb[:, : K // 2], sb, 1.0)
    y = gemm(q, to_dev(qa)[:, : K // 2], to_dev(sa), tscale(1.0), to_dev(qb)[:, : K // 2], to_dev(sb), tscale(1.0))
    ok, worst = r10_ok(y, ref)
    assert ok, worst
    c = torch.full((5, 7), float("nan"), device="cuda")
    e = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    f = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    q.qsg_gemm_nvfp4(e, e, tscale(1.0), f, f, tscale(1.0), c)
    assert np.array_equal(to_np(c), np.zeros((5, 7), dtype=np.float32))


@pytest.mark.parametrize("T,N,K", [(256, 384, 512), (272, 144, 400)])
def test_linear_layer_chain(q, T, N, K):
    """fprop, dgrad and wgrad of a Linear from the library's own NVFP4 copies
    (bit-exact against the oracle's first), each GEMM against the oracle on
    those bytes: Y = X W^T, dX = dY W, dW = dY^T X."""
    xd, xf = as_input(mixture([5, T, K], (T, K), lo=-3, hi=3), "bf16")
    wd, wf = as_input(mixture([6, N, K], (N, K), lo=-3, hi=3), "bf16")
    dd, df = as_input(mixture([7, T, N], (T, N), lo=-3, hi=3), "bf16")
    gx, gw, gd = run_quant(q, xd), run_quant(q, wd), run_quant(q, dd)
    check_quant(gx, xf), check_quant(gw, wf), check_quant(gd, df)
    dev = lambda r, k: to_dev(r[k])
    cases = {
        "fprop": ((gx, "q", "s"), (gw, "q", "s")),
        "dgrad": ((gd, "q", "s"), (gw, "qt", "st")),
        "wgrad": ((gd, "qt", "st"), (gx, "qt", "st")),
    }
    for name, ((ra, ka, ksa), (rb, kb, ksb)) in cases.items():
        ref = nv.gemm(ra[ka], ra[ksa], ra["ts"][2], rb[kb], rb[ksb], rb["ts"][2])
        ta, tb = to_dev(ra["ts"]), to_dev(rb["ts"])
        y = gemm(q, dev(ra, ka), dev(ra, ksa), ta, dev(rb, kb), dev(rb, ksb), tb, "bf16")
        ok, worst = r10_ok(y, ref)
        assert ok, (name, worst)


def test_nvfp4_4096_full_size_sampled(q):
    """The 16384 x 4096 activations and 14336 x 4096 weights of the NVFP4
    Linear, quantized and multiplied at full size; 256 sampled rows of each
    copy bit-exact against the oracle (row quantization depends only on the
    row and the tensor scale), and the 256 x 256 block of C at the sampled
    rows and columns within the acceptance rule."""
    import torch

    wl = workloads.nvfp4_4096()
    xd, wd = to_dev_bf16(wl["X"]), to_dev_bf16(wl["W"])
    M, K = xd.shape
    N = wd.shape[0]
    out = {}
    for name, d in (("X", xd), ("W", wd)):
        R = d.shape[0]
        ts = torch.empty(3, device="cuda")
        qd = torch.empty((R, K // 2), dtype=torch.uint8, device="cuda")
        sd = torch.empty((R, K // 16), dtype=torch.uint8, device="cuda")
        q.qsg_quantize_nvfp4(d, ts, qd, sd)
        out[name] = (qd, sd, ts)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q.qsg_gemm_nvfp4(out["X"][0], out["X"][1], out["X"][2], out["W"][0], out["W"][1], out["W"][2], c)
    torch.cuda.synchronize()
    g = workloads.generator(74)
    rows = np.sort(g.choice(M, 256, replace=False))
    cols = np.sort(g.choice(N, 256, replace=False))
    got = {}
    for name, idx in (("X", rows), ("W", cols)):
        xf = bf16_bits_to_f32(wl[name])
        amax = np.float32(np.max(np.abs(xf)))
        s_enc, s_dec = nv.tensor_scale(amax)
        ts = to_np(out[name][2])
        assert np.array_equal(f32bits(ts), f32bits(np.array([amax, s_enc, s_dec], dtype=np.float32)))
        rq, rs = nv.quantize_rows(xf[idx], s_enc)
        gq, gs = to_np(out[name][0][torch.from_numpy(idx).cuda()]), to_np(out[name][1][torch.from_numpy(idx).cuda()])
        assert np.array_equal(gq, rq) and np.array_equal(gs, rs), name
        got[name] = (rq, rs, s_dec)
    ref = nv.gemm(got["X"][0], got["X"][1], got["X"][2], got["W"][0], got["W"][1], got["W"][2])
    y = to_np(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]).astype(np.float64)
    ok, worst = r10_ok(y, ref)
    assert ok, worst
