"""GPU parity of the quantization entry points against the CPU oracle.

FP8 bytes, E8M0 bytes, fp32 scales and amaxes must be bit-exact.  Inputs are
seeded (workloads.py recipe) at sizes that span several 128 x 128 tiles and a
ragged tail, plus the degenerate cases (empty, 1 x 1, strided views, zeros,
infinities, NaN, subnormals).
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_bits_to_f32, to_dev, to_dev_bf16, to_np

pytestmark = pytest.mark.gpu

FMTS = [("e4m3", 0), ("e5m2", 1)]


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def f32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def dev_scalar(v):
    import torch

    return torch.tensor([v], dtype=torch.float32, device="cuda")


def empty_u8(shape):
    import torch

    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def run_cast(q, xd, fmt_code, scale, want_q=True, want_qt=True, want_amax=False):
    import torch

    rows, cols = xd.shape
    qd = empty_u8((rows, cols)) if want_q else None
    qtd = empty_u8((cols, rows)) if want_qt else None
    am = torch.full((1,), 123.0, device="cuda") if want_amax else None
    q.qsg_cast_transpose(xd, fmt_code, dev_scalar(scale), qd, qtd, am)
    torch.cuda.synchronize()
    return (to_np(qd) if want_q else None, to_np(qtd) if want_qt else None,
            to_np(am)[0] if want_amax else None)


# ---------------------------------------------------------------------------
# the encoder, exhaustively
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,code", FMTS)
def test_encode_every_bf16_pattern(q, fmt, code):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    x = bf16_bits_to_f32(bits)
    for scale in (1.0, 3.0, 2.0 ** -20, 2.0 ** 30):
        qq, qt, _ = run_cast(q, to_dev_bf16(bits), code, scale)
        with np.errstate(over="ignore", invalid="ignore"):
            ref = oracle.encode((x * np.float32(scale)).astype(np.float32), fmt)
        nan = np.isnan(x)
        # NaN inputs: a NaN code (the sign of a NaN product is not fixed by IEEE)
        assert np.all((qq[nan] & 0x7F) == 0x7F)
        assert np.array_equal(qq[~nan], ref[~nan]), f"scale {scale}"
        assert np.array_equal(qt, qq.T)


@pytest.mark.parametrize("fmt,code", FMTS)
def test_encode_fp32_sweep(q, fmt, code):
    # a stride-61 sample of all binary32 patterns plus dense binades around
    # the FP8 range, in 2^22-element chunks, scale 1
    chunks = []
    for lo in range(0, 1 << 32, 1 << 28):
        chunks.append(np.arange(lo, lo + (1 << 28), 61, dtype=np.uint64).astype(np.uint32))
    for b in ((-10, -7, -6, 8) if fmt == "e4m3" else (-17, -15, -14, 15)):
        lo = (b + 127) << 23
        chunks.append(np.arange(lo, lo + (1 << 23), dtype=np.uint32))
        chunks.append(np.arange(lo, lo + (1 << 23), dtype=np.uint32) | np.uint32(0x80000000))
    allbits = np.concatenate(chunks)
    n = (allbits.size // 4096) * 4096
    for s in range(0, n, 1 << 22):
        blk = allbits[s:min(n, s + (1 << 22))].reshape(-1, 4096)
        x = blk.view(np.float32)
        qq, _, _ = run_cast(q, to_dev(x), code, 1.0, want_qt=False)
        ref = oracle.encode(x, fmt)
        nan = np.isnan(x)
        assert np.all((qq[nan] & 0x7F) == 0x7F)
        bad = np.nonzero((qq != ref) & ~nan)
        assert bad[0].size == 0, [(hex(int(blk[i, j])), hex(int(qq[i, j])), hex(int(ref[i, j])))
                                  for i, j in zip(*[b[:8] for b in bad])]


def test_encode_subnormal_inputs_with_large_scale(q):
    # fp32 subnormal inputs times a large scale land in the FP8 range: the
    # multiply must keep binary32 subnormals
    x = np.array([[1e-40, -3e-39, 1.4e-45, 5e-39] * 4] * 16, dtype=np.float32)
    for fmt, code in FMTS:
        scale = np.float32(2.0 ** 126)
        qq, _, _ = run_cast(q, to_dev(x), code, float(scale), want_qt=False)
        ref = oracle.encode((x * scale).astype(np.float32), fmt)
        assert np.array_equal(qq, ref)


# ---------------------------------------------------------------------------
# amax and scale
# ---------------------------------------------------------------------------
SHAPES = [(1, 1), (7, 13), (128, 128), (130, 250), (300, 517), (1024, 768), (64, 4104)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_amax(q, shape, dtype):
    import torch

    g = workloads.generator(9, *shape)
    x = (g.standard_normal(shape) * np.exp(g.uniform(-3, 3))).astype(np.float32)
    x.flat[g.integers(0, x.size)] = -np.float32(g.uniform(10, 20))
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(x)
        xd, xf = to_dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        xd, xf = to_dev(x), x
    am = torch.full((1,), -5.0, device="cuda")
    q.qsg_amax(xd, am)
    assert f32bits(to_np(am))[0] == f32bits(oracle.amax(xf))[()]


def test_amax_special_values(q):
    import torch

    base = np.zeros((33, 70), np.float32)
    cases = {
        "zeros": base.copy(),
        "negzero": -base.copy(),
        "inf": base.copy(),
        "nan": base.copy(),
        "subnormal": base.copy(),
    }
    cases["inf"][5, 5] = -np.inf
    cases["nan"][7, 60] = np.nan
    cases["nan"][8, 1] = np.inf
    cases["subnormal"][1, 2] = -1e-42
    for name, x in cases.items():
        for dev in (to_dev(x), to_dev_bf16(workloads.f32_to_bf16_bits(x))):
            am = torch.full((1,), 7.0, device="cuda")
            q.qsg_amax(dev, am)
            got = to_np(am)[0]
            ref = oracle.amax(x if dev.dtype == torch.float32 else
                              bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)))
            if np.isnan(ref):
                assert f32bits(np.float32(got))[()] == 0x7FC00000, name
            else:
                assert got == ref, name


def test_amax_strided_view_and_empty(q):
    import torch

    g = workloads.generator(10)
    big = g.standard_normal((96, 300)).astype(np.float32)
    big[:, 200:] = 1000.0  # outside the view
    xd = to_dev(big)[:, 10:200]
    am = torch.zeros(1, device="cuda")
    q.qsg_amax(xd, am)
    assert to_np(am)[0] == oracle.amax(big[:, 10:200])
    e = torch.empty((0, 16), device="cuda")
    am.fill_(5.0)
    q.qsg_amax(e, am)
    assert to_np(am)[0] == 0.0


@pytest.mark.parametrize("fmt,code", FMTS)
def test_compute_scale(q, fmt, code):
    import torch

    g = workloads.generator(11)
    amaxes = np.exp(g.uniform(-40, 40, 300)).astype(np.float32)
    amaxes = np.concatenate([amaxes, np.float32([0.0, np.inf, np.nan, 1e-45, 3e-39, 448, 57344,
                                                 np.finfo(np.float32).max])])
    a_d = to_dev(amaxes)
    out = torch.zeros((amaxes.size, 2), device="cuda")
    for margin in (0, 1, 5):
        for i in range(amaxes.size):
            q.qsg_compute_scale(a_d[i:i + 1], code, margin, out[i, 0:1], out[i, 1:2])
        got = to_np(out)
        for i, a in enumerate(amaxes):
            s, si = oracle.tensorwise_scale(a, fmt, margin)
            assert f32bits(got[i, 0])[()] == f32bits(s)[()], (a, margin)
            assert f32bits(got[i, 1])[()] == f32bits(si)[()], (a, margin)


# ---------------------------------------------------------------------------
# per-tensor cast + transpose
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", SHAPES + [(0, 5), (5, 0)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt,code", FMTS)
def test_cast_transpose(q, shape, dtype, fmt, code):
    g = workloads.generator(12, *shape)
    x = g.standard_normal(shape).astype(np.float32)
    if x.size:
        x.flat[g.integers(0, x.size, 5)] = [np.inf, -np.inf, 0.0, -0.0, 1e-30]
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(x)
        xd, xf = to_dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        xd, xf = to_dev(x), x
    scale = np.float32(g.uniform(1, 100))
    qq, qt, am = run_cast(q, xd, code, float(scale), want_amax=True)
    rq, rqt = oracle.cast_transpose(xf, scale, fmt)
    assert np.array_equal(qq, rq)
    assert np.array_equal(qt, rqt)
    assert f32bits(np.float32(am))[()] == f32bits(oracle.amax(xf))[()]


def test_cast_transpose_single_outputs_and_strided(q):
    import torch

    g = workloads.generator(13)
    big = workloads.normal([13, 1], (384, 1000))
    xd = to_dev_bf16(big)[:, 8:520]
    xf = bf16_bits_to_f32(big)[:, 8:520]
    rq, rqt = oracle.cast_transpose(xf, np.float32(50.0), "e4m3")
    qq, _, _ = run_cast(q, xd, 0, 50.0, want_qt=False)
    assert np.array_equal(qq, rq)
    _, qt, _ = run_cast(q, xd, 0, 50.0, want_q=False)
    assert np.array_equal(qt, rqt)
    # misaligned start (odd element offset) takes the element-wise path
    xd2 = to_dev_bf16(big)[:, 3:400]
    xf2 = bf16_bits_to_f32(big)[:, 3:400]
    qq, qt, _ = run_cast(q, xd2, 1, 7.0)
    r2, r2t = oracle.cast_transpose(xf2, np.float32(7.0), "e5m2")
    assert np.array_equal(qq, r2) and np.array_equal(qt, r2t)
    del g, torch


@pytest.mark.parametrize("fmt,code", FMTS)
def test_quantize_tensorwise(q, fmt, code):
    import torch

    for shape in [(256, 256), (200, 333)]:
        x = workloads.normal([14, shape[0]], shape, 0.5)
        xf = bf16_bits_to_f32(x)
        for margin in (0, 2):
            qq, qt = empty_u8(shape), empty_u8(shape[::-1])
            s = torch.zeros(3, device="cuda")
            q.qsg_quantize(to_dev_bf16(x), q.TENSORWISE, code, q=qq, s=s, qt=qt, margin=margin)
            rq, rqt, ra, rs, rsi = oracle.quantize_tensorwise(xf, fmt, margin)
            assert np.array_equal(to_np(qq), rq) and np.array_equal(to_np(qt), rqt)
            assert np.array_equal(f32bits(to_np(s)), f32bits(np.float32([ra, rs, rsi])))


def test_tensorwise_256_workload(q):
    """The 256 x 256 fp32 tensorwise workload: amax, scale, cast of X and W."""
    import torch

    d = workloads.tensorwise_256()
    for name in ("X", "W"):
        x = d[name]
        qq, qt, s = empty_u8((256, 256)), empty_u8((256, 256)), torch.zeros(3, device="cuda")
        q.qsg_quantize(to_dev(x), q.TENSORWISE, q.E4M3, q=qq, s=s, qt=qt)
        rq, rqt, ra, rs, rsi = oracle.quantize_tensorwise(x, "e4m3")
        assert np.array_equal(to_np(qq), rq) and np.array_equal(to_np(qt), rqt)
        assert np.array_equal(f32bits(to_np(s)), f32bits(np.float32([ra, rs, rsi])))


# ---------------------------------------------------------------------------
# delayed scaling
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("L,steps", [(4, 17), (16, 40), (1024, 24)])
def test_delayed_trajectory(q, L, steps):
    import torch

    rows, cols = 256, 384
    hist = torch.zeros(L, device="cuda")
    scale = torch.ones(1, device="cuda")
    scale_inv = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    st = oracle.DelayedState(L, "e4m3", margin=1)
    for t in range(steps):
        xb = workloads.delayed_4096_step(t, rows, cols, out_cols=8)["X"]
        if t % 7 == 3:
            xb = np.zeros_like(xb)  # an all-zero step keeps the scale
        xf = bf16_bits_to_f32(xb)
        qq, qt = empty_u8((rows, cols)), empty_u8((cols, rows))
        q.qsg_cast_transpose(to_dev_bf16(xb), q.E4M3, scale, qq, qt, amax)
        q.qsg_amax_update(hist, t, amax, q.E4M3, 1, scale, scale_inv)
        rq, rqt, ra, used, _ = st.step(xf, t)
        assert np.array_equal(to_np(qq), rq), t
        assert np.array_equal(to_np(qt), rqt), t
        assert f32bits(to_np(amax))[0] == f32bits(ra)[()], t
        assert f32bits(to_np(scale))[0] == f32bits(st.scale)[()], t
        assert f32bits(to_np(scale_inv))[0] == f32bits(st.scale_inv)[()], t
    assert np.array_equal(f32bits(to_np(hist)), f32bits(st.history))


@pytest.mark.parametrize("L,steps,shape,fmt,dtype", [(4, 17, (256, 384), "e4m3", "bf16"),
                                                     (16, 9, (200, 300), "e5m2", "bf16"),
                                                     (1024, 6, (1024, 768), "e4m3", "f32")])
def test_cast_transpose_delayed_one_launch(q, L, steps, shape, fmt, dtype):
    """qsg_cast_transpose_delayed (cast + transpose, amax, history update in
    one launch) follows the oracle's delayed trajectory bit for bit: bytes,
    amax, scales and history, with an all-zero step and a step holding a NaN
    (ragged 200 x 300 takes the element-wise edge tiles); the workspace is
    zero again after every call."""
    import torch

    rows, cols = shape
    code = q.FMT[fmt]
    hist = torch.zeros(L, device="cuda")
    scale = torch.ones(1, device="cuda")
    scale_inv = torch.ones(1, device="cuda")
    amax = torch.full((1,), 7.0, device="cuda")
    ws = torch.zeros(q.DELAYED_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
    st = oracle.DelayedState(L, fmt, margin=1)
    for t in range(steps):
        xb = workloads.delayed_4096_step(t, rows, cols, out_cols=8)["X"]
        if t % 7 == 3:
            xb = np.zeros_like(xb)  # an all-zero step keeps the scale
        xf = bf16_bits_to_f32(xb)
        if t == 5 and L == 16:
            xf = xf.copy()
            xf[3, 7] = np.nan  # a NaN amax keeps the scale while it is in the window
        xd = to_dev(xf) if dtype == "f32" else to_dev_bf16(workloads.f32_to_bf16_bits(xf) if t == 5 else xb)
        qq, qt = empty_u8((rows, cols)), empty_u8((cols, rows))
        q.qsg_cast_transpose_delayed(xd, code, 1, hist, t, scale, scale_inv, qq, qt, amax, ws)
        rq, rqt, ra, used, _ = st.step(xf, t)
        gq = to_np(qq)
        nan = np.isnan(xf)
        assert np.array_equal(gq[~nan], rq[~nan]), t
        assert np.all((gq[nan] & 0x7F) == 0x7F)
        assert np.array_equal(to_np(qt), gq.T), t
        assert f32bits(to_np(amax))[0] == f32bits(ra)[()], t
        assert f32bits(to_np(scale))[0] == f32bits(st.scale)[()], t
        assert f32bits(to_np(scale_inv))[0] == f32bits(st.scale_inv)[()], t
        assert not to_np(ws).any(), t
    assert np.array_equal(f32bits(to_np(hist)), f32bits(st.history))


def test_cast_transpose_delayed_matches_two_calls_and_empty(q):
    """Against the two-call path (qsg_cast_transpose + qsg_amax_update) on the
    delayed workload's shape, bit for bit; an empty tensor records amax 0."""
    import torch

    R, C, L = 1024, 4096, 1024
    outs = {}
    for path in ("one", "two"):
        hist = torch.zeros(L, device="cuda")
        scale, inv = torch.ones(1, device="cuda"), torch.ones(1, device="cuda")
        amax = torch.zeros(1, device="cuda")
        ws = torch.zeros(q.DELAYED_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
        qq, qt = empty_u8((R, C)), empty_u8((C, R))
        for t in range(3):
            xd = to_dev_bf16(workloads.delayed_4096_step(t, R, C, out_cols=8)["X"])
            if path == "one":
                q.qsg_cast_transpose_delayed(xd, q.E4M3, 0, hist, t, scale, inv, qq, qt, amax, ws)
            else:
                q.qsg_cast_transpose(xd, q.E4M3, scale, qq, qt, amax)
                q.qsg_amax_update(hist, t, amax, q.E4M3, 0, scale, inv)
        outs[path] = [to_np(x).copy() for x in (qq, qt, amax, scale, inv, hist)]
    for a, b in zip(outs["one"], outs["two"]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    hist = torch.full((4,), 3.0, device="cuda")
    scale, inv = torch.ones(1, device="cuda"), torch.ones(1, device="cuda")
    amax = torch.full((1,), 9.0, device="cuda")
    ws = torch.zeros(q.DELAYED_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q.qsg_cast_transpose_delayed(e, q.E4M3, 0, hist, 6, scale, inv, None, None, amax, ws)
    assert to_np(amax)[0] == 0.0
    assert to_np(hist).tolist() == [3.0, 3.0, 0.0, 3.0]
    assert to_np(scale)[0] == np.float32(448.0 / 3.0)


def test_amax_update_nan_keeps_scale(q):
    import torch

    hist = torch.zeros(3, device="cuda")
    scale = torch.tensor([5.0], device="cuda")
    inv = torch.tensor([0.2], device="cuda")
    q.qsg_amax_update(hist, 0, torch.tensor([float("nan")], device="cuda"), q.E5M2, 0, scale, inv)
    assert to_np(scale)[0] == 5.0 and to_np(inv)[0] == np.float32(0.2)
    q.qsg_amax_update(hist, 1, torch.tensor([2.0], device="cuda"), q.E5M2, 0, scale, inv)
    assert to_np(scale)[0] == 5.0  # the NaN is still in the window
    q.qsg_amax_update(hist, 3, torch.tensor([2.0], device="cuda"), q.E5M2, 0, scale, inv)
    assert to_np(scale)[0] == np.float32(57344 / 2)


# ---------------------------------------------------------------------------
# MXFP8 and blockwise
# ---------------------------------------------------------------------------
MX_SHAPES = [(32, 32), (96, 160), (256, 512), (160, 4128), (1056, 288)]


@pytest.mark.parametrize("shape", MX_SHAPES)
@pytest.mark.parametrize("fmt,code", FMTS)
@pytest.mark.parametrize("rule", ["ceil", "ocp"])
def test_mx_quantize(q, shape, fmt, code, rule):
    g = workloads.generator(15, *shape)
    x = (g.standard_normal(shape) * np.exp(g.uniform(-8, 8, (shape[0], 1)))).astype(np.float32)
    x[0, :32] = 0
    x[min(3, shape[0] - 1), 5] = 3e4
    bits = workloads.f32_to_bf16_bits(x)
    xf = bf16_bits_to_f32(bits)
    R, C = shape
    qq, s, qt, st = empty_u8((R, C)), empty_u8((R, C // 32)), empty_u8((C, R)), empty_u8((C, R // 32))
    margin = 1 if rule == "ocp" else 0
    q.qsg_quantize(to_dev_bf16(bits), q.MXFP8, code, q=qq, s=s, qt=qt, st=st, margin=margin,
                   mx_rule=q.MX_CEIL if rule == "ceil" else q.MX_OCP_FLOOR)
    ref = oracle.mx_quantize(xf, fmt, rule, margin)
    assert np.array_equal(to_np(s), ref["s"])
    assert np.array_equal(to_np(qq), ref["q"])
    assert np.array_equal(to_np(st), ref["st"])
    assert np.array_equal(to_np(qt), ref["qt"])


def test_mx_quantize_fp32_and_one_sided(q):
    g = workloads.generator(16)
    x = (g.standard_normal((128, 256)) * 1e-3).astype(np.float32)
    x[4, :] = 1e-41  # subnormal block amax
    ref = oracle.mx_quantize(x, "e4m3", "ceil")
    qq, s = empty_u8((128, 256)), empty_u8((128, 8))
    q.qsg_quantize(to_dev(x), q.MXFP8, q.E4M3, q=qq, s=s)
    assert np.array_equal(to_np(qq), ref["q"]) and np.array_equal(to_np(s), ref["s"])
    qt, st = empty_u8((256, 128)), empty_u8((256, 4))
    q.qsg_quantize(to_dev(x), q.MXFP8, q.E4M3, qt=qt, st=st)
    assert np.array_equal(to_np(qt), ref["qt"]) and np.array_equal(to_np(st), ref["st"])


@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 1152), (640, 256)])
@pytest.mark.parametrize("fmt,code", FMTS)
def test_block_1x128(q, shape, fmt, code):
    import torch

    x = workloads.student_t([17, shape[0]], shape)
    xf = bf16_bits_to_f32(x)
    xf_zero = xf.copy()
    R, C = shape
    qq, qt = empty_u8((R, C)), empty_u8((C, R))
    s = torch.empty((R, C // 128), device="cuda")
    st = torch.empty((C, R // 128), device="cuda")
    q.qsg_quantize(to_dev_bf16(x), q.BLOCK_1X128, code, q=qq, s=s, qt=qt, st=st)
    ref = oracle.block_quantize_1x128(xf_zero, fmt)
    assert np.array_equal(f32bits(to_np(s)), f32bits(ref["s"]))
    assert np.array_equal(f32bits(to_np(st)), f32bits(ref["st"]))
    assert np.array_equal(to_np(qq), ref["q"])
    assert np.array_equal(to_np(qt), ref["qt"])


@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (640, 256)])
def test_block_128x128(q, shape):
    import torch

    x = workloads.student_t([18, shape[0]], shape)
    xf = bf16_bits_to_f32(x)
    R, C = shape
    qq, qt = empty_u8((R, C)), empty_u8((C, R))
    s = torch.empty((R // 128, C // 128), device="cuda")
    st = torch.empty((C // 128, R // 128), device="cuda")
    q.qsg_quantize(to_dev_bf16(x), q.BLOCK_128X128, q.E4M3, q=qq, s=s, qt=qt, st=st, margin=1)
    ref = oracle.block_quantize_128x128(xf, "e4m3", margin=1)
    assert np.array_equal(f32bits(to_np(s)), f32bits(ref["s"]))
    assert np.array_equal(f32bits(to_np(st)), f32bits(ref["st"]))
    assert np.array_equal(to_np(qq), ref["q"])
    assert np.array_equal(to_np(qt), ref["qt"])


def test_block_zero_block_scale_one(q):
    import torch

    x = np.zeros((128, 256), np.float32)
    x[:, 128:] = 2.0
    qq, s = empty_u8((128, 256)), torch.empty((128, 2), device="cuda")
    q.qsg_quantize(to_dev(x), q.BLOCK_1X128, q.E4M3, q=qq, s=s)
    got = to_np(s)
    assert np.all(got[:, 0] == 1.0) and np.all(got[:, 1] == np.float32(1.0) / np.float32(224.0))
