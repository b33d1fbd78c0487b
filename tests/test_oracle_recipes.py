"""Pins of the oracle's scaling recipes.

* per-tensor scale: closed forms (amax = fmax, powers of two, margin) and a
  single exact rounding of the rational fmax/amax computed here with
  fractions (not with a binary32 division);
* delayed scaling: a trajectory worked out by hand (tests/golden/delayed_l4.txt)
  including the wrap-around of the window;
* mxfp8: the minimality invariant amax*2^-e <= fmax < amax*2^-(e-1) checked
  with exact rationals, the OCP floor rule against math.frexp, clamping and the
  zero block, and a pure-Python loop quantizer on tiny tensors;
* blockwise: a pure-Python loop quantizer on tiny tensors and the dequantization
  error bound of round-to-nearest.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.fp8 import FORMATS

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")
FLT_MAX = float(np.finfo(np.float32).max)


def f32_round_exact(fr):
    """Round a positive Fraction to binary32, nearest even, by exact integer
    arithmetic (subnormal results included, no overflow)."""
    assert fr > 0
    n, d = fr.numerator, fr.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    if Fraction(2) ** (e + 1) <= fr:
        e += 1
    assert e <= 127
    qexp = max(e, -126) - 23  # binary32 spacing near fr
    sig = fr / Fraction(2) ** qexp
    lo = sig.numerator // sig.denominator
    rem = sig - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return np.float32(math.ldexp(lo, qexp))


def bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


# ---------------------------------------------------------------------------
# per-tensor scale
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_scale_closed_forms(fmt):
    fmax = FORMATS[fmt]["max"]
    s, si = oracle.tensorwise_scale(np.float32(fmax), fmt)
    assert (s, si) == (1.0, 1.0)
    for k in range(-20, 21):
        for margin in (0, 1, 3):
            s, si = oracle.tensorwise_scale(np.float32(2.0 ** k), fmt, margin)
            assert s == np.float32(fmax * 2.0 ** (-k - margin))
            # scale_inv of fmax*2^j is 2^-j/fmax, one rounding
            assert si == f32_round_exact(1 / Fraction(s.item()))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_scale_single_rounding(fmt):
    fmax = Fraction(FORMATS[fmt]["max"])
    g = np.random.Generator(np.random.PCG64(7))
    amaxes = (np.exp(g.uniform(-30, 30, 3000))).astype(np.float32)
    for a in amaxes:
        for margin in (0, 2):
            s, si = oracle.tensorwise_scale(a, fmt, margin)
            s0 = f32_round_exact(fmax / Fraction(float(a)))
            assert s == np.float32(float(s0) * 2.0 ** -margin)
            assert si == f32_round_exact(1 / Fraction(float(s)))


def test_scale_special_cases():
    for a in (0.0, -0.0, float("inf"), float("nan")):
        assert oracle.tensorwise_scale(np.float32(a), "e4m3") == (1.0, 1.0)
    # a subnormal amax: the quotient overflows, the scale saturates
    s, si = oracle.tensorwise_scale(np.float32(1e-45), "e4m3")
    assert s == np.float32(FLT_MAX)
    assert si == f32_round_exact(1 / Fraction(FLT_MAX))


def test_amax_definition():
    x = np.array([[1.0, -3.5], [-0.0, 2.0]], dtype=np.float32)
    assert oracle.amax(x) == 3.5
    assert oracle.amax(np.zeros((0, 4), np.float32)) == 0
    assert oracle.amax(np.array([-0.0], np.float32)) == 0
    assert np.isnan(oracle.amax(np.array([1.0, np.nan], np.float32)))
    assert oracle.amax(np.array([1.0, -np.inf], np.float32)) == np.inf


def test_cast_transpose_is_transpose_and_encode():
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal((37, 53)).astype(np.float32)
    q, qt = oracle.cast_transpose(x, np.float32(10.0), "e4m3")
    assert np.array_equal(qt, q.T)
    for r in range(0, 37, 5):
        for c in range(0, 53, 7):
            v = np.float32(x[r, c] * np.float32(10.0))
            assert q[r, c] == oracle.encode_exact(bits(v), "e4m3")


# ---------------------------------------------------------------------------
# delayed scaling
# ---------------------------------------------------------------------------
def _delayed_golden():
    rows = []
    with open(os.path.join(GOLDEN_DIR, "delayed_l4.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                t, a, used, nxt = line.split()
                rows.append((int(t), Fraction(a), Fraction(used), Fraction(nxt)))
    return rows


def test_delayed_trajectory_hand_worked():
    rows = _delayed_golden()
    hist = np.zeros(4, np.float32)
    scale, inv = np.float32(1), np.float32(1)
    for t, a, used, nxt in rows:
        assert scale == f32_round_exact(used)
        scale, inv = oracle.amax_update(hist, t, np.float32(float(a)), "e4m3", 0, scale, inv)
        assert scale == f32_round_exact(nxt), t
        assert inv == f32_round_exact(1 / Fraction(float(scale)))


def test_delayed_state_quantizes_with_previous_scale():
    st = oracle.DelayedState(8, "e5m2")
    x0 = np.full((4, 4), 2.0, np.float32)
    q, qt, a, used, _ = st.step(x0, 0)
    assert used == 1.0 and a == 2.0
    assert np.all(q == oracle.encode(np.full((4, 4), 2.0, np.float32), "e5m2"))
    assert st.scale == np.float32(57344 / 2)
    q, qt, a, used, _ = st.step(x0 * 4, 1)
    assert used == np.float32(57344 / 2)  # the scale of step 1 comes from step 0's amax
    assert st.scale == np.float32(57344 / 8)


def test_delayed_keeps_scale_on_zero_or_nan():
    hist = np.zeros(2, np.float32)
    s, i = oracle.amax_update(hist, 0, np.float32(0), "e4m3", 0, np.float32(1), np.float32(1))
    assert (s, i) == (1, 1)
    s, i = oracle.amax_update(hist, 1, np.float32(4), "e4m3", 0, s, i)
    assert s == 112
    s2, i2 = oracle.amax_update(hist, 2, np.float32(np.nan), "e4m3", 0, s, i)
    assert (s2, i2) == (s, i)
    s3, _ = oracle.amax_update(hist, 3, np.float32(1), "e4m3", 1, s2, i2)
    # window holds [nan, 1] at step 3? slot 0 = nan (step 2), slot 1 = 1 (step 3)
    assert s3 == s2
    s4, _ = oracle.amax_update(hist, 4, np.float32(2), "e4m3", 1, s3, i2)
    # window [2, 1]: max 2, margin 1 -> 448/2/2
    assert s4 == 112


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------
EMAX = {"e4m3": 8, "e5m2": 15}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mx_exponent_minimal(fmt):
    fmax = Fraction(FORMATS[fmt]["max"])
    g = np.random.Generator(np.random.PCG64(11))
    a = np.exp(g.uniform(-80, 80, 5000)).astype(np.float32)
    a = np.concatenate([a, np.float32([448, 449, 447, 57344, 1.75, 1.7500001, 1.0, 2.0 ** -130, 3e-39])])
    e = oracle.mx_exponent(a, fmt, "ceil")
    for ai, ei in zip(a, e):
        if -127 < ei < 127:
            fa = Fraction(float(ai))
            assert fa * Fraction(2) ** (-int(ei)) <= fmax
            assert fa * Fraction(2) ** (-int(ei) + 1) > fmax


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mx_exponent_ocp_floor(fmt):
    g = np.random.Generator(np.random.PCG64(12))
    a = np.exp(g.uniform(-80, 80, 5000)).astype(np.float32)
    a = np.concatenate([a, np.float32([2.0 ** -140, 1e-45, 448, 512])])
    e = oracle.mx_exponent(a, fmt, "ocp")
    for ai, ei in zip(a, e):
        m, x = math.frexp(float(ai))
        assert ei == max(-127, min(127, (x - 1) - EMAX[fmt]))


def test_mx_exponent_edges():
    a = np.float32([0.0, 2.0 ** -149, FLT_MAX, np.inf])
    e = oracle.mx_exponent(a, "e4m3", "ceil")
    # 0 -> 0; 2^-149 -> -157 clamped to -127; FLT_MAX = (2-2^-23)*2^127 -> 127-8+1
    # inf reads as E = 128, f = 0 -> 120
    assert list(e) == [0, -127, 120, 120]
    assert list(oracle.mx_exponent(np.float32([448.0]), "e4m3", "ceil", margin=2)) == [2]


def _mx_loop(x, fmt, rule):
    """Pure-Python loop MX row quantizer for tiny tensors."""
    R, C = x.shape
    fmax = FORMATS[fmt]["max"]
    q = np.zeros((R, C), np.uint8)
    s = np.zeros((R, C // 32), np.uint8)
    for r in range(R):
        for b in range(C // 32):
            blk = [float(v) for v in x[r, 32 * b:32 * b + 32]]
            a = max(abs(v) for v in blk)
            if a == 0:
                e = 0
            else:
                m, ex = math.frexp(a)
                E = ex - 1
                e = E - EMAX[fmt]
                if rule == "ceil" and 2 * m > 1.75:
                    e += 1
                e = max(-127, min(127, e))
                if rule == "ceil":
                    assert a * 2.0 ** -e <= fmax
            s[r, b] = e + 127
            for j, v in enumerate(blk):
                p = np.float32(np.float32(v) * np.float32(2.0 ** -e))
                q[r, 32 * b + j] = oracle.encode_exact(bits(p), fmt)
    return q, s


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rule", ["ceil", "ocp"])
def test_mx_quantize_matches_loop(fmt, rule):
    g = np.random.Generator(np.random.PCG64(5))
    x = (g.standard_normal((64, 96)) * np.exp(g.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[3, :32] = 0.0  # a zero block
    x[5, 40] = 1e4  # an outlier
    out = oracle.mx_quantize(x, fmt, rule)
    q, s = _mx_loop(x, fmt, rule)
    assert np.array_equal(out["q"], q) and np.array_equal(out["s"], s)
    qt, st = _mx_loop(np.ascontiguousarray(x.T), fmt, rule)
    assert np.array_equal(out["qt"], qt) and np.array_equal(out["st"], st)
    assert np.all(out["s"][3, 0] == 127)


def test_mx_ceil_never_saturates_ocp_can():
    g = np.random.Generator(np.random.PCG64(9))
    x = (g.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    ceil = oracle.mx_quantize(x, "e4m3", "ceil", colwise=False)["q"]
    ocp = oracle.mx_quantize(x, "e4m3", "ocp", colwise=False)["q"]
    # ceil: |x * 2^-e| <= 448 always, so a max code only appears for values that
    # are exactly representable there; floor saturates a fraction of elements
    fx = oracle.dequantize(ocp, "e4m3")
    assert np.sum(np.abs(fx) == 448) > 0
    dc = oracle.dequantize(ceil, "e4m3")
    assert np.all(np.abs(dc) <= 448)


# ---------------------------------------------------------------------------
# blockwise
# ---------------------------------------------------------------------------
def _block_loop_rows(x, fmt, bc):
    R, C = x.shape
    q = np.zeros((R, C), np.uint8)
    s = np.zeros((R, C // bc), np.float32)
    fmax = Fraction(FORMATS[fmt]["max"])
    for r in range(R):
        for b in range(C // bc):
            blk = x[r, bc * b:bc * b + bc]
            a = max(abs(float(v)) for v in blk)
            sc = np.float32(1.0) if a == 0 else f32_round_exact(fmax / Fraction(a))
            s[r, b] = f32_round_exact(1 / Fraction(float(sc)))
            for j in range(bc):
                p = np.float32(blk[j] * sc)
                q[r, bc * b + j] = oracle.encode_exact(bits(p), fmt)
    return q, s


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_1x128_matches_loop(fmt):
    g = np.random.Generator(np.random.PCG64(21))
    x = g.standard_t(3, (128, 256)).astype(np.float32)
    x[7, 128:] = 0
    out = oracle.block_quantize_1x128(x, fmt)
    q, s = _block_loop_rows(x, fmt, 128)
    assert np.array_equal(out["q"], q) and np.array_equal(out["s"], s)
    qt, st = _block_loop_rows(np.ascontiguousarray(x.T), fmt, 128)
    assert np.array_equal(out["qt"], qt) and np.array_equal(out["st"], st)
    assert out["s"][7, 1] == 1.0


def test_block_128x128_matches_loop():
    g = np.random.Generator(np.random.PCG64(22))
    w = g.standard_t(3, (256, 384)).astype(np.float32)
    out = oracle.block_quantize_128x128(w, "e4m3")
    fmax = Fraction(448)
    for br in range(2):
        for bc in range(3):
            blk = w[128 * br:128 * br + 128, 128 * bc:128 * bc + 128]
            a = float(np.max(np.abs(blk)))
            sc = f32_round_exact(fmax / Fraction(a))
            assert out["s"][br, bc] == f32_round_exact(1 / Fraction(float(sc)))
            for (i, j) in [(0, 0), (5, 77), (127, 127), (64, 3)]:
                p = np.float32(blk[i, j] * sc)
                assert out["q"][128 * br + i, 128 * bc + j] == oracle.encode_exact(bits(p), "e4m3")
    assert np.array_equal(out["qt"], out["q"].T)
    assert np.array_equal(out["st"], out["s"].T)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_dequant_error_bound(fmt):
    # round to nearest: |dec(q) - x*s| <= ulp(q)/2, and nothing saturates
    g = np.random.Generator(np.random.PCG64(23))
    x = g.standard_t(3, (64, 512)).astype(np.float32)
    out = oracle.block_quantize_1x128(x, fmt, colwise=False)
    table = oracle.decode_table(fmt)
    dec = table[out["q"]]
    s_inv = np.repeat(out["s"], 128, axis=1).astype(np.float64)
    scale = np.float64(1) / s_inv
    v = x.astype(np.float64) * scale
    M = FORMATS[fmt]["mbits"]
    emin = 1 - FORMATS[fmt]["bias"]
    e = np.floor(np.log2(np.maximum(np.abs(dec), 2.0 ** emin)))
    ulp = 2.0 ** (e - M)
    # the scale itself is rounded to binary32, so allow its relative error
    assert np.all(np.abs(dec - v) <= ulp / 2 + np.abs(v) * 2.0 ** -22)
    assert np.all(np.abs(dec) <= FORMATS[fmt]["max"])


def test_block_scale_matches_tensorwise_scale_elementwise():
    g = np.random.Generator(np.random.PCG64(24))
    with np.errstate(over="ignore"):
        a = np.exp(g.uniform(-100, 100, 4000)).astype(np.float32)  # includes inf
    a = np.concatenate([a, np.float32([0.0, np.inf, np.nan, 1e-45, 448.0, 3e38])])
    for fmt in ("e4m3", "e5m2"):
        for margin in (0, 3):
            s, si = oracle.block_scale(a, fmt, margin)
            for k in range(a.size):
                rs, rsi = oracle.tensorwise_scale(a[k], fmt, margin)
                assert bits(s[k]) == bits(rs) and bits(si[k]) == bits(rsi), (a[k], fmt, margin)
