"""Pins of the NVFP4 oracle (oracle/nvfp4.py; reading R14: E2M1 elements,
E4M3 scale per 1 x 16 block, fp32 tensor scale, as NVIDIA defines NVFP4).

* the E2M1 code table against the bit layout's closed form, written out;
* the vectorised encoder against the exact rational encoder on every bf16
  pattern, every code and midpoint with its float32 neighbours, and random
  fp32 values; every code round-trips;
* a two-block example worked by hand (tests/golden/nvfp4_blocks.txt);
* the vectorised quantizer against a plain per-block, per-element loop, with
  zero, tiny (flushed) and heavy-tailed blocks, both copies;
* the dequantization error stays within half an E2M1 step of the scaled
  value (or the saturation amount), scaled back;
* the GEMM against exact rational brute force, with a planted error.
"""

import os
from fractions import Fraction

import numpy as np

from oracle import nvfp4

GOLD = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_blocks.txt")


def f32bits(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def test_e2m1_table_closed_form():
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    got = [float(nvfp4.decode_e2m1_exact(c)) for c in range(16)]
    assert got == want
    assert np.signbit(nvfp4.decode_e2m1_table()[8])  # code 8 is -0


def test_e2m1_encoders_agree_everywhere():
    # every bf16 pattern (covers all binades, specials, subnormals)
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    x = b.view(np.float32)
    vec = nvfp4.encode_e2m1(x)
    ex = np.array([nvfp4.encode_e2m1_exact(int(v)) for v in b], dtype=np.uint8)
    assert np.array_equal(vec, ex)
    # codes and midpoints with their float32 neighbours, both signs
    pts = [0.0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 1e30]
    vals = []
    for p in pts:
        f = np.float32(p)
        vals += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    g = np.random.Generator(np.random.PCG64(5))
    vals = np.concatenate([vals, (g.standard_normal(20000) * np.exp2(g.uniform(-12, 6, 20000))).astype(np.float32)])
    assert np.array_equal(nvfp4.encode_e2m1(vals),
                          np.array([nvfp4.encode_e2m1_exact(f32bits(v)) for v in vals], dtype=np.uint8))


def test_e2m1_round_trip_ties_and_saturation():
    for c in range(16):
        v = np.float32(float(nvfp4.decode_e2m1_exact(c)))
        if c == 8:
            v = np.float32(-0.0)
        assert nvfp4.encode_e2m1_exact(f32bits(v)) == c
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert nvfp4.encode_e2m1_exact(f32bits(v)) == c
        assert nvfp4.encode_e2m1_exact(f32bits(-v)) == 8 | c
    for v in (6.0, 6.5, 1e9, np.inf):
        assert nvfp4.encode_e2m1_exact(f32bits(v)) == 7
        assert nvfp4.encode_e2m1_exact(f32bits(-v)) == 15


def read_gold():
    xs, codes, scales, s_enc = [], [], {}, None
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "scale":
            scales[int(parts[1])] = int(parts[2], 16)
        elif parts[0] == "s_enc":
            s_enc = float(parts[1])
        else:
            xs.append(np.float32(float(parts[1])) if parts[1] != "-0" else np.float32(-0.0))
            codes.append(int(parts[2]))
    return np.array(xs, dtype=np.float32)[None, :], np.array(codes, dtype=np.uint8), scales, s_enc


def test_worked_example():
    x, codes, scales, s_enc = read_gold()
    r = nvfp4.quantize(x, colwise=False)
    assert float(r["s_enc"]) == s_enc
    assert r["s"].tolist() == [[scales[0], scales[1]]]
    assert nvfp4.unpack(r["q"])[0].tolist() == codes.tolist()
    c, s, se = nvfp4.quantize_loop(x)
    assert c[0].tolist() == codes.tolist() and s.tolist() == [[scales[0], scales[1]]] and se == np.float32(s_enc)


def sample(g, R, C):
    x = (g.standard_t(3, (R, C)) * np.exp2(g.uniform(-6, 6, (R, 1)))).astype(np.float32)
    x[0, :16] = 0                      # an all-zero block
    x[1, 16:32] *= np.float32(2 ** -30)  # a block too small for its E4M3 scale
    x[2, 5] = np.float32(-0.0)
    return x


def test_quantize_matches_loop_both_copies():
    g = np.random.Generator(np.random.PCG64(6))
    x = sample(g, 32, 64)
    r = nvfp4.quantize(x)
    c, s, se = nvfp4.quantize_loop(x)
    assert r["s_enc"] == se
    assert np.array_equal(nvfp4.unpack(r["q"]), c) and np.array_equal(r["s"], s)
    ct, stt, _ = nvfp4.quantize_loop(np.ascontiguousarray(x.T))
    # the column copy uses the tensor's own s_enc, so it matches the loop on x^T
    assert np.array_equal(nvfp4.unpack(r["qt"]), ct) and np.array_equal(r["st"], stt)
    assert np.all(nvfp4.unpack(r["q"])[0, :16] == 0)


def test_dequantization_error_bound():
    g = np.random.Generator(np.random.PCG64(7))
    x = sample(g, 64, 128)
    r = nvfp4.quantize(x, colwise=False)
    S = nvfp4._fp8_table("e4m3")[r["s"]].astype(np.float64)
    s_enc = np.float64(r["s_enc"])
    m = np.where(S > 0, np.float32(s_enc) / np.where(S > 0, S, 1).astype(np.float32), 0).astype(np.float32)
    v = np.abs((x.reshape(64, 8, 16) * m[:, :, None]).astype(np.float32).astype(np.float64))
    deq = np.abs(nvfp4.decode_e2m1_table()[nvfp4.unpack(r["q"])]).reshape(64, 8, 16)
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    err = np.abs(deq - v)
    assert np.all((err <= step / 2) | ((v > 6) & (deq == 6)))
    # back in real units, through the block and tensor scales
    full = nvfp4.dequantize(r["q"], r["s"], r["s_dec"])
    live = (S > 0).repeat(16, axis=1)
    rel = np.abs(full - x)[live] / (S.repeat(16, axis=1)[live] / s_enc)
    assert np.all(rel <= 1.0 + 2.0 ** -20)


def test_gemm_exact_and_planted():
    g = np.random.Generator(np.random.PCG64(8))
    A = sample(g, 5, 48)
    B = (g.standard_normal((4, 48)) * 0.01).astype(np.float32)
    ra, rb = nvfp4.quantize(A, colwise=False), nvfp4.quantize(B, colwise=False)
    y = nvfp4.gemm(ra["q"], ra["s"], ra["s_dec"], rb["q"], rb["s"], rb["s_dec"])
    ca, cb = nvfp4.unpack(ra["q"]), nvfp4.unpack(rb["q"])
    from oracle.fp8 import decode_exact as d8
    sda, sdb = Fraction(float(ra["s_dec"])), Fraction(float(rb["s_dec"]))
    for m in range(5):
        for n in range(4):
            ex = sum(nvfp4.decode_e2m1_exact(ca[m, k]) * d8(int(ra["s"][m, k // 16]), "e4m3")
                     * nvfp4.decode_e2m1_exact(cb[n, k]) * d8(int(rb["s"][n, k // 16]), "e4m3")
                     for k in range(48)) * sda * sdb
            assert abs(Fraction(y[m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
    # a planted sign error in one block scale must show
    sa_bad = ra["s"].copy()
    sa_bad[2, 1] ^= 0x01
    y_bad = nvfp4.gemm(ra["q"], sa_bad, ra["s_dec"], rb["q"], rb["s"], rb["s_dec"])
    assert not np.allclose(y_bad[2], y[2], rtol=1e-3, atol=0)
