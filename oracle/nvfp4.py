"""NVFP4 block scaling: E2M1 elements, one E4M3 scale per 1 x 16 block and one
fp32 scale per tensor; the GEMM on NVFP4 operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the recipe and the element format only ("Low-Precision
Training Guide": recipe "nvfp4", "NVFP4 block scaling", --fp4-format e2m1;
table "Hardware and Recipe Compatibility", row nvfp4).  They give neither the
block size nor the scale formats.  Reading R14 takes them from NVIDIA's
published definition of NVFP4, outside the pages:

  * elements: E2M1 (OCP FP4): sign | 2 exponent bits (bias 1) | 1 mantissa
    bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity, no NaN;
  * blocks: 16 consecutive elements along the contraction dimension, each
    with a decode scale stored as an E4M3 byte;
  * a second, per-tensor fp32 scale s_enc = 448 * 6 / amax(tensor), which
    places the largest block's decode scale at the top of the E4M3 range.

Quantization of one block with block maximum b (every step one binary32
operation, rounded to nearest even; the column-wise copy uses blocks of 16
rows and is stored transposed, as for MXFP8):

  sdec  = fp32(b / 6)
  code  = enc_e4m3(fp32(sdec * s_enc))   (saturating RNE, fp8.encode)
  S     = dec_e4m3(code)
  m     = fp32(s_enc / S)                (0 when S is 0: the block is all zero
                                          or too small for E4M3)
  q     = enc_e2m1(fp32(x * m))          (saturating RNE, ties to the even code)

with s_enc = fp32(448 * 6 / amax), 1 for amax 0 or not finite, FLT_MAX on
overflow (as the per-tensor scale of the FP8 recipes).  The dequantized value
is dec_e2m1(q) * S / s_enc, so the GEMM multiplies each product of decoded
codes by S_a S_b and the sum by s_dec_a s_dec_b, s_dec = fp32(1 / s_enc).

Packing: two codes per byte along the row, element 2i in the low nibble.
E2M1 encoding reading: values >= 6 (and infinities) saturate to 6 with their
sign; NaN (outside the recipe's contract) gives sign | 6; the sign of zero is
kept (code 0x8).
"""

from fractions import Fraction

import numpy as np

from .fp8 import decode_exact as _fp8_decode_exact
from .fp8 import decode_table as _fp8_table
from .fp8 import encode as _fp8_encode

E2M1_MAX = 6.0
FP8_MAX = 448.0
BLOCK = 16


# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------
def decode_e2m1_exact(code):
    """Value of a 4-bit E2M1 code as a Fraction, from the bit layout:
    exponent field e, mantissa bit m: e = 0 -> m / 2, else (1 + m/2) 2^(e-1)."""
    code = int(code) & 0xF
    s = -1 if code & 0x8 else 1
    e = (code >> 1) & 0x3
    m = code & 1
    v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return s * v


def decode_e2m1_table():
    t = np.array([float(decode_e2m1_exact(c)) for c in range(16)], dtype=np.float64)
    t[8] = -0.0  # the sign of zero (a Fraction has none)
    return t


def _rne_int(r):
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl + (fl & 1)


def encode_e2m1_exact(bits):
    """Saturating RNE E2M1 encode of one binary32 value given by its bit
    pattern, following the generic binary floating-point rounding:
      1. the sign is kept;  2. NaN gives sign|6 (reading);  3. magnitudes >= 6
      saturate;  4. below 1 (the smallest normal) the value is rounded to a
      multiple of 1/2, ties to even (a round-up to 2 halves is the code of 1);
      5. otherwise the mantissa is rounded to one bit, a carry bumping the
      exponent."""
    bits = int(bits) & 0xFFFFFFFF
    s = (bits >> 31) & 1
    absb = bits & 0x7FFFFFFF
    if absb > 0x7F800000:
        return (s << 3) | 0x7
    if absb == 0x7F800000:
        return (s << 3) | 0x7
    e = (absb >> 23) & 0xFF
    man = absb & 0x7FFFFF
    a = Fraction(man, 1 << 23) * Fraction(2) ** (-126) if e == 0 else \
        Fraction(man | 0x800000, 1 << 23) * Fraction(2) ** (e - 127)
    if a >= 6:
        return (s << 3) | 0x7
    if a < 1:
        return (s << 3) | _rne_int(a * 2)  # 0, 1 or 2 (= the code of 1.0)
    E = 0
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    q = _rne_int((a / Fraction(2) ** E - 1) * 2)
    if q == 2:
        q = 0
        E += 1
    return (s << 3) | ((E + 1) << 1) | q


_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def encode_e2m1(x):
    """Vectorised saturating RNE E2M1 encode of a float32 array (uint8 codes
    0..15): the nearest of the 8 magnitudes, ties (the midpoints) to the even
    code, NaN -> sign|6."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = ((u >> 31) & 1).astype(np.uint8) << 3
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    lo = np.searchsorted(_MID, a, side="left")
    hi = np.searchsorted(_MID, a, side="right")
    tie = lo != hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), lo)
    code = np.where(np.isnan(x), 7, code)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------
def pack(codes):
    """rows x cols codes (cols even) -> rows x cols/2 bytes, element 2i low."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# scales and quantization
# --------------------------------------------------------------------------
def tensor_scale(amax):
    """(s_enc, s_dec): s_enc = fp32(448 * 6 / amax); 1 for amax 0 or not
    finite; FLT_MAX when the quotient overflows; s_dec = fp32(1 / s_enc)."""
    a = np.float32(amax)
    if a == 0 or not np.isfinite(a):
        s = np.float32(1.0)
    else:
        with np.errstate(over="ignore"):
            s = np.float32(np.float32(FP8_MAX * E2M1_MAX) / a)
        if not np.isfinite(s):
            s = np.float32(np.finfo(np.float32).max)
    return s, np.float32(np.float32(1.0) / s)


def _quantize_rows(x, s_enc):
    """Row-wise NVFP4 of a float32 matrix whose column count is a multiple of
    16: (codes rows x cols, E4M3 scale bytes rows x cols/16)."""
    R, C = x.shape
    blocks = np.abs(x).reshape(R, C // BLOCK, BLOCK)
    with np.errstate(invalid="ignore"):
        bmax = blocks.max(axis=2).astype(np.float32)
    sdec = (bmax / np.float32(E2M1_MAX)).astype(np.float32)
    with np.errstate(over="ignore"):
        code = _fp8_encode((sdec * np.float32(s_enc)).astype(np.float32), "e4m3")
    S = _fp8_table("e4m3")[code].astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        m = np.where(S > 0, np.float32(s_enc) / np.where(S > 0, S, np.float32(1)), np.float32(0)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (x.reshape(R, C // BLOCK, BLOCK) * m[:, :, None]).astype(np.float32).reshape(R, C)
    return encode_e2m1(v), code


def quantize_rows(x, s_enc):
    """Row-wise NVFP4 of some rows of a tensor whose tensor scale s_enc is
    already known (each row's blocks depend only on the row and s_enc):
    (packed q, E4M3 scale bytes)."""
    c, s = _quantize_rows(np.ascontiguousarray(x, dtype=np.float32), np.float32(s_enc))
    return pack(c), s


def quantize(x, rowwise=True, colwise=True):
    """NVFP4 row-wise (blocks of 16 along a row) and column-wise (blocks of 16
    along a column, stored transposed) copies of a float32 matrix.  Returns a
    dict: q (rows x cols/2 packed), s (rows x cols/16 E4M3 bytes), qt
    (cols x rows/2), st (cols x rows/16), amax, s_enc, s_dec."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if np.isnan(x).any():
        a = np.float32(np.nan)
    s_enc, s_dec = tensor_scale(a)
    out = {"amax": a, "s_enc": s_enc, "s_dec": s_dec}
    if rowwise:
        c, s = _quantize_rows(x, s_enc)
        out["q"], out["s"] = pack(c), s
    if colwise:
        c, s = _quantize_rows(np.ascontiguousarray(x.T), s_enc)
        out["qt"], out["st"] = pack(c), s
    return out


def dequantize(q, s, s_dec):
    """fp64 values of a packed NVFP4 matrix: dec(q) * dec_e4m3(s) * s_dec."""
    codes = unpack(q)
    R, C = codes.shape
    vals = decode_e2m1_table()[codes]
    S = np.repeat(_fp8_table("e4m3")[np.asarray(s, dtype=np.uint8)].astype(np.float64), BLOCK, axis=1)[:, :C]
    return vals * S * np.float64(np.float32(s_dec))


def gemm(qa, sa, s_dec_a, qb, sb, s_dec_b):
    """C = A B^T on NVFP4 operands (A M x K, B N x K, both row-wise copies),
    accumulated in fp64 and not rounded: the products of the exactly decoded
    block values are summed, then multiplied by s_dec_a * s_dec_b."""
    A = dequantize(qa, sa, 1.0)
    B = dequantize(qb, sb, 1.0)
    return (A @ B.T) * (np.float64(np.float32(s_dec_a)) * np.float64(np.float32(s_dec_b)))


def quantize_loop(x):
    """The row-wise quantization of ``quantize`` written as a plain loop over
    blocks and elements, with numpy float32 scalar arithmetic for the scale
    steps and the exact encoders; for small pins only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    amax = np.float32(0)
    for v in x.ravel():
        amax = max(amax, np.float32(abs(v)))
    s_enc, _ = tensor_scale(amax)
    codes = np.zeros((R, C), dtype=np.uint8)
    scales = np.zeros((R, C // BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(C // BLOCK):
            blk = x[r, b * BLOCK:(b + 1) * BLOCK]
            bmax = np.float32(0)
            for v in blk:
                bmax = max(bmax, np.float32(abs(v)))
            sdec = np.float32(bmax / np.float32(6))
            prod = np.float32(sdec * s_enc)
            sc = int(_fp8_encode(np.array([prod], dtype=np.float32), "e4m3")[0])
            S = np.float32(float(_fp8_decode_exact(sc, "e4m3")))
            m = np.float32(s_enc / S) if S > 0 else np.float32(0)
            scales[r, b] = sc
            for i in range(BLOCK):
                v = np.float32(blk[i] * m)
                codes[r, b * BLOCK + i] = encode_e2m1_exact(int(np.array(v, dtype=np.float32).view(np.uint32)))
    return codes, scales, s_enc
