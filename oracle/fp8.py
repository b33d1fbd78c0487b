"""FP8 E4M3 / E5M2 decode and saturating round-to-nearest-even encode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the two formats ("Low-Precision Training Guide", table
"Hardware and Recipe Compatibility": ``--fp8-format {e4m3,hybrid}``; "Benefits
of Using FP8 Precision with MegaDLMs and Required Hardware", section "Command-Line
Configuration": ``--fp8-format e4m3``) but never print their bit layouts.  The
layouts below are those of the OCP 8-bit floating point specification (OFP8):

  E4M3 ("fn" flavour): sign | 4 exponent bits (bias 7) | 3 mantissa bits.
      exponent 0 is subnormal; exponent 15 with mantissa 7 is NaN; there is no
      infinity; the largest finite value is 448 (code 0x7E).
  E5M2: sign | 5 exponent bits (bias 15) | 2 mantissa bits.
      exponent 0 is subnormal; exponent 31 is infinity (mantissa 0) or NaN;
      the largest finite value is 57344 (code 0x7B).

Encoding reading (the pages are silent; this is the plainest one consistent
with a "saturating" cast): round to nearest, ties to even; every finite input
whose magnitude is at least the format maximum, and every infinity, maps to
the signed maximum code; NaN maps to the NaN code ``sign | 0x7F``; the sign of
zero is kept.

Two implementations are given:
  * ``encode_exact`` works on one value with exact rational arithmetic and
    follows the definition step by step; it is the ground truth.
  * ``encode`` is the same definition written with integer operations on the
    IEEE binary32 bit pattern, vectorised with numpy, for full-size tensors.
The tests pin both against each other on every bfloat16 bit pattern and
against an independent library cast on fp32 inputs.
"""

from fractions import Fraction

import numpy as np

# Format constants from the OCP 8-bit floating point specification.
FORMATS = {
    "e4m3": {"ebits": 4, "mbits": 3, "bias": 7, "max": 448.0, "maxcode": 0x7E,
             "has_inf": False},
    "e5m2": {"ebits": 5, "mbits": 2, "bias": 15, "max": 57344.0, "maxcode": 0x7B,
             "has_inf": True},
}


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return FORMATS[fmt]


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def decode_exact(code, fmt):
    """Value of one FP8 byte: a Fraction, or the floats nan / +-inf.

    Follows the OFP8 layout stated in the module docstring.
    """
    f = _fmt(fmt)
    m_bits, bias = f["mbits"], f["bias"]
    emax_field = (1 << f["ebits"]) - 1
    sign = -1 if (code >> 7) & 1 else 1
    e = (code >> m_bits) & emax_field
    m = code & ((1 << m_bits) - 1)
    if fmt == "e4m3" and e == emax_field and m == (1 << m_bits) - 1:
        return float("nan")
    if fmt == "e5m2" and e == emax_field:
        return float("nan") if m else sign * float("inf")
    if e == 0:
        mag = Fraction(m, 1 << m_bits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << m_bits)) * Fraction(2) ** (e - bias)
    return sign * mag


def decode_table(fmt):
    """float64[256]: the value of every code (NaN / inf as floats)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        v = decode_exact(c, fmt)
        out[c] = float(v)
    return out


def dequantize(q, fmt):
    """Decode an array of FP8 bytes to float64."""
    return decode_table(fmt)[np.asarray(q, dtype=np.uint8)]


# --------------------------------------------------------------------------
# exact scalar encode
# --------------------------------------------------------------------------
def _rne_int(r):
    """Nearest integer to the non-negative Fraction r, ties to the even one."""
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl + (fl & 1)


def _f32_bits_to_fraction(bits):
    """Exact value of a finite binary32 bit pattern (sign dropped)."""
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0:
        return Fraction(m) * Fraction(2) ** (-149)
    return Fraction(m | 0x800000) * Fraction(2) ** (e - 150)


def _floor_log2(a):
    """floor(log2(a)) for a positive Fraction, exactly."""
    n, d = a.numerator, a.denominator
    k = n.bit_length() - d.bit_length()
    # 2^k <= a < 2^(k+1) is off by at most one; fix it exactly.
    if Fraction(2) ** k > a:
        k -= 1
    elif Fraction(2) ** (k + 1) <= a:
        k += 1
    return k


def encode_exact(bits, fmt):
    """Saturating RNE encode of one binary32 value given by its bit pattern.

    Steps, in the order of the definition in the module docstring:
      1. the sign bit is carried through unchanged;
      2. NaN gives sign|0x7F;
      3. a magnitude >= the format maximum (infinity included) saturates;
      4. below the smallest normal the value is a multiple of the smallest
         subnormal, rounded to nearest even (a round-up to 2^M lands exactly
         on the smallest normal code);
      5. otherwise the mantissa is rounded to M bits, a carry bumping the
         exponent.
    """
    f = _fmt(fmt)
    M, bias, fmax, maxcode = f["mbits"], f["bias"], Fraction(f["max"]), f["maxcode"]
    bits = int(bits) & 0xFFFFFFFF
    s = (bits >> 31) & 1
    if (bits & 0x7FFFFFFF) > 0x7F800000:
        return (s << 7) | 0x7F
    if (bits & 0x7FFFFFFF) == 0x7F800000:
        return (s << 7) | maxcode
    a = _f32_bits_to_fraction(bits)
    if a >= fmax:
        return (s << 7) | maxcode
    min_normal = Fraction(2) ** (1 - bias)
    min_sub = Fraction(2) ** (1 - bias - M)
    if a < min_normal:
        q = _rne_int(a / min_sub)
        return (s << 7) | q
    E = _floor_log2(a)
    frac = a / Fraction(2) ** E - 1
    q = _rne_int(frac * (1 << M))
    if q == (1 << M):
        q = 0
        E += 1
    return (s << 7) | ((E + bias) << M) | q


# --------------------------------------------------------------------------
# vectorised encode (integer arithmetic on binary32 bit patterns)
# --------------------------------------------------------------------------
def encode(x, fmt):
    """Saturating RNE encode of a float32 array; returns uint8 codes.

    The same definition as ``encode_exact``, on bit patterns: write the
    magnitude as an integer significand ``sig`` times ``2^(e-23)``; the FP8
    grid spacing near it is ``2^(max(e, emin) - M)``; dividing by that spacing
    is a right shift by ``d = 23 - M + max(0, emin - e)`` bits, rounded to
    nearest even; the code is then ``((max(e, emin) + bias - 1) << M) + q``,
    which also absorbs a mantissa carry into the exponent field and gives the
    subnormal codes when ``e < emin``.
    """
    f = _fmt(fmt)
    M, bias, maxcode = f["mbits"], f["bias"], f["maxcode"]
    emin = 1 - bias
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = (u >> 31) << 7
    absu = u & 0x7FFFFFFF
    efield = absu >> 23
    man = absu & 0x7FFFFF
    is_nan = absu > 0x7F800000
    fmax_bits = int(np.array(f["max"], dtype=np.float32).view(np.uint32))
    sat = (absu >= fmax_bits) & ~is_nan

    e = np.where(efield == 0, -126, efield - 127)
    sig = np.where(efield == 0, man, man | 0x800000)
    eq = np.maximum(e, emin)
    d = 23 - M + (eq - e)
    d = np.minimum(d, 40)  # sig < 2^24, so any shift >= 25 gives 0 or a tie below 1/2
    q = sig >> d
    rem = sig - (q << d)
    half = np.int64(1) << (d - 1)
    up = (rem > half) | ((rem == half) & ((q & 1) == 1))
    q = q + up
    code = ((eq + bias - 1) << M) + q

    code = np.where(sat, maxcode, code)
    code = np.where(is_nan, 0x7F, code)
    return (sign | code).astype(np.uint8)
