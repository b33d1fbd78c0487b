"""Scaling recipes: amax, per-tensor scale, amax history, MXFP8, blockwise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every function takes plain numpy arrays (float32 for real data; bfloat16 data
is first widened to float32, which is exact) and returns numpy arrays.  The
quantized value fed to the encoder is always the binary32 product
``fp32(x * scale)``: one IEEE round-to-nearest-even multiply, then the FP8
encode.  That double rounding is part of the definition, because the GPU
forms the same binary32 product before converting.

Readings taken where the pages are silent (each is also listed in the
design notes):
  R1  scale = fp32(fmax / amax), then times 2^-margin; scale_inv =
      fp32(1 / scale).  ("Low-Precision Training Guide", table "Numerical
      Stability Knobs": the margin adds M bits of headroom to the scaling
      factor.)
  R2  amax == 0 or amax not finite gives scale = 1; a quotient that overflows
      to infinity (a tiny amax) gives the largest finite binary32.
  R3  delayed scaling starts from an all-zero history and scale 1; step t
      quantizes with scale_t, records amax of the raw tensor in slot
      t mod L, and the next scale comes from max(history); if that max is 0
      or not finite the previous scale and scale_inv are kept.
  R4  mxfp8: the block exponent is the smallest power of two that keeps the
      block's amax at or below the format maximum (no element saturates);
      the OCP Microscaling v1.0 rule (floor) is selectable.  Margin is added
      to the exponent.  The exponent is clamped to [-127, 127] and stored as
      the E8M0 byte e + 127; an all-zero block stores 127.
  R5  blockwise: per block, the R1/R2 scale with fmax of the chosen format;
      the scale tensor holds the fp32 scale_inv (what the GEMM multiplies
      by); the scales are not rounded to powers of two.
  R6  the column-wise copy of an activation uses 1 x B blocks along the other
      dimension of the tensor (128 x 1 for blockwise, 32 x 1 for mxfp8), and
      is stored transposed, so that the backward GEMM reads it K-contiguous.
"""

import numpy as np

from .fp8 import FORMATS, encode

_FLT_MAX = np.float32(np.finfo(np.float32).max)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


# --------------------------------------------------------------------------
# amax and the per-tensor scale
# --------------------------------------------------------------------------
def amax(x):
    """max |x| as float32 ("Low-Precision Training Guide", recipe
    "tensorwise": the scale comes from the current tensor).

    -0 counts as 0.  Any NaN makes the result NaN.  An empty tensor gives 0.
    """
    x = _f32(x)
    if x.size == 0:
        return np.float32(0.0)
    if np.isnan(x).any():
        return np.float32(np.nan)
    return np.float32(np.max(np.abs(x)))


def tensorwise_scale(a, fmt, margin=0):
    """(scale, scale_inv) from an amax, readings R1 and R2.

    ("Low-Precision Training Guide": recipe "tensorwise" and the knob
    ``--fp8-margin``.)
    """
    fmax = np.float32(FORMATS[fmt]["max"])
    a = np.float32(a)
    if a == 0 or not np.isfinite(a):
        scale = np.float32(1.0)
    else:
        with np.errstate(over="ignore", divide="ignore"):
            scale = np.float32(fmax / a)
        if np.isinf(scale):
            scale = _FLT_MAX
        scale = np.float32(scale * np.float32(2.0 ** -margin))
    scale_inv = np.float32(np.float32(1.0) / scale)
    return scale, scale_inv


def cast_transpose(x, scale, fmt):
    """Q = enc(fp32(x*scale)) and QT = Q transposed, both uint8.

    ("How to reduce cuda memory usage of fp8?": the backward pass of a Linear
    reads a transposed FP8 copy of its input.)
    """
    x = _f32(x)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (x * np.float32(scale)).astype(np.float32)
    q = encode(v, fmt)
    return q, np.ascontiguousarray(q.T)


def quantize_tensorwise(x, fmt, margin=0):
    """Tensorwise current scaling of one tensor: amax, scale, cast+transpose."""
    a = amax(x)
    s, si = tensorwise_scale(a, fmt, margin)
    q, qt = cast_transpose(x, s, fmt)
    return q, qt, a, s, si


# --------------------------------------------------------------------------
# delayed scaling
# --------------------------------------------------------------------------
class DelayedState:
    """State of one tensor under delayed scaling (reading R3).

    ("Low-Precision Training Guide", recipe "delayed": the scaling factor is
    computed from a rolling amax history; ``--fp8-amax-history-len``,
    ``--fp8-amax-compute-algo max``.)
    """

    def __init__(self, hist_len, fmt, margin=0):
        if hist_len < 1:
            raise ValueError("history length must be at least 1")
        self.history = np.zeros(hist_len, dtype=np.float32)
        self.fmt = fmt
        self.margin = margin
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)

    def step(self, x, t):
        """One step: quantize x with the current scale, then update."""
        q, qt = cast_transpose(x, self.scale, self.fmt)
        a = amax(x)
        used_scale, used_inv = self.scale, self.scale_inv
        self.scale, self.scale_inv = amax_update(
            self.history, t, a, self.fmt, self.margin, self.scale, self.scale_inv)
        return q, qt, a, used_scale, used_inv


def amax_update(history, step, a, fmt, margin, prev_scale, prev_scale_inv):
    """Record amax in slot ``step mod L`` (in place) and return the next
    (scale, scale_inv): max over the window, then R1/R2, keeping the previous
    pair when the window max is 0 or not finite (R3)."""
    L = history.shape[0]
    history[step % L] = np.float32(a)
    if np.isnan(history).any():
        window_max = np.float32(np.nan)
    else:
        window_max = np.float32(np.max(history))
    if window_max == 0 or not np.isfinite(window_max):
        return np.float32(prev_scale), np.float32(prev_scale_inv)
    return tensorwise_scale(window_max, fmt, margin)


# --------------------------------------------------------------------------
# MXFP8
# --------------------------------------------------------------------------
def mx_exponent(block_amax, fmt, rule="ceil", margin=0):
    """Shared block exponent(s) e for an array of block amaxes (reading R4).

    ("Low-Precision Training Guide", recipe "mxfp8": one power-of-two scale
    per 1 x 32 block.)  Write amax = 2^E * (1 + f), 0 <= f < 1, E read from
    the binary32 exponent with subnormals normalised.  The format maximum is
    1.75 * 2^emax (emax = 8 for E4M3, 15 for E5M2), so the smallest e with
    amax * 2^-e <= fmax is E - emax, plus one when f > 0.75.  The OCP rule is
    E - emax.  Non-finite amaxes go through the same bit arithmetic (their
    exponent field reads as E = 128).  Returns int64 exponents in
    [-127, 127]; a zero amax gives 0.
    """
    emax = {"e4m3": 8, "e5m2": 15}[fmt]
    a = np.abs(np.ascontiguousarray(block_amax, dtype=np.float32))
    # finite values: a = m * 2^x with m in [0.5, 1) (frexp is exact, also for
    # binary32 subnormals); so E = x - 1 and 1 + f = 2m, i.e. f > 0.75 <=> m > 0.875
    with np.errstate(invalid="ignore"):
        m, x = np.frexp(a.astype(np.float64))
    E = x.astype(np.int64) - 1
    f_gt = m > 0.875
    # non-finite values: the exponent field reads 255, i.e. E = 128, and f is
    # taken from the 23 stored mantissa bits
    bits = a.view(np.uint32).astype(np.int64)
    nonfinite = ~np.isfinite(a)
    E = np.where(nonfinite, 128, E)
    f_gt = np.where(nonfinite, (bits & 0x7FFFFF) > 0x600000, f_gt)
    e = E - emax
    if rule == "ceil":
        e = e + f_gt
    elif rule != "ocp":
        raise ValueError(f"unknown mx rule {rule!r}")
    e = e + margin
    e = np.clip(e, -127, 127)
    e = np.where(a == 0, 0, e)
    return e.astype(np.int64)


def _pow2_f32(k):
    """2^k as float32 for integer k in [-127, 127] (exact)."""
    return np.ldexp(np.float32(1.0), np.asarray(k, dtype=np.int32)).astype(np.float32)


def _mx_rows(x, fmt, rule, margin):
    """Row-wise MX quantization: blocks of 32 consecutive columns."""
    R, C = x.shape
    xb = x.reshape(R, C // 32, 32)
    if xb.size:
        blk = np.max(np.abs(xb), axis=2)
        blk = np.where(np.isnan(xb).any(axis=2), np.float32(np.nan), blk).astype(np.float32)
    else:
        blk = np.zeros((R, C // 32), dtype=np.float32)
    e = mx_exponent(blk, fmt, rule, margin)
    mult = _pow2_f32(-e)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (xb * mult[:, :, None]).astype(np.float32)
    q = encode(v, fmt).reshape(R, C)
    return q, (e + 127).astype(np.uint8)


def mx_quantize(x, fmt="e4m3", rule="ceil", margin=0, rowwise=True, colwise=True):
    """MXFP8 row-wise and column-wise quantization of an R x C tensor.

    Row-wise: blocks of 1 x 32 along C; Q is R x C, S is R x C/32 E8M0 bytes.
    Column-wise (R6): blocks of 32 x 1 along R, stored transposed: QT is
    C x R and ST is C x R/32, i.e. exactly the row-wise quantization of x^T.
    """
    x = _f32(x)
    R, C = x.shape
    out = {}
    if rowwise:
        if C % 32:
            raise ValueError("mxfp8 row-wise needs cols % 32 == 0")
        out["q"], out["s"] = _mx_rows(x, fmt, rule, margin)
    if colwise:
        if R % 32:
            raise ValueError("mxfp8 column-wise needs rows % 32 == 0")
        out["qt"], out["st"] = _mx_rows(np.ascontiguousarray(x.T), fmt, rule, margin)
    return out


# --------------------------------------------------------------------------
# blockwise (1 x 128 activations, 128 x 128 weights)
# --------------------------------------------------------------------------
def block_scale(block_amax, fmt, margin=0):
    """Per-block (scale, scale_inv) arrays: R1/R2 applied to every block,
    element-wise (the same steps as ``tensorwise_scale``)."""
    a = np.ascontiguousarray(block_amax, dtype=np.float32)
    fmax = np.float32(FORMATS[fmt]["max"])
    degenerate = (a == 0) | ~np.isfinite(a)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = (fmax / np.where(degenerate, np.float32(1), a)).astype(np.float32)
    q = np.where(np.isinf(q), _FLT_MAX, q).astype(np.float32)
    q = (q * np.float32(2.0 ** -margin)).astype(np.float32)
    s = np.where(degenerate, np.float32(1.0), q).astype(np.float32)
    with np.errstate(divide="ignore"):
        si = (np.float32(1.0) / s).astype(np.float32)
    return s, si


def _block_amax(xb, axes):
    if xb.size == 0:
        return np.max(np.abs(xb), axis=axes, initial=0).astype(np.float32)
    m = np.max(np.abs(xb), axis=axes)
    return np.where(np.isnan(xb).any(axis=axes), np.float32(np.nan), m).astype(np.float32)


def _b1x128_rows(x, fmt, margin):
    R, C = x.shape
    xb = x.reshape(R, C // 128, 128)
    s, si = block_scale(_block_amax(xb, 2), fmt, margin)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (xb * s[:, :, None]).astype(np.float32)
    return encode(v, fmt).reshape(R, C), si


def block_quantize_1x128(x, fmt="e4m3", margin=0, rowwise=True, colwise=True):
    """Activation blockwise quantization ("Low-Precision Training Guide",
    recipe "blockwise": 1 x 128 activation blocks).

    Row-wise: 1 x 128 blocks along C; Q R x C, S R x C/128 fp32 scale_inv.
    Column-wise (R6): 128 x 1 blocks along R, stored transposed: QT C x R,
    ST C x R/128.
    """
    x = _f32(x)
    R, C = x.shape
    out = {}
    if rowwise:
        if C % 128:
            raise ValueError("1x128 row-wise needs cols % 128 == 0")
        out["q"], out["s"] = _b1x128_rows(x, fmt, margin)
    if colwise:
        if R % 128:
            raise ValueError("1x128 column-wise needs rows % 128 == 0")
        out["qt"], out["st"] = _b1x128_rows(np.ascontiguousarray(x.T), fmt, margin)
    return out


def block_quantize_128x128(w, fmt="e4m3", margin=0, transpose=True):
    """Weight blockwise quantization ("Low-Precision Training Guide", recipe
    "blockwise": 128 x 128 weight blocks).

    Q R x C, S (R/128) x (C/128) fp32 scale_inv; the transposed copy is the
    bit transpose QT = Q^T with the transposed scale grid ST = S^T.
    """
    w = _f32(w)
    R, C = w.shape
    if R % 128 or C % 128:
        raise ValueError("128x128 blocks need rows % 128 == 0 and cols % 128 == 0")
    wb = w.reshape(R // 128, 128, C // 128, 128)
    s, si = block_scale(_block_amax(wb, (1, 3)), fmt, margin)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (wb * s[:, None, :, None]).astype(np.float32)
    q = encode(v, fmt).reshape(R, C)
    out = {"q": q, "s": si}
    if transpose:
        out["qt"] = np.ascontiguousarray(q.T)
        out["st"] = np.ascontiguousarray(si.T)
    return out
