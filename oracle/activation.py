"""GeLU of an MLP activation whose input is stored in FP8 for the backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Benefits of Using FP8 Precision with MegaDLMs and Required Hardware"
(configuration field activation_func_fp8_input_store): the input of the MLP
activation is kept in FP8 for backpropagation instead of in bf16.  The pages
do not name the activation; the reading taken here is GeLU in its exact form,

    gelu(h)  = h * Phi(h),            Phi the standard normal CDF,
    gelu'(h) = Phi(h) + h * phi(h),   phi the standard normal density,

with Phi(h) = erfc(-h / sqrt 2) / 2 (scipy's erfc is the library primitive).

Forward: a = gelu(h) of the bf16 input (fp64, not rounded; the GPU returns
bf16), and the stored copy q = enc(fp32(h * scale)) exactly as any other
per-tensor cast.  Backward: the input is recovered from the stored bytes as
h' = fp32(dec(q) * scale_inv) (one binary32 rounding, as the GPU does), and
dh = da * gelu'(h') in fp64.
"""

import numpy as np
from scipy.special import erfc

from .fp8 import dequantize, encode

SQRT_HALF = np.sqrt(0.5)
INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def normal_cdf(h):
    return 0.5 * erfc(-np.asarray(h, dtype=np.float64) * SQRT_HALF)


def gelu(h):
    h = np.asarray(h, dtype=np.float64)
    return h * normal_cdf(h)


def gelu_grad(h):
    h = np.asarray(h, dtype=np.float64)
    return normal_cdf(h) + h * INV_SQRT_2PI * np.exp(-0.5 * h * h)


def act_fp8_store_fwd(h, scale, fmt):
    """(gelu(h) in fp64, FP8 bytes of fp32(h * scale)) for a binary32 h."""
    h32 = np.asarray(h, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        v = (h32 * np.float32(scale)).astype(np.float32)
    return gelu(h32), encode(v, fmt)


def act_fp8_store_bwd(da, q, fmt, scale_inv):
    """da * gelu'(fp32(dec(q) * scale_inv)) in fp64."""
    hq = (dequantize(q, fmt).astype(np.float32) * np.float32(scale_inv)).astype(np.float32)
    return np.asarray(da, dtype=np.float64) * gelu_grad(hq)


def elementwise_check(y, ref, gain=None, rel=2.0 ** -8, floor=2.0 ** -20):
    """Acceptance rule for the bf16 outputs of the activation (reading of the
    tolerance for an elementwise function: the bf16 rounding, at most 2^-9
    relative, plus the binary32 evaluation):

        |y - ref| <= rel * |ref| + floor * |gain| + 2^-126,

    where ``gain`` is the incoming gradient for the backward pass (the
    derivative's two terms cancel near its root, so its binary32 error is
    absolute in units of |da|) and None for the forward pass.  The last term
    covers results below the smallest normal binary32 number."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = rel * np.abs(ref) + 2.0 ** -126
    if gain is not None:
        bound = bound + floor * np.abs(np.asarray(gain, dtype=np.float64))
    err = np.abs(y - ref)
    ok = bool(np.all(err <= bound))
    worst = float(np.max(err / bound)) if err.size else 0.0
    return ok, {"worst": worst}
