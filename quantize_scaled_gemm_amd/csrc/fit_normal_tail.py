"""Fit of the normal tail used by act.hip (GeLU with an FP8-stored input).

For a >= 0 the upper normal tail is  E(a) = Q(a) = 1 - Phi(a) = exp(-a^2/2) R(a)
with R(a) = erfcx(a / sqrt 2) / 2 (erfcx(x) = exp(x^2) erfc(x), smooth and
positive).  R is approximated as  R(a) ~= t P(t),  t = 1 / (1 + p a),  P a
polynomial of degree 7, by least squares on the relative error over
a in [0, 14] (beyond 14, exp(-a^2/2) is below the binary32 range).  The
printed coefficients are those in act.hip; the script also reports the
maximum relative error of R in fp64 and of a binary32 Horner evaluation.

Run: python quantize_scaled_gemm_amd/csrc/fit_normal_tail.py
"""

import numpy as np
from scipy.special import erfcx

P_SCALE = 0.3
DEGREE = 7


def fit():
    a = np.concatenate([np.linspace(0, 2, 20001), np.linspace(2, 14, 60001)])
    R = 0.5 * erfcx(a / np.sqrt(2.0))
    t = 1.0 / (1.0 + P_SCALE * a)
    V = np.vander(t, DEGREE + 1, increasing=True) * t[:, None]
    w = 1.0 / R
    c, *_ = np.linalg.lstsq(V * w[:, None], R * w, rcond=None)
    rel64 = np.max(np.abs(V @ c - R) / R)
    c32 = c.astype(np.float32)
    a32 = a.astype(np.float32)
    t32 = (np.float32(1) / (np.float32(1) + np.float32(P_SCALE) * a32)).astype(np.float32)
    acc = np.full_like(t32, c32[-1])
    for k in range(DEGREE - 1, -1, -1):
        acc = (acc * t32 + c32[k]).astype(np.float32)
    r32 = (acc * t32).astype(np.float32)
    rel32 = np.max(np.abs(r32.astype(np.float64) - R) / R)
    return c32, rel64, rel32


if __name__ == "__main__":
    c32, rel64, rel32 = fit()
    print(f"max relative error of R: fp64 fit {rel64:.2e}, binary32 Horner {rel32:.2e}")
    print("coefficients c0..c%d (float32):" % DEGREE)
    for k, v in enumerate(c32):
        print(f"  c{k} = {float(v)!r}f")
