"""The GeLU kernels (act.hip) evaluate the normal tail with coefficients fitted
by quantize_scaled_gemm_amd/csrc/fit_normal_tail.py: the fit must reproduce
the constants written in the kernel, and its binary32 evaluation must stay
within 1e-6 relative of erfcx (far inside the bf16 outputs' 2^-8)."""

import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantize_scaled_gemm_amd", "csrc")


def test_kernel_constants_match_the_fit():
    spec = importlib.util.spec_from_file_location("fit_normal_tail", os.path.join(CSRC, "fit_normal_tail.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    c32, rel64, rel32 = mod.fit()
    assert rel64 < 5e-7 and rel32 < 1e-6
    src = open(os.path.join(CSRC, "act.hip")).read()
    body = src[src.index("float tail_r(float a)"):src.index("return p * t;")]
    consts = [np.float32(float(v)) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # 0.3 and 1.0 of t, then c7, c6, ..., c0 in Horner order
    assert consts[0] == np.float32(0.3) and consts[1] == np.float32(1.0)
    assert consts[2:] == list(c32[::-1])
