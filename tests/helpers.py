"""Shared helpers of the test suite (marshalling between numpy and torch)."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lib_is_stale():
    pkg = os.path.join(ROOT, "quantize_scaled_gemm_amd")
    lib = os.path.join(pkg, "libqsg.so")
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))]
    srcs.append(os.path.join(ROOT, "include", "qsg.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


def build_library():
    subprocess.run([sys.executable, "-m", "quantize_scaled_gemm_amd.build"], cwd=ROOT, check=True)


def to_dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> bfloat16 tensor on the GPU."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    """GPU tensor -> numpy (bf16 as float32, uint8 as uint8)."""
    import torch

    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne_f64(y):
    """Round values to bfloat16 with torch's CPU cast (RNE), returned as float64."""
    import torch

    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
