"""Seeded synthetic inputs for the FP8 Linear workloads.

This module only draws random tensors; it holds none of the quantization or
GEMM arithmetic.  Both the GPU tests / bench and the CPU oracle take their
inputs from here.

Recipe (for every tensor): the tensor is cut into row chunks of
``CHUNK_ROWS`` rows; chunk c is drawn by its own numpy
``Generator(PCG64(SeedSequence(key + [c])))`` (so chunks can be drawn in
parallel threads); normal samples are drawn in binary32
(``standard_normal(dtype=float32)``), Student-t samples in fp64 and rounded to
binary32; the samples are multiplied by the tensor's standard deviation in
binary32 and, for bfloat16 tensors, rounded to bfloat16 by
round-to-nearest-even on the bit pattern.
bfloat16 tensors are returned as their uint16 bit patterns; fp32 tensors as
float32 arrays.  ``key`` is ``[workload, tensor index]`` (plus the step for
per-step tensors).

Workloads (shapes and distributions of the FP8 Linear configurations):
  tensorwise_256   X, W 256x256 fp32 ~N(0,1)
  delayed_4096     X_t 8192x4096 bf16 ~N(0,1) with 41 fixed input channels
                   (columns) multiplied by 50; W 4096x4096 ~N(0,0.02);
                   dY_t 8192x4096 ~N(0,1e-3); 64 steps
  mxfp8_4096       X 16384x4096, W 14336x4096 ~N(0,0.02); dY 16384x14336
                   ~N(0,1e-3)
  blockwise_7168   X 16384x7168, W 18432x7168 Student-t (nu=3); dY
                   16384x18432 Student-t (nu=3) x 1e-3 for the backward GEMMs
  nvfp4_4096       X 16384x4096, W 14336x4096 ~N(0,0.02); dY 16384x14336
                   ~N(0,1e-3) (the mxfp8_4096 shapes, NVFP4 operands)
  linear_4096      X 32768x4096 ~N(0,1); W 4096x4096 and W2 14336x4096
                   ~N(0,0.02); dY 32768x4096 and dY2 32768x14336 ~N(0,1e-3)
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 1024
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

WORKLOAD_IDS = {
    "tensorwise_256": 1,
    "delayed_4096": 2,
    "mxfp8_4096": 3,
    "blockwise_7168": 4,
    "linear_4096": 5,
    "nvfp4_4096": 6,
}


def generator(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even) and return the uint16
    bit patterns.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(key, shape, draw_fn, std, dtype):
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def chunk(c):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        v = draw_fn(generator(*key, c), (r1 - r0, cols)).astype(np.float32) * np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    n = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    if n <= 1:
        for c in range(n):
            chunk(c)
    else:
        with ThreadPoolExecutor(max_workers=min(n, _THREADS)) as ex:
            list(ex.map(chunk, range(n)))
    return out


def normal(key, shape, std=1.0, dtype="bf16"):
    return _draw(key, shape, lambda g, s: g.standard_normal(s, dtype=np.float32), std, dtype)


def student_t(key, shape, nu=3.0, dtype="bf16", scale=1.0):
    return _draw(key, shape, lambda g, s: g.standard_t(nu, s), scale, dtype)


def with_outlier_channels(x_bits, key, frac=0.01, factor=50.0):
    """Multiply a fixed random set of round(frac*cols) columns by ``factor``
    before the bfloat16 rounding (the x50 outlier channels of the delayed
    workload).  Takes bf16 bits that came from ``normal`` at std 1 and
    returns new bf16 bits; the columns are drawn with their own key."""
    cols = x_bits.shape[1]
    n = int(round(frac * cols))
    idx = np.sort(generator(*key).choice(cols, n, replace=False))
    x = bf16_bits_to_f32(x_bits).copy()
    x[:, idx] = (x[:, idx].astype(np.float64) * factor).astype(np.float32)
    return f32_to_bf16_bits(x), idx


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------
def tensorwise_256():
    w = WORKLOAD_IDS["tensorwise_256"]
    return {"X": normal([w, 0], (256, 256), 1.0, "f32"),
            "W": normal([w, 1], (256, 256), 1.0, "f32")}


def delayed_4096_weight(rows=4096, cols=4096):
    w = WORKLOAD_IDS["delayed_4096"]
    return normal([w, 1], (rows, cols), 0.02)


def delayed_4096_step(t, rows=8192, cols=4096, out_cols=4096):
    """X_t (with the fixed outlier channels) and dY_t of step t."""
    w = WORKLOAD_IDS["delayed_4096"]
    x = normal([w, 0, t], (rows, cols), 1.0)
    x, _ = with_outlier_channels(x, [w, 3])
    dy = normal([w, 2, t], (rows, out_cols), 1e-3)
    return {"X": x, "dY": dy}


def mxfp8_4096(m=16384, n=14336, k=4096, with_dy=True):
    w = WORKLOAD_IDS["mxfp8_4096"]
    out = {"X": normal([w, 0], (m, k), 0.02), "W": normal([w, 1], (n, k), 0.02)}
    if with_dy:
        out["dY"] = normal([w, 2], (m, n), 1e-3)
    return out


def blockwise_7168(m=16384, n=18432, k=7168, with_dy=False):
    """X and W; with_dy adds the output gradient dY [m x n] that the backward
    GEMMs (dgrad, wgrad) consume, Student-t (nu=3) times 1e-3."""
    w = WORKLOAD_IDS["blockwise_7168"]
    out = {"X": student_t([w, 0], (m, k)), "W": student_t([w, 1], (n, k))}
    if with_dy:
        out["dY"] = student_t([w, 2], (m, n), scale=1e-3)
    return out


def linear_4096(m=32768, h=4096, f=14336, which=("X", "W", "W2", "dY", "dY2")):
    w = WORKLOAD_IDS["linear_4096"]
    spec = {
        "X": ([w, 0], (m, h), 1.0),
        "W": ([w, 1], (h, h), 0.02),
        "W2": ([w, 2], (f, h), 0.02),
        "dY": ([w, 3], (m, h), 1e-3),
        "dY2": ([w, 4], (m, f), 1e-3),
    }
    return {k: normal(spec[k][0], spec[k][1], spec[k][2]) for k in which}


def nvfp4_4096(m=16384, n=14336, k=4096, with_dy=False):
    w = WORKLOAD_IDS["nvfp4_4096"]
    out = {"X": normal([w, 0], (m, k), 0.02), "W": normal([w, 1], (n, k), 0.02)}
    if with_dy:
        out["dY"] = normal([w, 2], (m, n), 1e-3)
    return out
