"""Benchmark: the FP8 Linear hot path on one MI355X.

Headline workload (linear_4096: the 4096-hidden Linear, tensorwise current
scaling, hybrid formats): X[32768 x 4096] bf16 feeds two Linears,
W[4096 x 4096] and W2[14336 x 4096]; their output gradients are
dY[32768 x 4096] and dY2[32768 x 14336].  One step is the whole hot path:

  for X, W, W2 (E4M3) and dY, dY2 (E5M2):  amax -> scale -> cast + transpose
  fprop  Y = X W^T,  Y2 = X W2^T                 (E4M3 x E4M3)
  dgrad  dX = dY W,  dX2 = dY2 W2                (E5M2 x E4M3)
  wgrad  dW = dY^T X, dW2 = dY2^T X              (E5M2 x E4M3)

All outputs bf16.  Inputs are seeded synthetic tensors (workloads.py),
resident in HBM before timing starts.  `value` is whole-step throughput: the
step's 14.84 TFLOP of GEMM work divided by the wall-clock step time
(quantization included), over exactly --steps steps after --warmup steps.
Every call of the step is also timed with HIP events on the launch stream.

After the timed steps, every kernel call of interest is timed again "cold":
before each repetition a 1 GiB scratch buffer is read and written, which
replaces the 256 MB Infinity Cache, so no operand is served from a previous
call's cache lines.  The cold pass covers the headline calls (cast + transpose
of X and dY, the six GEMMs), the other workloads' kernels (tensorwise_256
latency, delayed_4096, mxfp8_4096, blockwise_7168, nvfp4_4096) and the fp32-master-weight,
main-gradient, bf16-wgrad and GeLU kernels, each with its fraction of the
roofline that bounds it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R]
                       [--no-cpu-baseline] [--no-workloads]
       python bench.py --references
       python bench.py --trace-summary DIR --steps K --warmup W
       python bench.py --pmc-summary DIR
Prints one JSON line on stdout.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOPS + cast-transpose GB/s (%peak), 4096-hidden Linear"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (E4M3 / E5M2 / MXFP8)
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
M, H, F = 32768, 4096, 14336
ROOFLINE_CALLS = ("fprop_W", "dgrad_W", "wgrad_W")  # the 32768 x 4096 x 4096 GEMMs
GEMM_CALLS = ("fprop_W", "fprop_W2", "dgrad_W", "dgrad_W2", "wgrad_W", "wgrad_W2")
TENSORS = ("X", "W", "W2", "dY", "dY2")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantize_scaled_gemm_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def rate(work, ms, kind):
    """(value, unit, frac) of `work` done in `ms`: kind "hbm" (bytes),
    "fp8" / "bf16" / "f16" (flops)."""
    if ms <= 0:
        return None, None, None
    if kind == "hbm":
        v = work / (ms * 1e-3) / 1e9
        return round(v, 1), "GB/s", round(v / PEAK_HBM_GBPS, 4)
    v = work / (ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if kind == "fp8" else PEAK_BF16_TFLOPS  # "bf16" / "f16": same dense peak
    return round(v, 1), "TFLOP/s", round(v / peak, 4)


def entry(work, ms_list, kind, extra=None):
    ms_list = sorted(ms_list)
    n = len(ms_list)
    med = ms_list[n // 2] if n % 2 else 0.5 * (ms_list[n // 2 - 1] + ms_list[n // 2])
    v, unit, frac = rate(work, med, kind)
    e = {"ms": round(med, 4), "p10_ms": round(ms_list[int(0.1 * (n - 1))], 4),
         "p90_ms": round(ms_list[int(round(0.9 * (n - 1)))], 4)}
    if v is not None and work > 0:
        e.update({unit: v, "frac": frac})
    if extra:
        e.update(extra)
    return e


class StepEvents:
    """HIP events around every call of the step, recorded on the launch stream
    (the current stream, which the binding passes to the library)."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def run(self, label, work, kind, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.marks.append((label, e0, e1, work, kind))

    def per_call(self, steps):
        out = {}
        for label, e0, e1, work, kind in self.marks:
            d = out.setdefault(label, {"ms": 0.0, "n": 0, "work": work, "kind": kind})
            d["ms"] += e0.elapsed_time(e1)
            d["n"] += 1
        return out


class Cold:
    """Cold per-call timing: before each repetition a 1 GiB buffer is read and
    written (replacing the Infinity Cache), then the call runs between two
    HIP events on the launch stream."""

    def __init__(self, torch, dev, reps):
        self.torch = torch
        self.reps = reps
        self.scratch = torch.zeros(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB

    def flush(self):
        self.scratch.add_(1)

    def time(self, fn, reps=None, warm=2):
        t = self.torch
        for _ in range(warm):
            fn()
        ms = []
        for _ in range(reps or self.reps):
            self.flush()
            e0 = t.cuda.Event(enable_timing=True)
            e1 = t.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ms.append((e0, e1))
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ms]


def dev_bf16(torch, bits, dev):
    import numpy as np

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


# ---------------------------------------------------------------------------
# linear_4096: the headline step
# ---------------------------------------------------------------------------
def build_step(torch, q, dev):
    import workloads

    t0 = time.time()
    host = workloads.linear_4096(M, H, F)
    log(f"[bench] generated linear_4096 inputs in {time.time() - t0:.1f}s")
    u8 = dict(dtype=torch.uint8, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    tens = {}
    for name, fmt in (("X", q.E4M3), ("W", q.E4M3), ("W2", q.E4M3), ("dY", q.E5M2), ("dY2", q.E5M2)):
        x = dev_bf16(torch, host.pop(name), dev)
        r, c = x.shape
        tens[name] = dict(x=x, fmt=fmt, q=torch.empty((r, c), **u8), qt=torch.empty((c, r), **u8),
                          amax=torch.zeros(1, device=dev), scale=torch.zeros(1, device=dev),
                          sinv=torch.zeros(1, device=dev))
    outs = dict(Y=torch.empty((M, H), **bf), Y2=torch.empty((M, F), **bf),
                dX=torch.empty((M, H), **bf), dX2=torch.empty((M, H), **bf),
                dW=torch.empty((H, H), **bf), dW2=torch.empty((F, H), **bf))
    T = q.TENSORWISE
    x, w, w2, d, d2 = (tens[k] for k in TENSORS)
    # call label -> (A, fa, sa, B, fb, sb, C)
    gemms = {
        "fprop_W": (x["q"], q.E4M3, x["sinv"], w["q"], q.E4M3, w["sinv"], outs["Y"]),
        "fprop_W2": (x["q"], q.E4M3, x["sinv"], w2["q"], q.E4M3, w2["sinv"], outs["Y2"]),
        "dgrad_W": (d["q"], q.E5M2, d["sinv"], w["qt"], q.E4M3, w["sinv"], outs["dX"]),
        "dgrad_W2": (d2["q"], q.E5M2, d2["sinv"], w2["qt"], q.E4M3, w2["sinv"], outs["dX2"]),
        "wgrad_W": (d["qt"], q.E5M2, d["sinv"], x["qt"], q.E4M3, x["sinv"], outs["dW"]),
        "wgrad_W2": (d2["qt"], q.E5M2, d2["sinv"], x["qt"], q.E4M3, x["sinv"], outs["dW2"]),
    }

    def calls_for(name):
        t = tens[name]
        r, c = t["x"].shape
        return [
            (f"amax_{name}", 2.0 * r * c, "hbm", lambda: q.qsg_amax(t["x"], t["amax"])),
            (f"scale_{name}", 0.0, "hbm",
             lambda: q.qsg_compute_scale(t["amax"], t["fmt"], 0, t["scale"], t["sinv"])),
            (f"cast_{name}", 4.0 * r * c, "hbm",
             lambda: q.qsg_cast_transpose(t["x"], t["fmt"], t["scale"], t["q"], t["qt"])),
        ]

    def gemm_call(label):
        a, fa, sa, b, fb, sb, c = gemms[label]
        work = gemm_flops(a.shape[0], b.shape[0], a.shape[1])
        return (label, work, "fp8", lambda: q.qsg_scaled_gemm(a, fa, T, sa, b, fb, T, sb, c))

    plan = []
    for n in ("X", "W", "W2"):
        plan += calls_for(n)
    plan += [gemm_call("fprop_W"), gemm_call("fprop_W2")]
    for n in ("dY", "dY2"):
        plan += calls_for(n)
    plan += [gemm_call(g) for g in ("dgrad_W", "dgrad_W2", "wgrad_W", "wgrad_W2")]

    def step(ev):
        for label, work, kind, fn in plan:
            ev.run(label, work, kind, fn)

    step_flops = 3 * (gemm_flops(M, H, H) + gemm_flops(M, F, H))
    calls = {label: (work, kind, fn) for label, work, kind, fn in plan}
    return step, step_flops, calls


# ---------------------------------------------------------------------------
# the other workloads, cold per call
# ---------------------------------------------------------------------------
def workload_tensorwise_256(torch, q, dev, cold):
    """tensorwise_256: X, W 256 x 256 fp32; amax, scale and cast + transpose of
    both, then Y = X W^T (E4M3 x E4M3, bf16 out).  Latency-bound: the whole
    pass is timed back to back (warm) and cold."""
    import workloads

    h = workloads.tensorwise_256()
    X, W = (torch.from_numpy(h[k]).to(dev) for k in ("X", "W"))
    u8 = dict(dtype=torch.uint8, device=dev)
    qx, qw = torch.empty((256, 256), **u8), torch.empty((256, 256), **u8)
    qxt, qwt = torch.empty((256, 256), **u8), torch.empty((256, 256), **u8)
    sx, sw = torch.zeros(3, device=dev), torch.zeros(3, device=dev)
    Y = torch.empty((256, 256), dtype=torch.bfloat16, device=dev)

    def run():
        q.qsg_quantize(X, q.TENSORWISE, q.E4M3, q=qx, s=sx, qt=qxt)
        q.qsg_quantize(W, q.TENSORWISE, q.E4M3, q=qw, s=sw, qt=qwt)
        q.qsg_scaled_gemm(qx, q.E4M3, q.TENSORWISE, sx[2:3], qw, q.E4M3, q.TENSORWISE, sw[2:3], Y)

    for _ in range(5):
        run()
    torch.cuda.synchronize()
    warm = []
    for _ in range(50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        warm.append((e0, e1))
    torch.cuda.synchronize()
    warm = sorted(a.elapsed_time(b) for a, b in warm)
    c = cold.time(run, reps=20)
    gemm_ms = cold.time(lambda: q.qsg_scaled_gemm(qx, q.E4M3, q.TENSORWISE, sx[2:3], qw, q.E4M3, q.TENSORWISE,
                                                  sw[2:3], Y), reps=20)
    return {"pass_latency_us_warm": round(1e3 * warm[len(warm) // 2], 1),
            "pass_latency_us_cold": round(1e3 * sorted(c)[len(c) // 2], 1),
            "launches_per_pass": 9,
            "gemm": entry(gemm_flops(256, 256, 256), gemm_ms, "fp8"),
            "note": "latency-bound (33.6 MFLOP); no roofline fraction is claimed for the pass"}


def workload_delayed_4096(torch, q, dev, cold):
    """delayed_4096: one step of delayed scaling (history 1024, max, margin 0)
    for X, W (E4M3) and dY (E5M2): cast + transpose, amax and history update
    in one launch per tensor, then fprop, dgrad and wgrad 8192 x 4096 x 4096."""
    import workloads

    st = workloads.delayed_4096_step(1)
    X, dY = dev_bf16(torch, st["X"], dev), dev_bf16(torch, st["dY"], dev)
    W = dev_bf16(torch, workloads.delayed_4096_weight(), dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    b = {}
    for n, t, f in (("X", X, q.E4M3), ("W", W, q.E4M3), ("dY", dY, q.E5M2)):
        r, c = t.shape
        b[n] = dict(x=t, f=f, q=torch.empty((r, c), **u8), qt=torch.empty((c, r), **u8),
                    amax=torch.zeros(1, device=dev), scale=torch.ones(1, device=dev),
                    sinv=torch.ones(1, device=dev), hist=torch.zeros(1024, device=dev))
    out = {}
    ws = torch.zeros(q.DELAYED_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev)
    for n in ("X", "W", "dY"):
        # one launch: cast + transpose with the scale in force, amax, history
        # update and the next scale
        t = b[n]
        r, c = t["x"].shape
        out[f"step_{n}"] = entry(4.0 * r * c, cold.time(
            lambda t=t: q.qsg_cast_transpose_delayed(t["x"], t["f"], 0, t["hist"], 1, t["scale"], t["sinv"],
                                                     t["q"], t["qt"], t["amax"], ws)), "hbm")
    # the same step as two calls (cast + transpose with fused amax, then the
    # history update): three launches
    t = b["X"]
    r, c = t["x"].shape
    out["step_X_two_calls"] = entry(4.0 * r * c, cold.time(
        lambda: (q.qsg_cast_transpose(t["x"], t["f"], t["scale"], t["q"], t["qt"], t["amax"]),
                 q.qsg_amax_update(t["hist"], 1, t["amax"], t["f"], 0, t["scale"], t["sinv"]))), "hbm")
    x, w, dy = b["X"], b["W"], b["dY"]
    R, C = X.shape
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, dX, dW = torch.empty((R, C), **bf), torch.empty((R, C), **bf), torch.empty((C, C), **bf)
    D = q.DELAYED
    g = {"fprop": (x["q"], q.E4M3, x["sinv"], w["q"], q.E4M3, w["sinv"], Y),
         "dgrad": (dy["q"], q.E5M2, dy["sinv"], w["qt"], q.E4M3, w["sinv"], dX),
         "wgrad": (dy["qt"], q.E5M2, dy["sinv"], x["qt"], q.E4M3, x["sinv"], dW)}
    for k, (a, fa, sa, bb, fb, sb, c) in g.items():
        out[k] = entry(gemm_flops(a.shape[0], bb.shape[0], a.shape[1]),
                       cold.time(lambda a=a, fa=fa, sa=sa, bb=bb, fb=fb, sb=sb, c=c:
                                 q.qsg_scaled_gemm(a, fa, D, sa, bb, fb, D, sb, c)), "fp8")
    return out


def workload_mxfp8_4096(torch, q, dev, cold):
    """mxfp8_4096: row + column MXFP8 quantization of X [16384 x 4096],
    W [14336 x 4096] and dY [16384 x 14336]; MX fprop, dgrad and wgrad."""
    import workloads

    h = workloads.mxfp8_4096()
    u8 = dict(dtype=torch.uint8, device=dev)
    mx = {}
    for n in ("X", "W", "dY"):
        t = dev_bf16(torch, h.pop(n), dev)
        r, c = t.shape
        mx[n] = dict(x=t, q=torch.empty((r, c), **u8), s=torch.empty((r, c // 32), **u8),
                     qt=torch.empty((c, r), **u8), st=torch.empty((c, r // 32), **u8))
    out = {}
    for n in ("X", "W", "dY"):
        b = mx[n]
        out[f"quantize_{n}"] = entry((4.0 + 2.0 / 32) * b["x"].numel(), cold.time(
            lambda b=b: q.qsg_quantize(b["x"], q.MXFP8, q.E4M3, q=b["q"], s=b["s"], qt=b["qt"], st=b["st"])),
            "hbm")
    x, w, dy = mx["X"], mx["W"], mx["dY"]
    Mx, K = x["x"].shape
    N = w["x"].shape[0]
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, dX, dW = torch.empty((Mx, N), **bf), torch.empty((Mx, K), **bf), torch.empty((N, K), **bf)
    X_ = q.MXFP8
    g = {"fprop": (x["q"], x["s"], w["q"], w["s"], Y),
         "dgrad": (dy["q"], dy["s"], w["qt"], w["st"], dX),
         "wgrad": (dy["qt"], dy["st"], x["qt"], x["st"], dW)}
    for k, (a, sa, bb, sb, c) in g.items():
        out[k] = entry(gemm_flops(a.shape[0], bb.shape[0], a.shape[1]),
                       cold.time(lambda a=a, sa=sa, bb=bb, sb=sb, c=c:
                                 q.qsg_scaled_gemm(a, q.E4M3, X_, sa, bb, q.E4M3, X_, sb, c)), "fp8")
    return out


def workload_blockwise_7168(torch, q, dev, cold):
    """blockwise_7168: X [16384 x 7168] and dY [16384 x 18432] 1x128 (row +
    column copies), W [18432 x 7168] 128x128; blockwise fprop, dgrad (1x128 x
    transposed 128x128) and wgrad (1x128 x 1x128 along the tokens)."""
    import workloads

    h = workloads.blockwise_7168(with_dy=True)
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    X, W, dY = (dev_bf16(torch, h.pop(k), dev) for k in ("X", "W", "dY"))
    Mx, K = X.shape
    N = W.shape[0]

    def act_bufs(t):
        r, c = t.shape
        return dict(q=torch.empty((r, c), **u8), s=torch.empty((r, c // 128), **f32),
                    qt=torch.empty((c, r), **u8), st=torch.empty((c, r // 128), **f32))

    qx, qy = act_bufs(X), act_bufs(dY)
    qw = dict(q=torch.empty((N, K), **u8), s=torch.empty((N // 128, K // 128), **f32),
              qt=torch.empty((K, N), **u8), st=torch.empty((K // 128, N // 128), **f32))
    out = {}
    for n, t, bufs in (("X", X, qx), ("dY", dY, qy)):
        out[f"quantize_{n}"] = entry((4.0 + 8.0 / 128) * t.numel(), cold.time(
            lambda t=t, bufs=bufs: q.qsg_quantize(t, q.BLOCK_1X128, q.E4M3, **bufs)), "hbm")
    out["quantize_W"] = entry((4.0 + 8.0 / 16384) * W.numel(), cold.time(
        lambda: q.qsg_quantize(W, q.BLOCK_128X128, q.E4M3, **qw)), "hbm")
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, dX, dW = torch.empty((Mx, N), **bf), torch.empty((Mx, K), **bf), torch.empty((N, K), **bf)
    B1, B128 = q.BLOCK_1X128, q.BLOCK_128X128
    g = {"fprop": (qx["q"], qx["s"], qw["q"], B128, qw["s"], Y),
         "dgrad": (qy["q"], qy["s"], qw["qt"], B128, qw["st"], dX),
         "wgrad": (qy["qt"], qy["st"], qx["qt"], B1, qx["st"], dW)}
    for k, (a, sa, bb, kb, sb, c) in g.items():
        out[k] = entry(gemm_flops(a.shape[0], bb.shape[0], a.shape[1]),
                       cold.time(lambda a=a, sa=sa, bb=bb, kb=kb, sb=sb, c=c:
                                 q.qsg_scaled_gemm(a, q.E4M3, B1, sa, bb, q.E4M3, kb, sb, c), reps=5), "fp8")
    return out


def workload_nvfp4_4096(torch, q, dev, cold):
    """nvfp4_4096: NVFP4 row + column copies of X [16384 x 4096], W [14336 x
    4096] and dY [16384 x 14336] (2 B in, 2 x (1/2 + 1/16) B out per element;
    the amax pass that precedes the quantization reads the input a second
    time and is not counted as algorithmic traffic), and the NVFP4 fprop,
    dgrad and wgrad (exactly decoded f16 operands: the f16 MFMA peak)."""
    import workloads

    h = workloads.nvfp4_4096(with_dy=True)
    u8 = dict(dtype=torch.uint8, device=dev)
    nv = {}
    for n in ("X", "W", "dY"):
        t = dev_bf16(torch, h.pop(n), dev)
        r, c = t.shape
        nv[n] = dict(x=t, ts=torch.empty(3, device=dev), q=torch.empty((r, c // 2), **u8),
                     s=torch.empty((r, c // 16), **u8), qt=torch.empty((c, r // 2), **u8),
                     st=torch.empty((c, r // 16), **u8))
    out = {}
    for n in ("X", "W", "dY"):
        b = nv[n]
        out[f"quantize_{n}"] = entry((2.0 + 2 * (0.5 + 1.0 / 16)) * b["x"].numel(), cold.time(
            lambda b=b: q.qsg_quantize_nvfp4(b["x"], b["ts"], b["q"], b["s"], b["qt"], b["st"])), "hbm")
    x, w, dy = nv["X"], nv["W"], nv["dY"]
    Mx, K = x["x"].shape
    N = w["x"].shape[0]
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, dX, dW = torch.empty((Mx, N), **bf), torch.empty((Mx, K), **bf), torch.empty((N, K), **bf)
    g = {"fprop": (x["q"], x["s"], x["ts"], w["q"], w["s"], w["ts"], Y),
         "dgrad": (dy["q"], dy["s"], dy["ts"], w["qt"], w["st"], w["ts"], dX),
         "wgrad": (dy["qt"], dy["st"], dy["ts"], x["qt"], x["st"], x["ts"], dW)}
    for k, (a, sa, ta, bb, sb, tb, c) in g.items():
        out[k] = entry(gemm_flops(a.shape[0], bb.shape[0], 2 * a.shape[1]),
                       cold.time(lambda a=a, sa=sa, ta=ta, bb=bb, sb=sb, tb=tb, c=c:
                                 q.qsg_gemm_nvfp4(a, sa, ta, bb, sb, tb, c), reps=5), "f16")
    return out


def workload_extras(torch, q, dev, cold):
    """The rows beyond the four recipes: fp32 master weights -> FP8, the FP8
    wgrad accumulated into an fp32 main gradient, the wgrad kept in bf16, and
    GeLU with its input stored in FP8."""
    import numpy as np

    import workloads

    u8 = dict(dtype=torch.uint8, device=dev)
    out = {}
    # fp32 master weights W2 14336 x 4096: tensorwise (amax 4 B + cast 4 + 1 + 1
    # B per element) and MXFP8 (4 + 1 + 1 + 2/32 B per element)
    Wm = torch.from_numpy(workloads.normal([70, 0], (F, H), 0.02, "f32")).to(dev)
    wq, wqt = torch.empty((F, H), **u8), torch.empty((H, F), **u8)
    ws = torch.zeros(3, device=dev)
    ws_mx, wst_mx = torch.empty((F, H // 32), **u8), torch.empty((H, F // 32), **u8)
    out["master_fp32_tensorwise_W2"] = entry(10.0 * Wm.numel(), cold.time(
        lambda: q.qsg_quantize(Wm, q.TENSORWISE, q.E4M3, q=wq, s=ws, qt=wqt)), "hbm")
    out["master_fp32_mxfp8_W2"] = entry((6.0 + 2.0 / 32) * Wm.numel(), cold.time(
        lambda: q.qsg_quantize(Wm, q.MXFP8, q.E4M3, q=wq, s=ws_mx, qt=wqt, st=wst_mx)), "hbm")
    del Wm, wq, wqt, ws_mx, wst_mx
    # wgrad dW [4096 x 4096] over 32768 tokens into an fp32 main gradient
    Tk = M
    a_t = torch.randint(0, 0x7B, (H, Tk), dtype=torch.uint8, device=dev)  # finite E5M2 codes
    b_t = torch.randint(0, 0x7E, (H, Tk), dtype=torch.uint8, device=dev)  # finite E4M3 codes
    one = torch.ones(1, device=dev)
    main_grad = torch.zeros((H, H), device=dev)
    T = q.TENSORWISE
    out["wgrad_fp8_accumulate_fp32_W"] = entry(gemm_flops(H, H, Tk), cold.time(
        lambda: q.qsg_scaled_gemm_accumulate(a_t, q.E5M2, T, one, b_t, q.E4M3, T, one, main_grad)), "fp8")
    del a_t, b_t, main_grad
    # wgrad kept in bf16 (--fp8-wgrad False)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    dyb = torch.randn((Tk, H), device=dev, generator=g).mul_(1e-3).to(torch.bfloat16)
    xb = torch.randn((Tk, H), device=dev, generator=g).to(torch.bfloat16)
    dw_bf = torch.empty((H, H), dtype=torch.bfloat16, device=dev)
    mg = torch.zeros((H, H), device=dev)
    out["wgrad_bf16_W"] = entry(gemm_flops(H, H, Tk), cold.time(lambda: q.qsg_wgrad_bf16(dyb, xb, dw_bf)), "bf16")
    out["wgrad_bf16_accumulate_fp32_W"] = entry(gemm_flops(H, H, Tk), cold.time(
        lambda: q.qsg_wgrad_bf16(dyb, xb, mg, accumulate=True)), "bf16")
    del dyb, xb, dw_bf, mg
    # GeLU with its input stored in FP8: h = the FC1 output [32768 x 14336]
    # (~N(0, 1.28)); forward 2 + 2 + 1 B/elt, backward 2 + 1 + 2 B/elt
    h = dev_bf16(torch, workloads.normal([90, 9], (M, F), 1.28), dev)
    da = dev_bf16(torch, workloads.normal([90, 10], (M, F), 1e-3), dev)
    act = torch.empty_like(h)
    hq = torch.empty((M, F), **u8)
    dh = torch.empty_like(h)
    sc = torch.full((1,), 448.0 / 8.0, device=dev)
    si = 1.0 / sc
    out["gelu_fp8_store_fwd"] = entry(5.0 * h.numel(), cold.time(
        lambda: q.qsg_act_fp8_store_fwd(h, q.E4M3, sc, act, hq)), "hbm")
    out["gelu_fp8_store_bwd"] = entry(5.0 * h.numel(), cold.time(
        lambda: q.qsg_act_fp8_store_bwd(da, q.E4M3, hq, si, dh)), "hbm")
    del np
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample
# ---------------------------------------------------------------------------
def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(step_flops, step_elems):
    """The oracle, untuned, on a bounded sample of the step, scaled to the
    step's TFLOP/s."""
    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = 1

    # quantization sample: amax + scale + cast + transpose of X, W, W2 and dY
    host = workloads.linear_4096(M, H, F, which=("X", "W", "W2", "dY"))
    ts = {k: workloads.bf16_bits_to_f32(host[k]) for k in ("X", "W", "W2", "dY")}
    del host
    nq = sum(t.size for t in ts.values())
    t0 = time.perf_counter()
    qx, _, _, _, sxi = oracle.quantize_tensorwise(ts["X"], "e4m3")
    oracle.quantize_tensorwise(ts["W"], "e4m3")
    qw, _, _, _, swi = oracle.quantize_tensorwise(ts["W2"], "e4m3")
    oracle.quantize_tensorwise(ts["dY"], "e5m2")
    tq = time.perf_counter() - t0
    per_elem = tq / nq
    del ts

    # GEMM sample: fp64 product of the dequantized operands, all 32768 rows of
    # X against all of W2 (the larger Linear's fprop)
    t0 = time.perf_counter()
    oracle.gemm_per_tensor(qx, "e4m3", sxi, qw, "e4m3", swi)
    tg = time.perf_counter() - t0
    gemm_rate = gemm_flops(M, F, H) / tg

    step_time = per_elem * step_elems + step_flops / gemm_rate
    hi = host_info()
    return {
        "value": step_flops / step_time / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "host": hi,
        "sample": (f"tensorwise quantize of X, W, W2 and dY ({nq / 1e6:.0f}M elements, {tq:.2f}s, numpy, "
                   f"1 thread) and the fp64 fprop GEMM of X ({M} rows) against W2 ({tg:.2f}s, BLAS "
                   f"{blas_threads} threads) on {hi['cpu_model']} ({hi['affinity']} of {hi['nproc']} CPUs "
                   f"usable), extrapolated to the full step's {step_elems / 1e6:.0f}M quantized elements and "
                   f"{step_flops / 1e12:.2f} TFLOP"),
    }


# ---------------------------------------------------------------------------
# reference points (library kernels of the same byte mix or GEMM shape; not
# part of the path, for context only)
# ---------------------------------------------------------------------------
def references(torch, dev, reps):
    """Cold-timed torch / HIP-runtime / hipBLASLt calls with the byte mix of
    the cast + transpose and the GEMM shapes of linear_4096, so the fractions
    of the library's kernels can be read against what other kernels reach on
    the same box."""
    cold = Cold(torch, dev, reps)
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for name, (r, c) in (("32768x4096", (M, H)), ("32768x14336", (M, F))):
        x = torch.randn((r, c), device=dev, generator=g).to(torch.bfloat16)
        y = torch.empty_like(x)
        n = x.numel()
        out[f"copy_bf16_{name}"] = entry(4.0 * n, cold.time(lambda: y.copy_(x)), "hbm",
                                         {"what": "torch copy_, bf16 -> bf16 (2 B in, 2 B out)"})
        f8 = torch.empty((r, c), dtype=torch.float8_e4m3fn, device=dev)
        out[f"cast_fp8_{name}"] = entry(3.0 * n, cold.time(lambda: f8.copy_(x)), "hbm",
                                        {"what": "torch copy_ bf16 -> float8_e4m3fn, no scale, no transpose "
                                                 "(2 B in, 1 B out)"})
        yt = torch.empty((c, r), dtype=torch.bfloat16, device=dev)
        out[f"transpose_bf16_{name}"] = entry(4.0 * n, cold.time(lambda: yt.copy_(x.t())), "hbm",
                                              {"what": "torch copy_ of the transposed view, bf16 (2 B in, 2 B out)"})
        del x, y, f8, yt
        torch.cuda.empty_cache()
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    out["copy_1GiB_uint8"] = entry(2.0 * big.numel(), cold.time(lambda: big2.copy_(big)), "hbm",
                                   {"what": "torch copy_ of 1 GiB (the HIP runtime's device copy)"})
    del big, big2
    torch.cuda.empty_cache()
    # hipBLASLt FP8 GEMM through torch._scaled_mm (bf16 out, per-tensor scales)
    one = torch.ones((), device=dev)
    shapes = {"fprop_W": (M, H, H), "fprop_W2": (M, F, H), "dgrad_W2": (M, H, F), "wgrad_W": (H, H, M)}
    for label, (m, n, k) in shapes.items():
        try:
            a = torch.randint(0, 0x7E, (m, k), dtype=torch.uint8, device=dev, generator=g).view(torch.float8_e4m3fn)
            b = torch.randint(0, 0x7E, (n, k), dtype=torch.uint8, device=dev, generator=g).view(torch.float8_e4m3fn)
            fn = lambda a=a, b=b: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            out[f"hipblaslt_fp8_{label}"] = entry(gemm_flops(m, n, k), cold.time(fn, reps=5), "fp8",
                                                  {"what": f"torch._scaled_mm E4M3 x E4M3 -> bf16, {m}x{n}x{k}"})
            del a, b
        except Exception as e:  # not every torch build exposes it
            out[f"hipblaslt_fp8_{label}"] = {"error": f"{type(e).__name__}: {e}"[:200]}
        torch.cuda.empty_cache()
    # bf16 wgrad dW = dY^T X over 32768 tokens (hipBLASLt through torch.matmul)
    dy = torch.randn((M, H), device=dev, generator=g).to(torch.bfloat16)
    xb = torch.randn((M, H), device=dev, generator=g).to(torch.bfloat16)
    dyt = dy.t().contiguous()
    out["hipblaslt_bf16_wgrad_W"] = entry(gemm_flops(H, H, M), cold.time(lambda: torch.matmul(dyt, xb), reps=5),
                                          "bf16", {"what": "torch.matmul(dY^T (contiguous), X), bf16, 4096x4096x32768"})
    del dy, xb, dyt, cold
    torch.cuda.empty_cache()
    out["protocol"] = (f"1 GiB read+write flush before each repetition; median of {reps} repetitions "
                       f"(GEMMs 5), HIP events on the launch stream")
    return out


# ---------------------------------------------------------------------------
# rocprofv3 summaries (run on the profiler's output, no GPU needed)
# ---------------------------------------------------------------------------
def _read_csvs(pattern):
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def trace_summary(d, steps, warmup):
    """Per-call kernel durations of the step from a rocprofv3 --kernel-trace
    CSV of `bench.py --steps K --warmup W ...`: the step's GEMM launches of
    the 256 x 256 tile instantiations come in the order GEMM_CALLS (wgrad W2
    adds one 256 x 128 tail launch), its cast + transpose launches in the order
    TENSORS; the first (K + W) steps' launches are the step's, later ones
    belong to the cold pass."""
    rows = _read_csvs(os.path.join(d, "**", "*kernel_trace.csv"))
    assert rows, f"no kernel_trace.csv under {d}"
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    n = steps + warmup
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
    g4 = [r for r in rows if re.search(r"gemm_fast_kernel<0, [01], 0, true, 4>", r["Kernel_Name"])]
    tiles = [r for r in rows if "tile_kernel<unsigned short, 0," in r["Kernel_Name"]]
    tails = [r for r in rows if re.search(r"gemm_fast_kernel<0, 1, 0, true, 2>", r["Kernel_Name"])]
    out = {}
    for i, label in enumerate(GEMM_CALLS):
        seq = [dur(r) for r in g4[i:6 * n:6]][warmup:]
        if label == "wgrad_W2" and len(tails) >= n:  # its 256 x 128 tail launch, one per step
            seq = [a + dur(r) for a, r in zip(seq, tails[warmup:n])]
        out[label] = seq
    for i, t in enumerate(TENSORS):
        out["cast_" + t] = [dur(r) for r in tiles[i:5 * n:5]][warmup:]
    res = {}
    for label, seq in out.items():
        res[label] = {"launches": len(seq), "avg_us": round(sum(seq) / max(len(seq), 1), 1)}
    fl = {"fprop_W": gemm_flops(M, H, H), "fprop_W2": gemm_flops(M, F, H), "dgrad_W": gemm_flops(M, H, H),
          "dgrad_W2": gemm_flops(M, H, F), "wgrad_W": gemm_flops(H, H, M), "wgrad_W2": gemm_flops(F, H, M)}
    for label in GEMM_CALLS:
        res[label]["TFLOP/s"] = round(fl[label] / (res[label]["avg_us"] * 1e-6) / 1e12, 1)
    tot_us = sum(res[c]["avg_us"] for c in ROOFLINE_CALLS)
    res["roofline_c5_W"] = {"avg_us_per_gemm": round(tot_us / 3, 1),
                            "TFLOP/s": round(3 * gemm_flops(M, H, H) / (tot_us * 1e-6) / 1e12, 1)}
    sizes = {"X": M * H, "W": H * H, "W2": F * H, "dY": M * H, "dY2": M * F}
    for t in TENSORS:
        res["cast_" + t]["GB/s"] = round(4.0 * sizes[t] / (res["cast_" + t]["avg_us"] * 1e-6) / 1e9, 1)
    return res


def pmc_summary(d):
    """FETCH_SIZE / WRITE_SIZE of the c5-W GEMMs from two rocprofv3 --pmc runs
    (directories pmc_FETCH_SIZE and pmc_WRITE_SIZE under d) of
    `bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-workloads --copy-calibration`,
    scaled by what the counters read for the runtime's 1 GiB device copy."""
    def load(counter):
        rows = _read_csvs(os.path.join(d, f"pmc_{counter}", "**", "*counter_collection.csv"))
        per = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            k = int(r["Dispatch_Id"])
            per.setdefault(k, [r["Kernel_Name"], 0.0])
            per[k][1] += float(r["Counter_Value"])
        return [(k, per[k][0], per[k][1]) for k in sorted(per)]

    fetch, write = load("FETCH_SIZE"), load("WRITE_SIZE")
    copies_f = [x for x in fetch if "copyBuffer" in x[1]]
    copies_w = [x for x in write if "copyBuffer" in x[1]]
    ffac = (1 << 30) / (copies_f[-1][2] * 1024.0)
    wfac = (1 << 30) / (copies_w[-1][2] * 1024.0)
    pat = r"gemm_fast_kernel<0, [01], 0, true, 4>"
    gf = [x for x in fetch if re.search(pat, x[1])]
    gw = [x for x in write if re.search(pat, x[1])]
    res = {"fetch_factor": round(ffac, 4), "write_factor": round(wfac, 4), "calls": {}}
    for i, label in enumerate(GEMM_CALLS):
        fb = gf[i][2] * 1024.0 * ffac
        wb = gw[i][2] * 1024.0 * wfac
        res["calls"][label] = {"fetch_bytes": fb, "write_bytes": wb}
    per = [res["calls"][c]["fetch_bytes"] + res["calls"][c]["write_bytes"] for c in ROOFLINE_CALLS]
    res["roofline_c5_W"] = {"bytes_per_launch": sum(per) / len(per), "source_hash": source_hash("gemm_fast.hip")}
    return res


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=10, help="cold repetitions per kernel call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the cold pass (headline calls and the other workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--references", action="store_true",
                    help="only time reference kernels (torch copies and casts, hipBLASLt GEMMs) and print them")
    ap.add_argument("--trace-summary", metavar="DIR", help="summarise a rocprofv3 kernel trace of this bench")
    ap.add_argument("--pmc-summary", metavar="DIR", help="summarise FETCH_SIZE / WRITE_SIZE counter runs")
    args = ap.parse_args()

    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.steps, args.warmup), indent=1))
        return
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary), indent=1))
        return
    if args.gpus != 1:
        log(f"bench.py measures one GPU only: the FP8 Linear hot path here is the single-GPU "
            f"kernel work; --gpus {args.gpus} is not supported (run with --gpus 1).")
        sys.exit(2)

    import torch

    import quantize_scaled_gemm_amd as q

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.load_library()

    if args.references:
        print(json.dumps(references(torch, dev, args.reps)), flush=True)
        return

    step, step_flops, calls = build_step(torch, q, dev)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step(StepEvents(torch))
    torch.cuda.synchronize()

    ev = StepEvents(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    pc = ev.per_call(args.steps)
    in_step = {}
    for label, d in pc.items():
        avg = d["ms"] / d["n"]
        e = {"avg_ms": round(avg, 4)}
        if d["work"] > 0:
            v, unit, frac = rate(d["work"], avg, d["kind"])
            e.update({unit: v, "frac": frac})
        in_step[label] = e
    roof_ms = sum(pc[c]["ms"] / pc[c]["n"] for c in ROOFLINE_CALLS)
    roof_flops = sum(pc[c]["work"] for c in ROOFLINE_CALLS)
    achieved = roof_flops / (roof_ms * 1e-3) / 1e12
    gemm_ms = sum(pc[c]["ms"] / pc[c]["n"] for c in GEMM_CALLS)
    ct_ms = sum(pc["cast_" + t]["ms"] / pc["cast_" + t]["n"] for t in ("X", "dY"))
    ct_gbps = 4.0 * 2 * M * H / (ct_ms * 1e-3) / 1e9

    traffic = None
    prof_path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(prof_path):
        with open(prof_path) as fh:
            tr = json.load(fh).get("roofline_c5_W")
        if tr and tr.get("source_hash") == source_hash("gemm_fast.hip"):
            traffic = tr.get("bytes_per_launch")

    line = {
        "metric": METRIC,
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "linear_4096: tensorwise hybrid FP8 Linear fwd+bwd, X 32768x4096, "
                               "W 4096x4096, W2 14336x4096, bf16 in/out",
                   "tokens": M, "hidden": H, "ffn": F, "recipe": "tensorwise",
                   "formats": "E4M3 X/W, E5M2 dY"},
        "roofline": {"bound": "mfma", "kernel": "gemm_fast_kernel: fprop, dgrad, wgrad 32768x4096x4096 (in-step)",
                     "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic},
        "gemm_tflops_in_step": round(step_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "cast_transpose_gbps_in_step": round(ct_gbps, 1),
        "cast_transpose_frac_in_step": round(ct_gbps / PEAK_HBM_GBPS, 4),
        "in_step": in_step,
    }

    if not args.no_workloads:
        t1 = time.time()
        cold = Cold(torch, dev, args.reps)
        c5 = {}
        for label in ("cast_X", "cast_dY", "cast_dY2", "amax_X") + GEMM_CALLS:
            work, kind, fn = calls[label]
            c5[label] = entry(work, cold.time(fn, reps=5 if label in GEMM_CALLS else args.reps), kind)
        rms = [c5[c]["ms"] for c in ROOFLINE_CALLS]
        v, unit, frac = rate(roof_flops, sum(rms), "fp8")
        c5["c5_W_gemms"] = {unit: v, "frac": frac}
        ct = sum(c5[c]["ms"] for c in ("cast_X", "cast_dY"))
        v, unit, frac = rate(2 * 4.0 * M * H, ct, "hbm")
        c5["cast_X_dY"] = {unit: v, "frac": frac}
        line["cold"] = {"linear_4096": c5}
        del step, calls
        torch.cuda.empty_cache()
        for name, fn in (("tensorwise_256", workload_tensorwise_256), ("delayed_4096", workload_delayed_4096),
                         ("mxfp8_4096", workload_mxfp8_4096), ("blockwise_7168", workload_blockwise_7168),
                         ("nvfp4_4096", workload_nvfp4_4096), ("extras", workload_extras)):
            t2 = time.time()
            line["cold"][name] = fn(torch, q, dev, cold)
            torch.cuda.empty_cache()
            log(f"[bench] {name} done in {time.time() - t2:.1f}s")
        line["cold"]["protocol"] = (f"1 GiB read+write flush before each repetition; median of {args.reps} "
                                    f"repetitions (GEMMs 5), HIP events on the launch stream")
        del cold
        log(f"[bench] cold pass took {time.time() - t1:.1f}s")
    if not args.no_cpu_baseline:
        t0 = time.time()
        step_elems = M * H + H * H + F * H + M * H + M * F
        line["cpu_baseline"] = cpu_baseline(step_flops, step_elems)
        log(f"[bench] cpu baseline took {time.time() - t0:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
