"""Benchmark: one FP8 Linear fwd+bwd step on one MI355X.

Workload (the 4096-hidden Linear, tensorwise current scaling, hybrid
formats): X[32768 x 4096] bf16 feeds two Linears, W[4096 x 4096] and
W2[14336 x 4096]; their output gradients are dY[32768 x 4096] and
dY2[32768 x 14336].  One step is the whole hot path:

  for X, W, W2 (E4M3) and dY, dY2 (E5M2):  amax -> scale -> cast + transpose
  fprop  Y = X W^T,  Y2 = X W2^T                 (E4M3 x E4M3)
  dgrad  dX = dY W,  dX2 = dY2 W2                (E5M2 x E4M3)
  wgrad  dW = dY^T X, dW2 = dY2^T X              (E5M2 x E4M3)

All outputs bf16.  Inputs are seeded synthetic tensors (workloads.py), resident
in HBM before timing starts.  `value` is whole-step throughput: the step's
14.84 TFLOP of GEMM work divided by the step time (quantization included).
Per-kernel times come from HIP events on the launch stream.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
Prints one JSON line on stdout.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOPS + cast-transpose GB/s (%peak), 4096-hidden Linear"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
M, H, F = 32768, 4096, 14336


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


class Timer:
    """HIP events recorded on the launch stream, grouped by kernel name."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []  # (name, start_event, end_event, work, work_unit)

    def run(self, name, work, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.marks.append((name, ev0, ev1, work))

    def summary(self):
        out = {}
        for name, e0, e1, work in self.marks:
            ms = e0.elapsed_time(e1)
            d = out.setdefault(name, {"launches": 0, "ms": 0.0, "work": 0.0})
            d["launches"] += 1
            d["ms"] += ms
            d["work"] += work
        return out


def build_step(torch, q, dev):
    import numpy as np

    import workloads

    t0 = time.time()
    host = workloads.linear_4096(M, H, F)
    log(f"[bench] generated inputs in {time.time() - t0:.1f}s")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W, W2, dY, dY2 = (to_dev(host[k]) for k in ("X", "W", "W2", "dY", "dY2"))
    del host
    u8 = dict(dtype=torch.uint8, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    tens = {}
    for name, x, fmt in (("X", X, q.E4M3), ("W", W, q.E4M3), ("W2", W2, q.E4M3),
                         ("dY", dY, q.E5M2), ("dY2", dY2, q.E5M2)):
        r, c = x.shape
        tens[name] = dict(x=x, fmt=fmt, q=torch.empty((r, c), **u8), qt=torch.empty((c, r), **u8),
                          amax=torch.zeros(1, device=dev), scale=torch.zeros(1, device=dev),
                          sinv=torch.zeros(1, device=dev))
    outs = dict(Y=torch.empty((M, H), **bf), Y2=torch.empty((M, F), **bf),
                dX=torch.empty((M, H), **bf), dX2=torch.empty((M, H), **bf),
                dW=torch.empty((H, H), **bf), dW2=torch.empty((F, H), **bf))

    T = q.TENSORWISE

    def quantize(timer, name):
        t = tens[name]
        r, c = t["x"].shape
        timer.run("amax", 2.0 * r * c, lambda: q.qsg_amax(t["x"], t["amax"]))
        timer.run("compute_scale", 0.0,
                  lambda: q.qsg_compute_scale(t["amax"], t["fmt"], 0, t["scale"], t["sinv"]))
        timer.run("cast_transpose", 4.0 * r * c,
                  lambda: q.qsg_cast_transpose(t["x"], t["fmt"], t["scale"], t["q"], t["qt"]))

    def gemm(timer, kname, a, fa, sa, b, fb, sb, c):
        m, k = a.shape
        n = b.shape[0]
        timer.run(kname, gemm_flops(m, n, k),
                  lambda: q.qsg_scaled_gemm(a, fa, T, sa, b, fb, T, sb, c))

    def step(timer):
        for n in ("X", "W", "W2"):
            quantize(timer, n)
        x, w, w2 = tens["X"], tens["W"], tens["W2"]
        gemm(timer, "gemm_e4m3_e4m3", x["q"], q.E4M3, x["sinv"], w["q"], q.E4M3, w["sinv"], outs["Y"])
        gemm(timer, "gemm_e4m3_e4m3", x["q"], q.E4M3, x["sinv"], w2["q"], q.E4M3, w2["sinv"], outs["Y2"])
        for n in ("dY", "dY2"):
            quantize(timer, n)
        d, d2 = tens["dY"], tens["dY2"]
        gemm(timer, "gemm_e5m2_e4m3", d["q"], q.E5M2, d["sinv"], w["qt"], q.E4M3, w["sinv"], outs["dX"])
        gemm(timer, "gemm_e5m2_e4m3", d2["q"], q.E5M2, d2["sinv"], w2["qt"], q.E4M3, w2["sinv"], outs["dX2"])
        gemm(timer, "gemm_e5m2_e4m3", d["qt"], q.E5M2, d["sinv"], x["qt"], q.E4M3, x["sinv"], outs["dW"])
        gemm(timer, "gemm_e5m2_e4m3", d2["qt"], q.E5M2, d2["sinv"], x["qt"], q.E4M3, x["sinv"], outs["dW2"])

    step_flops = 3 * (gemm_flops(M, H, H) + gemm_flops(M, F, H))
    step_elems = M * H + H * H + F * H + M * H + M * F
    return step, step_flops, step_elems


def time_fn(torch, fn, reps=10, warm=2):
    """Average milliseconds of fn() over reps, HIP events on the current stream."""
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def other_recipes(torch, q, dev):
    """Kernel throughput of the delayed, MXFP8 and blockwise workloads (the
    shapes of the parity tests), reported next to the headline step."""
    import numpy as np

    import workloads

    def d(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    u8 = dict(dtype=torch.uint8, device=dev)
    out = {}

    # delayed scaling, Linear 4096 -> 4096, 8192 tokens: one step
    st = workloads.delayed_4096_step(0)
    X, dY = d(st["X"]), d(st["dY"])
    W = d(workloads.delayed_4096_weight())
    R, C = X.shape
    bufs = {}
    for n, t, f in (("X", X, q.E4M3), ("W", W, q.E4M3), ("dY", dY, q.E5M2)):
        r, c = t.shape
        bufs[n] = dict(x=t, f=f, q=torch.empty((r, c), **u8), qt=torch.empty((c, r), **u8),
                       amax=torch.zeros(1, device=dev), scale=torch.ones(1, device=dev),
                       sinv=torch.ones(1, device=dev), hist=torch.zeros(1024, device=dev))
    Y = torch.empty((R, W.shape[0]), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    dW = torch.empty(W.shape, dtype=torch.bfloat16, device=dev)
    T = q.DELAYED

    def quant(n):
        b = bufs[n]
        q.qsg_cast_transpose(b["x"], b["f"], b["scale"], b["q"], b["qt"], b["amax"])
        q.qsg_amax_update(b["hist"], 0, b["amax"], b["f"], 0, b["scale"], b["sinv"])

    x, w, dy = bufs["X"], bufs["W"], bufs["dY"]
    ms_q = time_fn(torch, lambda: [quant(n) for n in ("X", "W", "dY")])
    ms_g = time_fn(torch, lambda: (
        q.qsg_scaled_gemm(x["q"], q.E4M3, T, x["sinv"], w["q"], q.E4M3, T, w["sinv"], Y),
        q.qsg_scaled_gemm(dy["q"], q.E5M2, T, dy["sinv"], w["qt"], q.E4M3, T, w["sinv"], dX),
        q.qsg_scaled_gemm(dy["qt"], q.E5M2, T, dy["sinv"], x["qt"], q.E4M3, T, x["sinv"], dW)))
    qbytes = 4.0 * (X.numel() + W.numel() + dY.numel())
    gfl = 3 * gemm_flops(R, W.shape[0], C)
    out["delayed_4096"] = {"quantize_ms": round(ms_q, 4), "quantize_GB/s": round(qbytes / ms_q / 1e6, 1),
                           "gemm_ms": round(ms_g, 4), "gemm_TFLOP/s": round(gfl / ms_g / 1e9, 1),
                           "step_ms": round(ms_q + ms_g, 4)}
    del bufs, X, dY, W, Y, dX, dW

    # MXFP8: X 16384x4096, W 14336x4096, dY 16384x14336
    h = workloads.mxfp8_4096()
    mx = {}
    for n in ("X", "W", "dY"):
        t = d(h[n])
        r, c = t.shape
        mx[n] = dict(x=t, q=torch.empty((r, c), **u8), s=torch.empty((r, c // 32), **u8),
                     qt=torch.empty((c, r), **u8), st=torch.empty((c, r // 32), **u8))
    del h

    def mxq(n):
        b = mx[n]
        q.qsg_quantize(b["x"], q.MXFP8, q.E4M3, q=b["q"], s=b["s"], qt=b["qt"], st=b["st"])

    ms_q = time_fn(torch, lambda: [mxq(n) for n in ("X", "W", "dY")])
    x, w, dy = mx["X"], mx["W"], mx["dY"]
    M, K = x["x"].shape
    N = w["x"].shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    X_ = q.MXFP8
    ms_f = time_fn(torch, lambda: q.qsg_scaled_gemm(x["q"], q.E4M3, X_, x["s"], w["q"], q.E4M3, X_, w["s"], Y))
    ms_d = time_fn(torch, lambda: q.qsg_scaled_gemm(dy["q"], q.E4M3, X_, dy["s"], w["qt"], q.E4M3, X_, w["st"], dX))
    ms_w = time_fn(torch, lambda: q.qsg_scaled_gemm(dy["qt"], q.E4M3, X_, dy["st"], x["qt"], q.E4M3, X_, x["st"], dW))
    qbytes = (4.0 + 2.0 / 32) * sum(mx[n]["x"].numel() for n in mx)
    gf = gemm_flops(M, N, K)
    out["mxfp8_4096"] = {"quantize_ms": round(ms_q, 4), "quantize_GB/s": round(qbytes / ms_q / 1e6, 1),
                         "fprop_TFLOP/s": round(gf / ms_f / 1e9, 1), "dgrad_TFLOP/s": round(gf / ms_d / 1e9, 1),
                         "wgrad_TFLOP/s": round(gf / ms_w / 1e9, 1),
                         "step_ms": round(ms_q + ms_f + ms_d + ms_w, 4)}
    del mx, Y, dX, dW

    # blockwise: X 16384x7168 (1x128, row + column copies), W 18432x7168 (128x128)
    h = workloads.blockwise_7168()
    X, W = d(h["X"]), d(h["W"])
    del h
    M, K = X.shape
    N = W.shape[0]
    qx = dict(q=torch.empty((M, K), **u8), s=torch.empty((M, K // 128), device=dev),
              qt=torch.empty((K, M), **u8), st=torch.empty((K, M // 128), device=dev))
    qw = dict(q=torch.empty((N, K), **u8), s=torch.empty((N // 128, K // 128), device=dev),
              qt=torch.empty((K, N), **u8), st=torch.empty((K // 128, N // 128), device=dev))
    ms_qx = time_fn(torch, lambda: q.qsg_quantize(X, q.BLOCK_1X128, q.E4M3, **qx))
    ms_qw = time_fn(torch, lambda: q.qsg_quantize(W, q.BLOCK_128X128, q.E4M3, **qw))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ms_f = time_fn(torch, lambda: q.qsg_scaled_gemm(qx["q"], q.E4M3, q.BLOCK_1X128, qx["s"], qw["q"], q.E4M3,
                                                    q.BLOCK_128X128, qw["s"], Y), reps=5)
    out["blockwise_7168"] = {"quantize_act_ms": round(ms_qx, 4),
                             "quantize_act_GB/s": round((4.0 + 8.0 / 128) * X.numel() / ms_qx / 1e6, 1),
                             "quantize_weight_ms": round(ms_qw, 4),
                             "quantize_weight_GB/s": round((4.0 + 8.0 / 16384) * W.numel() / ms_qw / 1e6, 1),
                             "fprop_TFLOP/s": round(gemm_flops(M, N, K) / ms_f / 1e9, 1)}
    del X, W, qx, qw, Y

    # fp32 master weights -> FP8 (W2 14336 x 4096): tensorwise (amax, scale,
    # cast + transpose: 4 + 4 + 1 + 1 B/elt) and MXFP8 (4 + 1 + 1 + 2/32 B/elt)
    Wm = torch.from_numpy(workloads.normal([70, 0], (F, H), 0.02, "f32")).to(dev)
    wq, wqt = torch.empty((F, H), **u8), torch.empty((H, F), **u8)
    ws = torch.zeros(3, device=dev)
    ms_t = time_fn(torch, lambda: q.qsg_quantize(Wm, q.TENSORWISE, q.E4M3, q=wq, s=ws, qt=wqt))
    ws_mx, wst_mx = torch.empty((F, H // 32), **u8), torch.empty((H, F // 32), **u8)
    ms_m = time_fn(torch, lambda: q.qsg_quantize(Wm, q.MXFP8, q.E4M3, q=wq, s=ws_mx, qt=wqt, st=wst_mx))
    out["master_weights_fp32_14336x4096"] = {
        "tensorwise_ms": round(ms_t, 4), "tensorwise_GB/s": round(10.0 * Wm.numel() / ms_t / 1e6, 1),
        "mxfp8_ms": round(ms_m, 4), "mxfp8_GB/s": round((6.0 + 2.0 / 32) * Wm.numel() / ms_m / 1e6, 1)}
    del Wm, wq, wqt, ws_mx, wst_mx

    # wgrad accumulated into an fp32 main gradient: dW [4096 x 4096] +=
    # dY^T X over 32768 tokens (E5M2 x E4M3), next to the same GEMM with bf16 out
    Tk = 32768
    a_t = torch.randint(0, 0x7B, (H, Tk), dtype=torch.uint8, device=dev)  # finite E5M2 codes
    b_t = torch.randint(0, 0x7E, (H, Tk), dtype=torch.uint8, device=dev)  # finite E4M3 codes
    one = torch.ones(1, device=dev)
    main_grad = torch.zeros((H, H), device=dev)
    dw16 = torch.empty((H, H), dtype=torch.bfloat16, device=dev)
    T = q.TENSORWISE
    ms_acc = time_fn(torch, lambda: q.qsg_scaled_gemm_accumulate(a_t, q.E5M2, T, one, b_t, q.E4M3, T, one, main_grad))
    ms_bf = time_fn(torch, lambda: q.qsg_scaled_gemm(a_t, q.E5M2, T, one, b_t, q.E4M3, T, one, dw16))
    gfl = gemm_flops(H, H, Tk)
    out["wgrad_main_grad_fp32_4096"] = {"accumulate_TFLOP/s": round(gfl / ms_acc / 1e9, 1),
                                        "bf16_out_TFLOP/s": round(gfl / ms_bf / 1e9, 1)}
    del a_t, b_t, main_grad, dw16

    # wgrad kept in bf16 (--fp8-wgrad False): dW [4096 x 4096] = dY^T X over 32768 tokens
    dyb = torch.randn((Tk, H), device=dev).mul_(1e-3).to(torch.bfloat16)
    xb = torch.randn((Tk, H), device=dev).to(torch.bfloat16)
    dw_bf = torch.empty((H, H), dtype=torch.bfloat16, device=dev)
    mg = torch.zeros((H, H), device=dev)
    ms_w16 = time_fn(torch, lambda: q.qsg_wgrad_bf16(dyb, xb, dw_bf))
    ms_w32 = time_fn(torch, lambda: q.qsg_wgrad_bf16(dyb, xb, mg, accumulate=True))
    out["wgrad_bf16_4096"] = {"bf16_out_TFLOP/s": round(gfl / ms_w16 / 1e9, 1),
                              "fp32_accumulate_TFLOP/s": round(gfl / ms_w32 / 1e9, 1),
                              "frac_of_bf16_peak": round(gfl / ms_w16 / 1e9 / 2500.0, 4)}
    del dyb, xb, dw_bf, mg

    # GeLU with its input stored in FP8: h = the FC1 output X W2^T [32768 x 14336]
    # (~N(0, 1.28)); forward 2 + 2 + 1 B/elt, backward 2 + 1 + 2 B/elt
    M_ = 32768
    h = torch.from_numpy(workloads.normal([90, 9], (M_, F), 1.28).view(np.int16)).view(torch.bfloat16).to(dev)
    da = torch.from_numpy(workloads.normal([90, 10], (M_, F), 1e-3).view(np.int16)).view(torch.bfloat16).to(dev)
    act = torch.empty_like(h)
    hq = torch.empty((M_, F), **u8)
    dh = torch.empty_like(h)
    sc = torch.full((1,), 448.0 / 8.0, device=dev)
    si = 1.0 / sc
    ms_f = time_fn(torch, lambda: q.qsg_act_fp8_store_fwd(h, q.E4M3, sc, act, hq))
    ms_b = time_fn(torch, lambda: q.qsg_act_fp8_store_bwd(da, q.E4M3, hq, si, dh))
    out["gelu_fp8_input_store_32768x14336"] = {"fwd_ms": round(ms_f, 4), "fwd_GB/s": round(5.0 * h.numel() / ms_f / 1e6, 1),
                                               "bwd_ms": round(ms_b, 4), "bwd_GB/s": round(5.0 * h.numel() / ms_b / 1e6, 1)}
    return out


def cpu_baseline(step_flops, step_elems):
    """The oracle, untuned, on a bounded sample of the same workload, scaled
    to the step's TFLOP/s."""
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = 1

    # quantization sample: amax + scale + cast + transpose of X, W, W2 and dY
    # (344M of the step's 814M quantized elements)
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

    # GEMM sample: fp64 product of the dequantized operands, all 32768 rows
    # of X against all of W2 (the larger Linear's fprop)
    rows_g = M
    t0 = time.perf_counter()
    oracle.gemm_per_tensor(qx, "e4m3", sxi, qw, "e4m3", swi)
    tg = time.perf_counter() - t0
    gemm_rate = gemm_flops(rows_g, F, H) / tg

    step_time = per_elem * step_elems + step_flops / gemm_rate
    return {
        "value": step_flops / step_time / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"tensorwise quantize of X, W, W2 and dY ({nq / 1e6:.0f}M elements, {tq:.2f}s, numpy, "
                   f"1 thread) and the fp64 fprop GEMM of X ({rows_g} rows) against W2 ({tg:.2f}s, BLAS "
                   f"{blas_threads} threads), extrapolated to the full step's {step_elems/1e6:.0f}M quantized "
                   f"elements and {step_flops/1e12:.2f} TFLOP"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-recipes", action="store_true",
                    help="also time the delayed, MXFP8 and blockwise workloads (reported under 'recipes')")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()

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

    step, step_flops, step_elems = build_step(torch, q, dev)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step(Timer(torch))
    torch.cuda.synchronize()

    timer = Timer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    ks = timer.summary()
    kernels = {}
    for name, d in ks.items():
        avg_ms = d["ms"] / d["launches"]
        rec = {"launches_per_step": d["launches"] // args.steps, "avg_ms": round(avg_ms, 4)}
        if name.startswith("gemm"):
            tf = d["work"] / (d["ms"] * 1e-3) / 1e12
            rec.update({"TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_FP8_TFLOPS, 4)})
        elif d["work"] > 0:
            gb = d["work"] / (d["ms"] * 1e-3) / 1e9
            rec.update({"GB/s": round(gb, 1), "frac": round(gb / PEAK_HBM_GBPS, 4)})
        kernels[name] = rec

    gemm_ms = sum(d["ms"] for n, d in ks.items() if n.startswith("gemm")) / args.steps
    dom = max((n for n in ks if n.startswith("gemm")), key=lambda n: ks[n]["ms"])
    dd = ks[dom]
    achieved = dd["work"] / (dd["ms"] * 1e-3) / 1e12
    ct = ks["cast_transpose"]
    ct_gbps = ct["work"] / (ct["ms"] * 1e-3) / 1e9

    traffic = None
    prof_path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(prof_path):
        with open(prof_path) as fh:
            tr = json.load(fh).get(dom)
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
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic},
        "gemm_tflops": round(step_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "cast_transpose_gbps": round(ct_gbps, 1),
        "cast_transpose_frac": round(ct_gbps / PEAK_HBM_GBPS, 4),
        "kernels": kernels,
    }
    if args.all_recipes:
        line["recipes"] = other_recipes(torch, q, dev)
    if not args.no_cpu_baseline:
        t0 = time.time()
        line["cpu_baseline"] = cpu_baseline(step_flops, step_elems)
        log(f"[bench] cpu baseline took {time.time() - t0:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
