"""The C ABI promises asynchronous calls with no host synchronisation, so a
sequence of them can be captured in a HIP graph.  This captures one
tensorwise step of a small Linear -- amax, scale, cast + transpose of X, W
(E4M3) and dY (E5M2), then fprop, dgrad and wgrad -- and replays it four
times, with eager work and synchronisations between the replays, after
changing the inputs in place; every replay must equal the eager run on the
same inputs bit for bit (the clears of the amax are fill kernels, not
memsets, so they replay too)."""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def test_graph_replay_matches_eager(q):
    import torch

    dev = torch.device("cuda")
    M, K, N = 512, 768, 1024
    bf = dict(dtype=torch.bfloat16, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    X = torch.empty((M, K), **bf)
    W = torch.empty((N, K), **bf)
    dY = torch.empty((M, N), **bf)
    tens = {}
    for name, t, fmt in (("X", X, q.E4M3), ("W", W, q.E4M3), ("dY", dY, q.E5M2)):
        r, c = t.shape
        tens[name] = dict(x=t, f=fmt, q=torch.empty((r, c), **u8), qt=torch.empty((c, r), **u8),
                          amax=torch.zeros(1, device=dev), s=torch.zeros(1, device=dev),
                          si=torch.zeros(1, device=dev))
    Y = torch.empty((M, N), **bf)
    dX = torch.empty((M, K), **bf)
    dW = torch.empty((N, K), device=dev)  # fp32 main gradient, accumulated

    def fill(seed):
        for name, t, std in (("X", X, 1.0), ("W", W, 0.02), ("dY", dY, 1e-3)):
            bits = workloads.normal([95, seed, len(name)], tuple(t.shape), std)
            t.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev))
        dW.zero_()

    T = q.TENSORWISE

    def step():
        for name in ("X", "W", "dY"):
            t = tens[name]
            q.qsg_amax(t["x"], t["amax"])
            q.qsg_compute_scale(t["amax"], t["f"], 0, t["s"], t["si"])
            q.qsg_cast_transpose(t["x"], t["f"], t["s"], t["q"], t["qt"])
        x, w, d = tens["X"], tens["W"], tens["dY"]
        q.qsg_scaled_gemm(x["q"], q.E4M3, T, x["si"], w["q"], q.E4M3, T, w["si"], Y)
        q.qsg_scaled_gemm(d["q"], q.E5M2, T, d["si"], w["qt"], q.E4M3, T, w["si"], dX)
        q.qsg_scaled_gemm_accumulate(d["qt"], q.E5M2, T, d["si"], x["qt"], q.E4M3, T, x["si"], dW)

    def snapshot():
        torch.cuda.synchronize()
        out = {k: v.clone() for k, v in (("Y", Y), ("dX", dX), ("dW", dW))}
        for name, t in tens.items():
            out[name + ".q"] = t["q"].clone()
            out[name + ".qt"] = t["qt"].clone()
            out[name + ".si"] = t["si"].clone()
        return out

    eager = {}
    for seed in range(4):
        fill(seed)
        step()
        eager[seed] = snapshot()

    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in range(4):
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        # eager work between replays
        torch.matmul(X.float(), X.float().T)
        for key, ref in eager[seed].items():
            a, b = got[key], ref
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            elif a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), (seed, key)
