"""The allocation-free delayed step (qsg_cast_transpose_delayed_noalloc,
workspace in the library's per-GPU device array) gives the same bytes, amax,
history and scales as qsg_cast_transpose_delayed with a caller workspace, on
two calls in a row, the second on a smaller tensor (so the array's contents
after a large call must not disturb a small one)."""

import numpy as np
import pytest

import workloads
from helpers import to_dev_bf16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantize_scaled_gemm_amd as q

    q.load_library()
    return q


def test_noalloc_matches_workspace_variant(q):
    import torch

    L = 16
    shapes = [(4096, 4096), (200, 300)]  # the second call is smaller (and ragged)
    res = {}
    for path in ("ws", "noalloc"):
        hist = torch.zeros(L, device="cuda")
        scale, inv = torch.ones(1, device="cuda"), torch.ones(1, device="cuda")
        ws = torch.zeros(q.DELAYED_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
        out = []
        for t, (R, C) in enumerate(shapes):
            xd = to_dev_bf16(workloads.delayed_4096_step(t, R, C, out_cols=8)["X"])
            qq = torch.empty((R, C), dtype=torch.uint8, device="cuda")
            qt = torch.empty((C, R), dtype=torch.uint8, device="cuda")
            amax = torch.full((1,), -1.0, device="cuda")
            if path == "ws":
                q.qsg_cast_transpose_delayed(xd, q.E4M3, 0, hist, t, scale, inv, qq, qt, amax, ws)
            else:
                q.qsg_cast_transpose_delayed_noalloc(xd, q.E4M3, 0, hist, t, scale, inv, qq, qt, amax)
            out.append([to_np(v).copy() for v in (qq, qt, amax, scale, inv, hist)])
        res[path] = out
    for t in range(len(shapes)):
        for a, b in zip(res["ws"][t], res["noalloc"][t]):
            assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8)), t
    assert res["noalloc"][1][2][0] > 0 and res["noalloc"][1][3][0] != 1.0
