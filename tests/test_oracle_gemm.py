"""Pins of the oracle's fp64 GEMMs against exact rational brute force.

* per-tensor, MX and blockwise GEMMs on tiny random FP8 operands equal the
  exact Fraction sum (per-tensor: exactly; the others: within fp64 rounding);
* integer-valued operands give an exactly known product;
* the three GEMMs of a Linear (fprop, dgrad, wgrad) built from the quantized
  tensors and their transposed copies agree with the dense products;
* the acceptance rule rejects a planted error (a wrong sign, a transposed
  operand, a 2% scale error);
* accumulating into an fp32 C micro-batch by micro-batch equals C plus the
  product over the concatenated contraction (exact rational brute force).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def rand_codes(g, shape, fmt):
    """Random finite FP8 codes."""
    t = oracle.decode_table(fmt)
    finite = np.nonzero(np.isfinite(t))[0]
    return finite[g.integers(0, finite.size, size=shape)].astype(np.uint8)


def as_float(mat):
    return np.array([[float(v) for v in row] for row in mat], dtype=np.float64)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
def test_per_tensor_exact(fa, fb):
    g = np.random.Generator(np.random.PCG64(31))
    qa = rand_codes(g, (5, 70), fa)
    qb = rand_codes(g, (6, 70), fb)
    sa, sb = np.float32(0.375), np.float32(3.0)
    ref = oracle.gemm_per_tensor(qa, fa, sa, qb, fb, sb)
    ex = oracle.gemm_exact_fraction(qa, fa, lambda m, k: Fraction(0.375),
                                    qb, fb, lambda n, k: Fraction(3))
    # E4M3 x E4M3 code products are multiples of 2^-18 below 2^18: exact in fp64
    if (fa, fb) == ("e4m3", "e4m3"):
        assert np.array_equal(ref, as_float(ex))
    else:
        assert np.allclose(ref, as_float(ex), rtol=1e-14, atol=0)


def test_mx_gemm_vs_fraction():
    g = np.random.Generator(np.random.PCG64(32))
    M, N, K = 4, 5, 96
    qa = rand_codes(g, (M, K), "e4m3")
    qb = rand_codes(g, (N, K), "e4m3")
    sa = g.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    ref = oracle.gemm_mx(qa, "e4m3", sa, qb, "e4m3", sb)
    ex = oracle.gemm_exact_fraction(
        qa, "e4m3", lambda m, k: Fraction(2) ** (int(sa[m, k // 32]) - 127),
        qb, "e4m3", lambda n, k: Fraction(2) ** (int(sb[n, k // 32]) - 127))
    exf = as_float(ex)
    assert np.allclose(ref, exf, rtol=1e-13, atol=1e-14 * np.abs(exf).max())


@pytest.mark.parametrize("layout", ["128x128", "1x128"])
def test_block_gemm_vs_fraction(layout):
    g = np.random.Generator(np.random.PCG64(33))
    M, N, K = 3, 130, 256
    qa = rand_codes(g, (M, K), "e4m3")
    qb = rand_codes(g, (N, K), "e4m3")
    sa = g.uniform(0.001, 0.01, (M, K // 128)).astype(np.float32)
    if layout == "128x128":
        sb = g.uniform(0.001, 0.01, ((N + 127) // 128, K // 128)).astype(np.float32)
        bsc = lambda n, k: Fraction(float(sb[n // 128, k // 128]))  # noqa: E731
    else:
        sb = g.uniform(0.001, 0.01, (N, K // 128)).astype(np.float32)
        bsc = lambda n, k: Fraction(float(sb[n, k // 128]))  # noqa: E731
    ref = oracle.gemm_block(qa, "e4m3", sa, qb, "e4m3", sb, layout)
    ex = oracle.gemm_exact_fraction(qa, "e4m3", lambda m, k: Fraction(float(sa[m, k // 128])),
                                    qb, "e4m3", bsc)
    exf = as_float(ex)
    assert np.allclose(ref, exf, rtol=1e-12, atol=1e-14 * np.abs(exf).max())


def test_integer_operands_exact():
    # small integers are exact FP8 values; the product is an exact integer
    g = np.random.Generator(np.random.PCG64(34))
    ia = g.integers(-15, 16, size=(33, 200))
    ib = g.integers(-15, 16, size=(17, 200))
    qa = oracle.encode(ia.astype(np.float32), "e4m3")
    qb = oracle.encode(ib.astype(np.float32), "e4m3")
    ref = oracle.gemm_per_tensor(qa, "e4m3", np.float32(1), qb, "e4m3", np.float32(1))
    assert np.array_equal(ref, (ia @ ib.T).astype(np.float64))


def test_linear_three_gemms_from_quantized_copies():
    g = np.random.Generator(np.random.PCG64(35))
    M, K, N = 64, 96, 48
    x = g.standard_normal((M, K)).astype(np.float32)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    dy = (g.standard_normal((M, N)) * 1e-3).astype(np.float32)
    qx, qxt, _, _, sxi = oracle.quantize_tensorwise(x, "e4m3")
    qw, qwt, _, _, swi = oracle.quantize_tensorwise(w, "e4m3")
    qd, qdt, _, _, sdi = oracle.quantize_tensorwise(dy, "e5m2")
    X = oracle.dequantize(qx, "e4m3") * float(sxi)
    W = oracle.dequantize(qw, "e4m3") * float(swi)
    D = oracle.dequantize(qd, "e5m2") * float(sdi)
    y = oracle.gemm_per_tensor(qx, "e4m3", sxi, qw, "e4m3", swi)
    dx = oracle.gemm_per_tensor(qd, "e5m2", sdi, qwt, "e4m3", swi)
    dw = oracle.gemm_per_tensor(qdt, "e5m2", sdi, qxt, "e4m3", sxi)
    assert np.allclose(y, X @ W.T, rtol=1e-12, atol=1e-300)
    assert np.allclose(dx, D @ W, rtol=1e-12, atol=1e-300)
    assert np.allclose(dw, D.T @ X, rtol=1e-12, atol=1e-300)
    # and they approximate the unquantized products (FP8 is a few % accurate)
    assert np.linalg.norm(y - x @ w.T) / np.linalg.norm(x @ w.T) < 0.08


def test_tolerance_rule_rejects_planted_errors():
    g = np.random.Generator(np.random.PCG64(36))
    qa = rand_codes(g, (32, 64), "e4m3")
    qb = rand_codes(g, (24, 64), "e4m3")
    ref = oracle.gemm_per_tensor(qa, "e4m3", 1.0, qb, "e4m3", 1.0)
    ok, _ = oracle.tolerance_check(ref.astype(np.float32), ref)
    assert ok
    assert not oracle.tolerance_check(-ref, ref)[0]
    assert not oracle.tolerance_check(ref * 1.02, ref)[0]
    qbt = np.ascontiguousarray(qb[:, ::-1])  # a permuted K index
    wrong = oracle.gemm_per_tensor(qa, "e4m3", 1.0, qbt, "e4m3", 1.0)
    assert not oracle.tolerance_check(wrong, ref)[0]
    # bf16 rounding of the output is inside the rule
    import torch
    yb = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert oracle.tolerance_check(yb, ref)[0]


def test_accumulate_over_micro_batches_vs_fraction():
    """Two accumulations of wgrad-shaped products (contraction over the
    tokens of two micro-batches) into an fp32 C equal C + the product over
    all tokens, which is one exact rational sum; a planted sign error in the
    accumulation fails the comparison."""
    g = np.random.Generator(np.random.PCG64(36))
    N, K, T = 5, 7, 24  # dW is N x K; each micro-batch has T tokens
    qdy = [rand_codes(g, (N, T), "e5m2") for _ in range(2)]  # Q(dY)^T of each micro-batch
    qx = [rand_codes(g, (K, T), "e4m3") for _ in range(2)]   # Q(X)^T
    c0 = g.standard_normal((N, K)).astype(np.float32)
    sa, sb = np.float32(0.375), np.float32(2.0 ** -7)
    c1 = oracle.accumulate(c0, oracle.gemm_per_tensor(qdy[0], "e5m2", sa, qx[0], "e4m3", sb))
    c = oracle.accumulate(np.float32(c1), oracle.gemm_per_tensor(qdy[1], "e5m2", sa, qx[1], "e4m3", sb))
    full = oracle.gemm_exact_fraction(np.concatenate(qdy, axis=1), "e5m2", lambda m, k: Fraction(float(sa)),
                                      np.concatenate(qx, axis=1), "e4m3", lambda n, k: Fraction(float(sb)))
    exact = as_float([[Fraction(float(c0[i, j])) + full[i][j] for j in range(K)] for i in range(N)])
    # the roundings: binary32 C between the two accumulations (half an ulp
    # of c1) and fp64 in the sums (far below that)
    bound = 2.0 ** -24 * np.abs(c1) + 2.0 ** -40 * (np.abs(exact) + 1)
    assert np.all(np.abs(c - exact) <= bound)
    bad = np.asarray(c0, dtype=np.float64) - oracle.gemm_per_tensor(qdy[0], "e5m2", sa, qx[0], "e4m3", sb)
    bad = oracle.accumulate(np.float32(bad), oracle.gemm_per_tensor(qdy[1], "e5m2", sa, qx[1], "e4m3", sb))
    assert not np.all(np.abs(bad - exact) <= bound)


def test_wgrad_bf16_vs_token_loop_and_fp8_convention():
    """The bf16 wgrad against an exact rational loop over the tokens, and
    against the FP8 wgrad convention (A = dY^T, B = X^T, C = A B^T) on values
    that both formats hold exactly; a transposed operand fails both."""
    g = np.random.Generator(np.random.PCG64(37))
    T, N, K = 9, 4, 6
    dy = g.integers(-8, 9, (T, N)).astype(np.float32) * np.float32(0.25)
    x = g.integers(-15, 16, (T, K)).astype(np.float32)
    ref = oracle.wgrad_bf16(dy, x)
    exact = [[sum(Fraction(float(dy[t, n])) * Fraction(float(x[t, k])) for t in range(T)) for k in range(K)]
             for n in range(N)]
    assert np.array_equal(ref, as_float(exact))
    qa = oracle.encode(np.ascontiguousarray(dy.T), "e5m2")
    qb = oracle.encode(np.ascontiguousarray(x.T), "e4m3")
    assert np.array_equal(ref, oracle.gemm_per_tensor(qa, "e5m2", np.float32(1), qb, "e4m3", np.float32(1)))
    # square operands: dY used without its transpose has the right shape but
    # not the right value
    sq_dy = g.integers(-8, 9, (5, 5)).astype(np.float32)
    sq_x = g.integers(-8, 9, (5, 5)).astype(np.float32)
    sq = [[sum(Fraction(float(sq_dy[t, n])) * Fraction(float(sq_x[t, k])) for t in range(5)) for k in range(5)]
          for n in range(5)]
    assert np.array_equal(oracle.wgrad_bf16(sq_dy, sq_x), as_float(sq))
    assert not np.array_equal(np.asarray(sq_dy, np.float64) @ np.asarray(sq_x, np.float64), as_float(sq))
