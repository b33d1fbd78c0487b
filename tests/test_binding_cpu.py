"""The Python binding rejects output and scale buffers whose device, dtype,
size or contiguity does not match the layout the C library will write or read
(include/qsg.h), before anything reaches the library.  A wrong buffer here
would otherwise become an out-of-bounds device access.

The checks run on stand-in tensor objects that report a GPU device, so no GPU
and no library call is needed.
"""

import pytest
import torch

import quantize_scaled_gemm_amd as q


class Dev:
    """A stand-in for a GPU tensor: shape, dtype, strides and contiguity."""

    def __init__(self, shape, dtype, strides=None, cuda=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        n = 1
        for d in self.shape:
            n *= d
        self._numel = n
        if strides is None:
            strides, acc = [], 1
            for d in reversed(self.shape):
                strides.append(acc)
                acc *= max(d, 1)
            strides = tuple(reversed(strides))
        self._strides = tuple(strides)
        self.is_cuda = cuda

    def dim(self):
        return len(self.shape)

    def numel(self):
        return self._numel

    def stride(self, i):
        return self._strides[i]

    def is_contiguous(self):
        acc = 1
        for d, s in zip(reversed(self.shape), reversed(self._strides)):
            if d > 1 and s != acc:
                return False
            acc *= d
        return True

    def data_ptr(self):
        raise AssertionError("the binding must reject this call before taking pointers")


U8, F32, BF = torch.uint8, torch.float32, torch.bfloat16


def raises(fn, text):
    with pytest.raises(q.QsgError, match=text):
        fn()


def test_cast_transpose_outputs():
    x = Dev((64, 96), BF)
    sc = Dev((1,), F32)
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, sc, Dev((64, 95), U8)), "q must hold exactly 6144")
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, sc, Dev((64, 96), F32)), "q must be u8")
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, sc, None, Dev((96, 64), U8, strides=(128, 1))), "qt must be contiguous")
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, Dev((2,), F32), Dev((64, 96), U8)), "scale must hold exactly 1")
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, sc, Dev((64, 96), U8, cuda=False)), "q must live on the GPU")
    raises(lambda: q.qsg_cast_transpose(x, q.E4M3, sc, Dev((64, 96), U8), amax_out=Dev((1,), BF)), "amax_out must be f32")


def test_quantize_scale_layouts():
    x = Dev((256, 512), BF)
    qq, qt = Dev((256, 512), U8), Dev((512, 256), U8)
    # tensorwise: s holds {amax, scale, scale_inv}
    raises(lambda: q.qsg_quantize(x, q.TENSORWISE, q.E4M3, q=qq, s=Dev((2,), F32)), "s must hold exactly 3")
    # MXFP8: E8M0 bytes rows x cols/32 and cols x rows/32
    raises(lambda: q.qsg_quantize(x, q.MXFP8, q.E4M3, q=qq, s=Dev((256, 16), F32)), "s must be u8")
    raises(lambda: q.qsg_quantize(x, q.MXFP8, q.E4M3, q=qq, s=Dev((256, 15), U8)), "s must hold exactly 4096")
    raises(lambda: q.qsg_quantize(x, q.MXFP8, q.E4M3, qt=qt, st=Dev((512, 4), U8)), "st must hold exactly 4096")
    # 1x128: fp32 rows x cols/128, cols x rows/128
    raises(lambda: q.qsg_quantize(x, q.BLOCK_1X128, q.E4M3, q=qq, s=Dev((256, 4), U8)), "s must be f32")
    raises(lambda: q.qsg_quantize(x, q.BLOCK_1X128, q.E4M3, qt=qt, st=Dev((512, 1), F32)), "st must hold exactly 1024")
    # 128x128: fp32 (rows/128) x (cols/128), the same count for the transposed grid
    raises(lambda: q.qsg_quantize(x, q.BLOCK_128X128, q.E4M3, q=qq, s=Dev((2, 3), F32)), "s must hold exactly 8")
    raises(lambda: q.qsg_quantize(x, q.BLOCK_128X128, q.E4M3, qt=qt, st=Dev((4, 3), F32)), "st must hold exactly 8")
    # a requested copy without its scale tensor
    raises(lambda: q.qsg_quantize(x, q.MXFP8, q.E4M3, q=qq), "s is required")


def test_gemm_scales_and_operands():
    M, N, K = 256, 384, 512
    a, b = Dev((M, K), U8), Dev((N, K), U8)
    c = Dev((M, N), BF)
    one = Dev((1,), F32)
    raises(lambda: q.qsg_scaled_gemm(Dev((M, K), BF), 0, q.TENSORWISE, one, b, 0, q.TENSORWISE, one, c),
           "A must hold FP8 bytes")
    raises(lambda: q.qsg_scaled_gemm(a, 0, q.TENSORWISE, Dev((3,), F32), b, 0, q.TENSORWISE, one, c),
           "sa must hold exactly 1")
    raises(lambda: q.qsg_scaled_gemm(a, 0, q.MXFP8, Dev((M, K // 32 - 1), U8), b, 0, q.MXFP8,
                                     Dev((N, K // 32), U8), c), "sa must hold exactly")
    raises(lambda: q.qsg_scaled_gemm(a, 0, q.MXFP8, Dev((M, K // 32), U8), b, 0, q.MXFP8,
                                     Dev((N, K // 32), F32), c), "sb must be u8")
    raises(lambda: q.qsg_scaled_gemm(a, 0, q.BLOCK_1X128, Dev((M, K // 128), F32), b, 0, q.BLOCK_128X128,
                                     Dev((N // 128 + 1, K // 128), F32), c), "sb must hold exactly 12")
    raises(lambda: q.qsg_scaled_gemm(a, 0, q.BLOCK_1X128, Dev((M, K // 128), F32), b, 0, q.BLOCK_1X128,
                                     Dev((N // 128, K // 128), F32), c), "sb must hold exactly 1536")
    raises(lambda: q.qsg_scaled_gemm_accumulate(a, 0, q.BLOCK_1X128, Dev((M + 1, K // 128), F32), b, 0,
                                                q.BLOCK_1X128, Dev((N, K // 128), F32), Dev((M, N), F32)),
           "sa must hold exactly 1024")


def test_activation_outputs():
    h = Dev((32, 64), BF)
    sc = Dev((1,), F32)
    raises(lambda: q.qsg_act_fp8_store_fwd(h, 0, sc, Dev((32, 64), F32), Dev((32, 64), U8)), "a must be bf16")
    raises(lambda: q.qsg_act_fp8_store_fwd(h, 0, sc, Dev((32, 64), BF), Dev((32, 63), U8)), "q must hold exactly")
    raises(lambda: q.qsg_act_fp8_store_bwd(h, 0, Dev((32, 64), U8), sc, Dev((16, 64), BF)), "dh must hold exactly")


def test_scalar_buffers():
    raises(lambda: q.qsg_amax(Dev((4, 4), BF), Dev((1,), BF)), "amax must be f32")
    raises(lambda: q.qsg_compute_scale(Dev((1,), F32), 0, 0, Dev((1,), F32), Dev((2,), F32)),
           "scale_inv must hold exactly 1")
    raises(lambda: q.qsg_amax_update(Dev((16,), F32), 0, Dev((1,), F32), 0, 0, Dev((1,), F32), Dev((1,), BF)),
           "scale_inv must be f32")
