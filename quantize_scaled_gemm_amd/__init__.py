"""Python binding of libqsg.so (FP8 quantization and scaled FP8 GEMM on
MI355X / gfx950).

Argument marshalling only: every function below has the name of the C entry
point it calls (declared in include/qsg.h), turns torch tensors into device
pointers, sizes and leading dimensions, passes the current HIP stream, and
raises ``QsgError`` on a non-zero status.  All computation happens in the HIP
kernels of the library.  There is no fallback: if the library is missing or
fails to load, every call raises.
"""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqsg.so")

# enums of include/qsg.h
E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
TENSORWISE, DELAYED, MXFP8, BLOCK_1X128, BLOCK_128X128 = 0, 1, 2, 3, 4
MX_CEIL, MX_OCP_FLOOR = 0, 1
AMAX_MAX = 0

FMT = {"e4m3": E4M3, "e5m2": E5M2}

ENTRY_POINTS = (
    "qsg_version",
    "qsg_status_string",
    "qsg_last_error",
    "qsg_amax",
    "qsg_compute_scale",
    "qsg_cast_transpose",
    "qsg_cast_transpose_delayed",
    "qsg_cast_transpose_delayed_noalloc",
    "qsg_amax_update",
    "qsg_quantize",
    "qsg_scaled_gemm",
    "qsg_scaled_gemm_accumulate",
    "qsg_act_fp8_store_fwd",
    "qsg_act_fp8_store_bwd",
    "qsg_wgrad_bf16",
    "qsg_quantize_nvfp4",
    "qsg_gemm_nvfp4",
)


class QsgError(RuntimeError):
    pass


class Recipe(ctypes.Structure):
    _fields_ = [("scaling", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("margin", ctypes.c_int32), ("mx_rule", ctypes.c_int32)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libqsg.so (once) and declare the argument types."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QsgError(f"{path} is not built: run `python -m quantize_scaled_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.qsg_version.restype = I
    lib.qsg_version.argtypes = []
    lib.qsg_status_string.restype = ctypes.c_char_p
    lib.qsg_status_string.argtypes = [I]
    lib.qsg_last_error.restype = ctypes.c_char_p
    lib.qsg_last_error.argtypes = []
    lib.qsg_amax.restype = I
    lib.qsg_amax.argtypes = [P, I, I64, I64, I64, F, P]
    lib.qsg_compute_scale.restype = I
    lib.qsg_compute_scale.argtypes = [F, I, I, F, F, P]
    lib.qsg_cast_transpose.restype = I
    lib.qsg_cast_transpose.argtypes = [P, I, I64, I64, I64, I, F, P, P, F, P]
    lib.qsg_cast_transpose_delayed.restype = I
    lib.qsg_cast_transpose_delayed.argtypes = [P, I, I64, I64, I64, I, I, F, I64, I64, F, F, P, P, F, P, P]
    lib.qsg_cast_transpose_delayed_noalloc.restype = I
    lib.qsg_cast_transpose_delayed_noalloc.argtypes = [P, I, I64, I64, I64, I, I, F, I64, I64, F, F, P, P, F, P]
    lib.qsg_amax_update.restype = I
    lib.qsg_amax_update.argtypes = [F, I64, I64, F, I, I, I, F, F, P]
    lib.qsg_quantize.restype = I
    lib.qsg_quantize.argtypes = [P, I, I64, I64, I64, ctypes.POINTER(Recipe), P, P, P, P, P]
    lib.qsg_scaled_gemm.restype = I
    lib.qsg_scaled_gemm.argtypes = [P, I, I, P, P, I, I, P, I64, I64, I64, I64, I64, P, I, I64, P]
    lib.qsg_scaled_gemm_accumulate.restype = I
    lib.qsg_wgrad_bf16.restype = I
    lib.qsg_wgrad_bf16.argtypes = [P, I64, I64, I64, P, I64, I64, P, I, I64, I, P]
    lib.qsg_act_fp8_store_fwd.restype = I
    lib.qsg_act_fp8_store_fwd.argtypes = [P, I64, I64, I64, I, F, P, P, F, P]
    lib.qsg_act_fp8_store_bwd.restype = I
    lib.qsg_act_fp8_store_bwd.argtypes = [P, I64, I64, I64, I, P, F, P, P]
    lib.qsg_scaled_gemm_accumulate.argtypes = [P, I, I, P, P, I, I, P, I64, I64, I64, I64, I64, P, I64, P]
    lib.qsg_quantize_nvfp4.argtypes = [P, I, I64, I64, I64, P, P, P, P, P, P]
    lib.qsg_gemm_nvfp4.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P, I, I64, P]
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise QsgError("tensors passed to libqsg must live on the GPU")
    return t.data_ptr()


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise QsgError(f"unsupported input dtype {t.dtype}")


def _matrix(t):
    """(rows, cols, ld) of a 2-D row-major tensor view (unit column stride)."""
    if t.dim() != 2:
        raise QsgError("expected a 2-D tensor")
    rows, cols = t.shape
    if t.numel() == 0:
        return rows, cols, max(cols, 1)
    if cols > 1 and t.stride(1) != 1:
        raise QsgError("the last dimension must be contiguous")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return rows, cols, max(ld, cols)


def _buffer(t, name, numel, dtype, required=True):
    """Check a buffer the library reads or writes densely: on the GPU,
    contiguous, exactly ``numel`` elements of ``dtype`` ("u8", "f32", "bf16").
    Raw integer pointers are passed through unchecked (the C ABI's own
    contract applies to them)."""
    if t is None:
        if required:
            raise QsgError(f"{name} is required")
        return
    if isinstance(t, int):
        return
    import torch

    want = {"u8": torch.uint8, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    if not t.is_cuda:
        raise QsgError(f"{name} must live on the GPU")
    if t.dtype != want:
        raise QsgError(f"{name} must be {dtype} (got {t.dtype})")
    if t.numel() != numel:
        raise QsgError(f"{name} must hold exactly {numel} elements (got {t.numel()}, shape {tuple(t.shape)})")
    if numel > 0 and not t.is_contiguous():
        raise QsgError(f"{name} must be contiguous")


def _scale_layout(kind, rows, K):
    """(numel, dtype) of a scale tensor of the given kind for an operand of
    `rows` rows and contraction length K (include/qsg.h, qsg_scaling), or
    None when K breaks the kind's block rule (the library then reports the
    shape error)."""
    if kind in (TENSORWISE, DELAYED):
        return 1, "f32"
    if kind == MXFP8:
        return (rows * (K // 32), "u8") if K % 32 == 0 else None
    if kind == BLOCK_1X128:
        return (rows * (K // 128), "f32") if K % 128 == 0 else None
    if kind == BLOCK_128X128:
        return (((rows + 127) // 128) * (K // 128), "f32") if K % 128 == 0 else None
    return None


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(rc):
    if rc != 0:
        lib = load_library()
        msg = lib.qsg_last_error().decode()
        raise QsgError(f"{lib.qsg_status_string(rc).decode()} ({rc}): {msg}")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def qsg_version():
    return load_library().qsg_version()


def qsg_amax(x, amax, stream=None):
    """amax (1 fp32 on the GPU) = max |x|."""
    rows, cols, ld = _matrix(x)
    _buffer(amax, "amax", 1, "f32")
    _check(load_library().qsg_amax(_ptr(x), _dtype_code(x), rows, cols, ld, _ptr(amax), _stream(stream)))


def qsg_compute_scale(amax, fmt, margin, scale, scale_inv, stream=None):
    for t, n in ((amax, "amax"), (scale, "scale"), (scale_inv, "scale_inv")):
        _buffer(t, n, 1, "f32")
    _check(load_library().qsg_compute_scale(_ptr(amax), fmt, margin, _ptr(scale), _ptr(scale_inv),
                                            _stream(stream)))


def qsg_cast_transpose(x, fmt, scale, q=None, qt=None, amax_out=None, stream=None):
    rows, cols, ld = _matrix(x)
    _buffer(scale, "scale", 1, "f32")
    _buffer(q, "q", rows * cols, "u8", required=False)
    _buffer(qt, "qt", rows * cols, "u8", required=False)
    _buffer(amax_out, "amax_out", 1, "f32", required=False)
    _check(load_library().qsg_cast_transpose(_ptr(x), _dtype_code(x), rows, cols, ld, fmt, _ptr(scale),
                                             _ptr(q), _ptr(qt), _ptr(amax_out), _stream(stream)))


DELAYED_WORKSPACE_BYTES = 4224  # QSG_DELAYED_WORKSPACE_BYTES of include/qsg.h


def qsg_cast_transpose_delayed(x, fmt, margin, history, step, scale, scale_inv, q=None, qt=None, amax_out=None,
                               workspace=None, stream=None):
    """One delayed-scaling step of x in one launch: q / qt with the scale in
    force, amax into history[step mod len], scale / scale_inv for the next
    step.  workspace: DELAYED_WORKSPACE_BYTES zeroed bytes on the GPU, reused
    from call to call (every call leaves it zero)."""
    rows, cols, ld = _matrix(x)
    _buffer(history, "history", history.numel(), "f32")
    for t, n in ((scale, "scale"), (scale_inv, "scale_inv")):
        _buffer(t, n, 1, "f32")
    _buffer(q, "q", rows * cols, "u8", required=False)
    _buffer(qt, "qt", rows * cols, "u8", required=False)
    _buffer(amax_out, "amax_out", 1, "f32", required=False)
    if workspace is None:
        raise QsgError("workspace is required")
    if not isinstance(workspace, int):
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise QsgError("workspace must be a contiguous GPU tensor")
        if workspace.numel() * workspace.element_size() < DELAYED_WORKSPACE_BYTES:
            raise QsgError(f"workspace must hold at least {DELAYED_WORKSPACE_BYTES} bytes")
    _check(load_library().qsg_cast_transpose_delayed(_ptr(x), _dtype_code(x), rows, cols, ld, fmt, margin,
                                                     _ptr(history), history.numel(), step, _ptr(scale),
                                                     _ptr(scale_inv), _ptr(q), _ptr(qt), _ptr(amax_out),
                                                     _ptr(workspace), _stream(stream)))


def qsg_cast_transpose_delayed_noalloc(x, fmt, margin, history, step, scale, scale_inv, q=None, qt=None,
                                       amax_out=None, stream=None):
    """qsg_cast_transpose_delayed with the library's own per-GPU workspace
    (no allocation; overlapping calls on one GPU race)."""
    rows, cols, ld = _matrix(x)
    _buffer(history, "history", history.numel(), "f32")
    for t, n in ((scale, "scale"), (scale_inv, "scale_inv")):
        _buffer(t, n, 1, "f32")
    _buffer(q, "q", rows * cols, "u8", required=False)
    _buffer(qt, "qt", rows * cols, "u8", required=False)
    _buffer(amax_out, "amax_out", 1, "f32", required=False)
    _check(load_library().qsg_cast_transpose_delayed_noalloc(_ptr(x), _dtype_code(x), rows, cols, ld, fmt, margin,
                                                             _ptr(history), history.numel(), step, _ptr(scale),
                                                             _ptr(scale_inv), _ptr(q), _ptr(qt), _ptr(amax_out),
                                                             _stream(stream)))


def qsg_amax_update(history, step, amax, fmt, margin, scale, scale_inv, algo=AMAX_MAX, stream=None):
    _buffer(history, "history", history.numel(), "f32")
    for t, n in ((amax, "amax"), (scale, "scale"), (scale_inv, "scale_inv")):
        _buffer(t, n, 1, "f32")
    _check(load_library().qsg_amax_update(_ptr(history), history.numel(), step, _ptr(amax), algo, fmt,
                                          margin, _ptr(scale), _ptr(scale_inv), _stream(stream)))


def qsg_quantize(x, scaling, fmt, q=None, s=None, qt=None, st=None, margin=0, mx_rule=MX_CEIL,
                 stream=None):
    rows, cols, ld = _matrix(x)
    _buffer(q, "q", rows * cols, "u8", required=False)
    _buffer(qt, "qt", rows * cols, "u8", required=False)
    if scaling == TENSORWISE:
        _buffer(s, "s", 3, "f32")
    elif scaling in (MXFP8, BLOCK_1X128, BLOCK_128X128):
        # row-wise copy: blocks along cols; column-wise copy: blocks along rows
        if scaling == BLOCK_128X128:
            ok = rows % 128 == 0 and cols % 128 == 0
            row = col = ((rows // 128) * (cols // 128), "f32") if ok else None
        else:
            row, col = _scale_layout(scaling, rows, cols), _scale_layout(scaling, cols, rows)
        if row is not None and q is not None:
            _buffer(s, "s", row[0], row[1])
        if col is not None and qt is not None:
            _buffer(st, "st", col[0], col[1])
    rec = Recipe(scaling, fmt, margin, mx_rule)
    _check(load_library().qsg_quantize(_ptr(x), _dtype_code(x), rows, cols, ld, ctypes.byref(rec),
                                       _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _stream(stream)))


def _gemm_operands(a, b):
    import torch

    for t, name in ((a, "A"), (b, "B")):
        if t.dtype != torch.uint8:
            raise QsgError(f"{name} must hold FP8 bytes as uint8 (got {t.dtype})")
        if not t.is_cuda:
            raise QsgError(f"{name} must live on the GPU")


def _gemm_scales(ka, sa, M, kb, sb, N, K):
    for kind, t, rows, name in ((ka, sa, M, "sa"), (kb, sb, N, "sb")):
        lay = _scale_layout(kind, rows, K)
        if lay is not None:
            _buffer(t, name, lay[0], lay[1])


def qsg_scaled_gemm(a, fa, ka, sa, b, fb, kb, sb, c, stream=None):
    """C (M x N) = (A sa)(B sb)^T; A is M x K and B is N x K (uint8 FP8 bytes)."""
    M, K, lda = _matrix(a)
    N, Kb, ldb = _matrix(b)
    if Kb != K:
        raise QsgError(f"K mismatch: A has {K}, B has {Kb}")
    Mc, Nc, ldc = _matrix(c)
    if (Mc, Nc) != (M, N):
        raise QsgError(f"C is {Mc}x{Nc}, expected {M}x{N}")
    _gemm_operands(a, b)
    _gemm_scales(ka, sa, M, kb, sb, N, K)
    _check(load_library().qsg_scaled_gemm(_ptr(a), fa, ka, _ptr(sa), _ptr(b), fb, kb, _ptr(sb), M, N, K,
                                          lda, ldb, _ptr(c), _dtype_code(c), ldc, _stream(stream)))


def qsg_scaled_gemm_accumulate(a, fa, ka, sa, b, fb, kb, sb, c, stream=None):
    """C (M x N, fp32) = fp32(C + (A sa)(B sb)^T), in place."""
    import torch

    M, K, lda = _matrix(a)
    N, Kb, ldb = _matrix(b)
    if Kb != K:
        raise QsgError(f"K mismatch: A has {K}, B has {Kb}")
    Mc, Nc, ldc = _matrix(c)
    if (Mc, Nc) != (M, N):
        raise QsgError(f"C is {Mc}x{Nc}, expected {M}x{N}")
    if c.dtype != torch.float32:
        raise QsgError("qsg_scaled_gemm_accumulate accumulates into an fp32 C")
    _gemm_operands(a, b)
    _gemm_scales(ka, sa, M, kb, sb, N, K)
    _check(load_library().qsg_scaled_gemm_accumulate(_ptr(a), fa, ka, _ptr(sa), _ptr(b), fb, kb, _ptr(sb), M, N,
                                                     K, lda, ldb, _ptr(c), ldc, _stream(stream)))


def qsg_act_fp8_store_fwd(h, fmt, scale, a, q, amax_out=None, stream=None):
    """a = bf16(gelu(h)); q = FP8 of h * scale (h bf16, a and q dense)."""
    rows, cols, ld = _matrix(h)
    if _dtype_code(h) != BF16:
        raise QsgError("qsg_act_fp8_store_fwd takes a bf16 input")
    _buffer(scale, "scale", 1, "f32")
    _buffer(a, "a", rows * cols, "bf16")
    _buffer(q, "q", rows * cols, "u8")
    _buffer(amax_out, "amax_out", 1, "f32", required=False)
    _check(load_library().qsg_act_fp8_store_fwd(_ptr(h), rows, cols, ld, fmt, _ptr(scale), _ptr(a), _ptr(q),
                                                _ptr(amax_out), _stream(stream)))


def qsg_act_fp8_store_bwd(da, fmt, q, scale_inv, dh, stream=None):
    """dh = bf16(da * gelu'(dec(q) * scale_inv)) (da bf16, q and dh dense)."""
    rows, cols, ld = _matrix(da)
    if _dtype_code(da) != BF16:
        raise QsgError("qsg_act_fp8_store_bwd takes a bf16 gradient")
    _buffer(q, "q", rows * cols, "u8")
    _buffer(scale_inv, "scale_inv", 1, "f32")
    _buffer(dh, "dh", rows * cols, "bf16")
    _check(load_library().qsg_act_fp8_store_bwd(_ptr(da), rows, cols, ld, fmt, _ptr(q), _ptr(scale_inv), _ptr(dh),
                                                _stream(stream)))


def qsg_wgrad_bf16(dy, x, c, accumulate=False, stream=None):
    """C (N x K) = dY^T X, or C += dY^T X for an fp32 C (dY T x N, X T x K, bf16)."""
    T, N, lddy = _matrix(dy)
    Tx, K, ldx = _matrix(x)
    if Tx != T:
        raise QsgError(f"token count mismatch: dY has {T}, X has {Tx}")
    if _dtype_code(dy) != BF16 or _dtype_code(x) != BF16:
        raise QsgError("qsg_wgrad_bf16 takes bf16 operands")
    Nc, Kc, ldc = _matrix(c)
    if (Nc, Kc) != (N, K):
        raise QsgError(f"C is {Nc}x{Kc}, expected {N}x{K}")
    _check(load_library().qsg_wgrad_bf16(_ptr(dy), T, N, lddy, _ptr(x), K, ldx, _ptr(c), _dtype_code(c), ldc,
                                         1 if accumulate else 0, _stream(stream)))


def qsg_quantize_nvfp4(x, tensor_scale, q=None, s=None, qt=None, st=None, stream=None):
    """NVFP4 copies of x: tensor_scale (3 fp32: amax, s_enc, s_dec); row-wise
    q (rows x cols/2 packed E2M1) with s (rows x cols/16 E4M3 bytes) and/or
    column-wise qt (cols x rows/2) with st (cols x rows/16)."""
    rows, cols, ld = _matrix(x)
    _buffer(tensor_scale, "tensor_scale", 3, "f32")
    if q is not None and cols % 16 == 0:
        _buffer(q, "q", rows * (cols // 2), "u8")
        _buffer(s, "s", rows * (cols // 16), "u8")
    if qt is not None and rows % 16 == 0:
        _buffer(qt, "qt", cols * (rows // 2), "u8")
        _buffer(st, "st", cols * (rows // 16), "u8")
    _check(load_library().qsg_quantize_nvfp4(_ptr(x), _dtype_code(x), rows, cols, ld, _ptr(tensor_scale),
                                             _ptr(q), _ptr(s), _ptr(qt), _ptr(st), _stream(stream)))


def qsg_gemm_nvfp4(a, sa, ts_a, b, sb, ts_b, c, stream=None):
    """C (M x N) = s_dec_a s_dec_b (A Sa)(B Sb)^T on NVFP4 operands: a is
    M x K/2 packed bytes, b is N x K/2, sa / sb their E4M3 block scales
    (M x K/16, N x K/16), ts_a / ts_b their 3-float tensor scales (element 2,
    s_dec, is what the library reads)."""
    M, Kh, lda = _matrix(a)
    N, Khb, ldb = _matrix(b)
    if Khb != Kh:
        raise QsgError(f"K mismatch: A has {2 * Kh}, B has {2 * Khb}")
    K = 2 * Kh
    Mc, Nc, ldc = _matrix(c)
    if (Mc, Nc) != (M, N):
        raise QsgError(f"C is {Mc}x{Nc}, expected {M}x{N}")
    _gemm_operands(a, b)
    if K % 16 == 0:
        _buffer(sa, "sa", M * (K // 16), "u8")
        _buffer(sb, "sb", N * (K // 16), "u8")
    _buffer(ts_a, "ts_a", 3, "f32")
    _buffer(ts_b, "ts_b", 3, "f32")
    sdec_a = _ptr(ts_a) + 8 if not isinstance(ts_a, int) else ts_a
    sdec_b = _ptr(ts_b) + 8 if not isinstance(ts_b, int) else ts_b
    _check(load_library().qsg_gemm_nvfp4(_ptr(a), _ptr(sa), sdec_a, _ptr(b), _ptr(sb), sdec_b, M, N, K, lda, ldb,
                                         _ptr(c), _dtype_code(c), ldc, _stream(stream)))
