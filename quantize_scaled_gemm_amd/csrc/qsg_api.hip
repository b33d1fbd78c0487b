// C ABI of libqsg.so (declared in include/qsg.h): argument validation, then
// the launchers.  No exception crosses this boundary; nothing here allocates
// device memory or synchronises with the device.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "qsg.h"
#include "qsg_internal.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QSG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return QSG_OK;
}

bool valid_fmt(int f) { return f == QSG_E4M3 || f == QSG_E5M2; }
bool valid_dtype(int d) { return d == QSG_F32 || d == QSG_BF16; }
int esize(int dtype) { return dtype == QSG_BF16 ? 2 : 4; }
bool aligned(const void* p, int n) { return ((uintptr_t)p % (uintptr_t)n) == 0; }

int check_matrix(const char* fn, const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld) {
  if (!valid_dtype(dtype)) return fail(QSG_ERR_ARG, "%s: bad dtype %d", fn, dtype);
  if (rows < 0 || cols < 0) return fail(QSG_ERR_ARG, "%s: negative shape %lld x %lld", fn, (long long)rows, (long long)cols);
  if (rows > 0 && cols > 0) {
    if (!x) return fail(QSG_ERR_ARG, "%s: null input", fn);
    if (ld < cols) return fail(QSG_ERR_ARG, "%s: ld %lld < cols %lld", fn, (long long)ld, (long long)cols);
    if (!aligned(x, esize(dtype))) return fail(QSG_ERR_ALIGN, "%s: input not aligned to its element size", fn);
  }
  return QSG_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int qsg_version(void) { return 100; }

const char* qsg_status_string(int status) {
  switch (status) {
    case QSG_OK: return "ok";
    case QSG_ERR_ARG: return "invalid argument";
    case QSG_ERR_SHAPE: return "shape not allowed by the recipe";
    case QSG_ERR_ALIGN: return "misaligned pointer";
    case QSG_ERR_UNSUPPORTED: return "unsupported combination";
    case QSG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qsg_last_error(void) { return g_msg; }

int qsg_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* amax_dev,
             void* stream) {
  int rc = check_matrix("qsg_amax", x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!amax_dev) return fail(QSG_ERR_ARG, "qsg_amax: null amax");
  if (!aligned(amax_dev, 4)) return fail(QSG_ERR_ALIGN, "qsg_amax: amax not 4-byte aligned");
  qsg::launch_amax(x, dtype, rows, cols, ld, amax_dev, as_stream(stream));
  return check_launch("qsg_amax");
}

int qsg_compute_scale(const float* amax_dev, int fmt, int margin, float* scale_dev,
                      float* scale_inv_dev, void* stream) {
  if (!amax_dev || !scale_dev || !scale_inv_dev) return fail(QSG_ERR_ARG, "qsg_compute_scale: null pointer");
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "qsg_compute_scale: bad fmt %d", fmt);
  if (margin < 0 || margin > 64) return fail(QSG_ERR_ARG, "qsg_compute_scale: margin %d outside [0, 64]", margin);
  qsg::launch_compute_scale(amax_dev, fmt, margin, scale_dev, scale_inv_dev, as_stream(stream));
  return check_launch("qsg_compute_scale");
}

int qsg_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                       const float* scale_dev, uint8_t* q, uint8_t* qt, float* amax_out_dev,
                       void* stream) {
  int rc = check_matrix("qsg_cast_transpose", x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "qsg_cast_transpose: bad fmt %d", fmt);
  if (!scale_dev) return fail(QSG_ERR_ARG, "qsg_cast_transpose: null scale");
  const bool empty = rows == 0 || cols == 0;
  if (!q && !qt && !empty) return fail(QSG_ERR_ARG, "qsg_cast_transpose: q and qt are both null");
  if (amax_out_dev && !aligned(amax_out_dev, 4)) return fail(QSG_ERR_ALIGN, "qsg_cast_transpose: amax_out not aligned");
  qsg::launch_cast_transpose(x, dtype, rows, cols, ld, fmt, scale_dev, q, qt, amax_out_dev, as_stream(stream));
  return check_launch("qsg_cast_transpose");
}

int qsg_cast_transpose_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                               int margin, float* history_dev, int64_t hist_len, int64_t step,
                               float* scale_dev, float* scale_inv_dev, uint8_t* q, uint8_t* qt,
                               float* amax_out_dev, void* workspace, void* stream) {
  const char* fn = "qsg_cast_transpose_delayed";
  int rc = check_matrix(fn, x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "%s: bad fmt %d", fn, fmt);
  if (margin < 0 || margin > 64) return fail(QSG_ERR_ARG, "%s: margin %d outside [0, 64]", fn, margin);
  if (!history_dev || !scale_dev || !scale_inv_dev || !workspace) return fail(QSG_ERR_ARG, "%s: null pointer", fn);
  if (hist_len < 1) return fail(QSG_ERR_ARG, "%s: hist_len %lld < 1", fn, (long long)hist_len);
  if (step < 0) return fail(QSG_ERR_ARG, "%s: negative step", fn);
  const bool empty = rows == 0 || cols == 0;
  if (!q && !qt && !empty) return fail(QSG_ERR_ARG, "%s: q and qt are both null", fn);
  if (!aligned(workspace, 4)) return fail(QSG_ERR_ALIGN, "%s: workspace not 4-byte aligned", fn);
  if (amax_out_dev && !aligned(amax_out_dev, 4)) return fail(QSG_ERR_ALIGN, "%s: amax_out not aligned", fn);
  qsg::launch_cast_transpose_delayed(x, dtype, rows, cols, ld, fmt, margin, history_dev, hist_len, step, scale_dev,
                                     scale_inv_dev, q, qt, amax_out_dev, reinterpret_cast<uint32_t*>(workspace),
                                     as_stream(stream));
  return check_launch(fn);
}

int qsg_cast_transpose_delayed_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                       int margin, float* history_dev, int64_t hist_len, int64_t step,
                                       float* scale_dev, float* scale_inv_dev, uint8_t* q, uint8_t* qt,
                                       float* amax_out_dev, void* stream) {
  const char* fn = "qsg_cast_transpose_delayed_noalloc";
  int rc = check_matrix(fn, x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "%s: bad fmt %d", fn, fmt);
  if (margin < 0 || margin > 64) return fail(QSG_ERR_ARG, "%s: margin %d outside [0, 64]", fn, margin);
  if (!history_dev || !scale_dev || !scale_inv_dev) return fail(QSG_ERR_ARG, "%s: null pointer", fn);
  if (hist_len < 1) return fail(QSG_ERR_ARG, "%s: hist_len %lld < 1", fn, (long long)hist_len);
  if (step < 0) return fail(QSG_ERR_ARG, "%s: negative step", fn);
  const bool empty = rows == 0 || cols == 0;
  if (!q && !qt && !empty) return fail(QSG_ERR_ARG, "%s: q and qt are both null", fn);
  if (amax_out_dev && !aligned(amax_out_dev, 4)) return fail(QSG_ERR_ALIGN, "%s: amax_out not aligned", fn);
  uint32_t* ws = nullptr;
  if (qsg::delayed_scratch(&ws, as_stream(stream)) != 0)
    return fail(QSG_ERR_HIP, "%s: the device address of the library's scratch array could not be found", fn);
  qsg::launch_cast_transpose_delayed(x, dtype, rows, cols, ld, fmt, margin, history_dev, hist_len, step, scale_dev,
                                     scale_inv_dev, q, qt, amax_out_dev, ws, as_stream(stream));
  return check_launch(fn);
}

int qsg_act_fp8_store_fwd(const void* h, int64_t rows, int64_t cols, int64_t ld, int fmt, const float* scale_dev,
                          void* a, uint8_t* q, float* amax_out_dev, void* stream) {
  const char* fn = "qsg_act_fp8_store_fwd";
  int rc = check_matrix(fn, h, QSG_BF16, rows, cols, ld);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "%s: bad fmt %d", fn, fmt);
  if (!scale_dev) return fail(QSG_ERR_ARG, "%s: null scale", fn);
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!a || !q)) return fail(QSG_ERR_ARG, "%s: null output", fn);
  if (a && !aligned(a, 2)) return fail(QSG_ERR_ALIGN, "%s: a not aligned to 2 bytes", fn);
  if (amax_out_dev && !aligned(amax_out_dev, 4)) return fail(QSG_ERR_ALIGN, "%s: amax_out not aligned", fn);
  qsg::launch_act_fp8_store_fwd(h, rows, cols, ld, fmt, scale_dev, a, q, amax_out_dev, as_stream(stream));
  return check_launch(fn);
}

int qsg_act_fp8_store_bwd(const void* da, int64_t rows, int64_t cols, int64_t ld, int fmt, const uint8_t* q,
                          const float* scale_inv_dev, void* dh, void* stream) {
  const char* fn = "qsg_act_fp8_store_bwd";
  int rc = check_matrix(fn, da, QSG_BF16, rows, cols, ld);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "%s: bad fmt %d", fn, fmt);
  if (!scale_inv_dev) return fail(QSG_ERR_ARG, "%s: null scale_inv", fn);
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (!q || !dh)) return fail(QSG_ERR_ARG, "%s: null q or dh", fn);
  if (dh && !aligned(dh, 2)) return fail(QSG_ERR_ALIGN, "%s: dh not aligned to 2 bytes", fn);
  qsg::launch_act_fp8_store_bwd(da, rows, cols, ld, fmt, q, scale_inv_dev, dh, as_stream(stream));
  return check_launch(fn);
}

int qsg_wgrad_bf16(const void* dy, int64_t T, int64_t N, int64_t lddy, const void* x, int64_t K, int64_t ldx,
                   void* c, int c_dtype, int64_t ldc, int accumulate, void* stream) {
  const char* fn = "qsg_wgrad_bf16";
  if (!valid_dtype(c_dtype)) return fail(QSG_ERR_ARG, "%s: bad output dtype", fn);
  if (T < 0 || N < 0 || K < 0) return fail(QSG_ERR_ARG, "%s: negative shape", fn);
  if (accumulate && c_dtype != QSG_F32) return fail(QSG_ERR_UNSUPPORTED, "%s: accumulation needs an fp32 C", fn);
  if (N == 0 || K == 0) return QSG_OK;
  if (!c) return fail(QSG_ERR_ARG, "%s: null C", fn);
  if (ldc < K) return fail(QSG_ERR_ARG, "%s: ldc < K", fn);
  if (!aligned(c, c_dtype == QSG_BF16 ? 2 : 4)) return fail(QSG_ERR_ALIGN, "%s: C not aligned to its element size", fn);
  if (T > 0) {
    if (!dy || !x) return fail(QSG_ERR_ARG, "%s: null operand", fn);
    if (lddy < N || ldx < K) return fail(QSG_ERR_ARG, "%s: lddy < N or ldx < K", fn);
    if (!aligned(dy, 2) || !aligned(x, 2)) return fail(QSG_ERR_ALIGN, "%s: operands not aligned to 2 bytes", fn);
  }
  qsg::launch_wgrad_bf16(dy, T, N, lddy, x, K, ldx, c, c_dtype, ldc, accumulate != 0, as_stream(stream));
  return check_launch(fn);
}

int qsg_amax_update(float* history_dev, int64_t hist_len, int64_t step, const float* amax_dev,
                    int algo, int fmt, int margin, float* scale_dev, float* scale_inv_dev,
                    void* stream) {
  if (!history_dev || !amax_dev || !scale_dev || !scale_inv_dev) return fail(QSG_ERR_ARG, "qsg_amax_update: null pointer");
  if (hist_len < 1) return fail(QSG_ERR_ARG, "qsg_amax_update: hist_len %lld < 1", (long long)hist_len);
  if (step < 0) return fail(QSG_ERR_ARG, "qsg_amax_update: negative step");
  if (algo != QSG_AMAX_MAX) return fail(QSG_ERR_UNSUPPORTED, "qsg_amax_update: only the max algorithm is defined");
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "qsg_amax_update: bad fmt %d", fmt);
  if (margin < 0 || margin > 64) return fail(QSG_ERR_ARG, "qsg_amax_update: margin %d outside [0, 64]", margin);
  qsg::launch_amax_update(history_dev, hist_len, step, amax_dev, fmt, margin, scale_dev, scale_inv_dev,
                          as_stream(stream));
  return check_launch("qsg_amax_update");
}

int qsg_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 const qsg_recipe* recipe, uint8_t* q, void* s, uint8_t* qt, void* st, void* stream) {
  const char* fn = "qsg_quantize";
  int rc = check_matrix(fn, x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!recipe) return fail(QSG_ERR_ARG, "%s: null recipe", fn);
  const int scaling = recipe->scaling, fmt = recipe->fmt, margin = recipe->margin;
  if (!valid_fmt(fmt)) return fail(QSG_ERR_ARG, "%s: bad fmt %d", fn, fmt);
  if (margin < 0 || margin > 64) return fail(QSG_ERR_ARG, "%s: margin %d outside [0, 64]", fn, margin);
  hipStream_t hs = as_stream(stream);
  if (scaling == QSG_TENSORWISE) {
    if (!s) return fail(QSG_ERR_ARG, "%s: tensorwise needs s = {amax, scale, scale_inv}", fn);
    if (!q && !qt && rows > 0 && cols > 0) return fail(QSG_ERR_ARG, "%s: q and qt are both null", fn);
    if (!aligned(s, 4)) return fail(QSG_ERR_ALIGN, "%s: s not aligned", fn);
    float* f = reinterpret_cast<float*>(s);
    qsg::launch_amax(x, dtype, rows, cols, ld, f, hs);
    qsg::launch_compute_scale(f, fmt, margin, f + 1, f + 2, hs);
    qsg::launch_cast_transpose(x, dtype, rows, cols, ld, fmt, f + 1, q, qt, nullptr, hs);
    return check_launch(fn);
  }
  if (scaling == QSG_DELAYED)
    return fail(QSG_ERR_UNSUPPORTED, "%s: delayed scaling uses qsg_cast_transpose + qsg_amax_update", fn);
  if (scaling != QSG_MXFP8 && scaling != QSG_BLOCK_1X128 && scaling != QSG_BLOCK_128X128)
    return fail(QSG_ERR_ARG, "%s: bad scaling %d", fn, scaling);
  if (scaling == QSG_MXFP8 && recipe->mx_rule != QSG_MX_CEIL && recipe->mx_rule != QSG_MX_OCP_FLOOR)
    return fail(QSG_ERR_ARG, "%s: bad mx_rule %d", fn, recipe->mx_rule);
  if (rows == 0 || cols == 0) return QSG_OK;  // nothing to quantize, no scale to write
  const bool row = q != nullptr, col = qt != nullptr;
  if (!row && !col) return fail(QSG_ERR_ARG, "%s: q and qt are both null", fn);
  if ((row && !s) || (col && !st)) return fail(QSG_ERR_ARG, "%s: a requested copy has a null scale tensor", fn);
  if (scaling != QSG_MXFP8) {
    if ((s && !aligned(s, 4)) || (st && !aligned(st, 4))) return fail(QSG_ERR_ALIGN, "%s: fp32 scales not aligned", fn);
  }
  const int64_t B = scaling == QSG_MXFP8 ? 32 : 128;
  if (scaling == QSG_BLOCK_128X128) {
    if (rows % 128 || cols % 128)
      return fail(QSG_ERR_SHAPE, "%s: 128x128 blocks need rows and cols multiples of 128 (%lld x %lld)", fn,
                  (long long)rows, (long long)cols);
  } else {
    if (row && cols % B)
      return fail(QSG_ERR_SHAPE, "%s: row-wise blocks need cols %% %lld == 0 (cols %lld)", fn, (long long)B, (long long)cols);
    if (col && rows % B)
      return fail(QSG_ERR_SHAPE, "%s: column-wise blocks need rows %% %lld == 0 (rows %lld)", fn, (long long)B, (long long)rows);
  }
  qsg::launch_quantize_blocked(x, dtype, rows, cols, ld, scaling, fmt, margin,
                               recipe->mx_rule == QSG_MX_CEIL, q, s, qt, st, hs);
  return check_launch(fn);
}

static int scaled_gemm(const char* fn, const uint8_t* a, int fa, int ka, const void* sa, const uint8_t* b,
                       int fb, int kb, const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda,
                       int64_t ldb, void* c, int c_dtype, int64_t ldc, bool accumulate, void* stream) {
  if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(QSG_ERR_ARG, "%s: bad fp8 format", fn);
  if (!valid_dtype(c_dtype)) return fail(QSG_ERR_ARG, "%s: bad output dtype", fn);
  if (M < 0 || N < 0 || K < 0) return fail(QSG_ERR_ARG, "%s: negative shape", fn);
  const bool pt_a = ka == QSG_TENSORWISE || ka == QSG_DELAYED;
  const bool pt_b = kb == QSG_TENSORWISE || kb == QSG_DELAYED;
  int mode;
  if (pt_a && pt_b) mode = 0;
  else if (ka == QSG_MXFP8 && kb == QSG_MXFP8) mode = 1;
  else if (ka == QSG_BLOCK_1X128 && kb == QSG_BLOCK_128X128) mode = 2;
  else if (ka == QSG_BLOCK_1X128 && kb == QSG_BLOCK_1X128) mode = 3;
  else {
    const bool known = (ka >= 0 && ka <= 4) && (kb >= 0 && kb <= 4);
    return fail(known ? QSG_ERR_UNSUPPORTED : QSG_ERR_ARG, "%s: scale kinds (%d, %d) not supported", fn, ka, kb);
  }
  if (mode == 1 && K % 32) return fail(QSG_ERR_SHAPE, "%s: MXFP8 needs K %% 32 == 0 (K %lld)", fn, (long long)K);
  if ((mode == 2 || mode == 3) && K % 128) return fail(QSG_ERR_SHAPE, "%s: blockwise needs K %% 128 == 0 (K %lld)", fn, (long long)K);
  if (M == 0 || N == 0) return QSG_OK;
  if (!c) return fail(QSG_ERR_ARG, "%s: null C", fn);
  if (ldc < N) return fail(QSG_ERR_ARG, "%s: ldc < N", fn);
  if (!aligned(c, c_dtype == QSG_BF16 ? 2 : 4)) return fail(QSG_ERR_ALIGN, "%s: C not aligned to its element size", fn);
  if (K > 0) {
    if (!a || !b) return fail(QSG_ERR_ARG, "%s: null operand", fn);
    if (lda < K || ldb < K) return fail(QSG_ERR_ARG, "%s: lda/ldb < K", fn);
  }
  if (!sa || !sb) return fail(QSG_ERR_ARG, "%s: null scale", fn);
  if (mode != 1 && (!aligned(sa, 4) || !aligned(sb, 4))) return fail(QSG_ERR_ALIGN, "%s: fp32 scales not aligned", fn);
  qsg::launch_scaled_gemm(a, fa, ka, sa, b, fb, kb, sb, M, N, K, lda, ldb, c, c_dtype, ldc, accumulate,
                          as_stream(stream));
  return check_launch(fn);
}

int qsg_scaled_gemm(const uint8_t* a, int fa, int ka, const void* sa, const uint8_t* b, int fb,
                    int kb, const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda,
                    int64_t ldb, void* c, int c_dtype, int64_t ldc, void* stream) {
  return scaled_gemm("qsg_scaled_gemm", a, fa, ka, sa, b, fb, kb, sb, M, N, K, lda, ldb, c, c_dtype, ldc, false,
                     stream);
}

int qsg_scaled_gemm_accumulate(const uint8_t* a, int fa, int ka, const void* sa, const uint8_t* b, int fb,
                               int kb, const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda,
                               int64_t ldb, float* c, int64_t ldc, void* stream) {
  return scaled_gemm("qsg_scaled_gemm_accumulate", a, fa, ka, sa, b, fb, kb, sb, M, N, K, lda, ldb, c, QSG_F32,
                     ldc, true, stream);
}

int qsg_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* tensor_scale_dev,
                       uint8_t* q, uint8_t* s, uint8_t* qt, uint8_t* st, void* stream) {
  const char* fn = "qsg_quantize_nvfp4";
  int rc = check_matrix(fn, x, dtype, rows, cols, ld);
  if (rc) return rc;
  if (!tensor_scale_dev) return fail(QSG_ERR_ARG, "%s: null tensor_scale", fn);
  if (!aligned(tensor_scale_dev, 4)) return fail(QSG_ERR_ALIGN, "%s: tensor_scale not 4-byte aligned", fn);
  const bool empty = rows == 0 || cols == 0;
  const bool row = q != nullptr, col = qt != nullptr;
  if (!row && !col && !empty) return fail(QSG_ERR_ARG, "%s: q and qt are both null", fn);
  if ((row && !s) || (col && !st)) return fail(QSG_ERR_ARG, "%s: a requested copy has a null scale tensor", fn);
  if ((q && !aligned(q, 4)) || (qt && !aligned(qt, 4))) return fail(QSG_ERR_ALIGN, "%s: q / qt not 4-byte aligned", fn);
  if (row && cols % 16)
    return fail(QSG_ERR_SHAPE, "%s: row-wise blocks need cols %% 16 == 0 (cols %lld)", fn, (long long)cols);
  if (col && rows % 16)
    return fail(QSG_ERR_SHAPE, "%s: column-wise blocks need rows %% 16 == 0 (rows %lld)", fn, (long long)rows);
  qsg::launch_quantize_nvfp4(x, dtype, rows, cols, ld, q, s, qt, st, tensor_scale_dev, as_stream(stream));
  return check_launch(fn);
}

int qsg_gemm_nvfp4(const uint8_t* a, const uint8_t* sa, const float* sdec_a_dev, const uint8_t* b, const uint8_t* sb,
                   const float* sdec_b_dev, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                   int c_dtype, int64_t ldc, void* stream) {
  const char* fn = "qsg_gemm_nvfp4";
  if (!valid_dtype(c_dtype)) return fail(QSG_ERR_ARG, "%s: bad output dtype", fn);
  if (M < 0 || N < 0 || K < 0) return fail(QSG_ERR_ARG, "%s: negative shape", fn);
  if (K % 16) return fail(QSG_ERR_SHAPE, "%s: NVFP4 needs K %% 16 == 0 (K %lld)", fn, (long long)K);
  if (M == 0 || N == 0) return QSG_OK;
  if ((M + 127) / 128 > 65535 || (N + 127) / 128 > 0x7FFFFFFF)
    return fail(QSG_ERR_UNSUPPORTED, "%s: M %lld exceeds 65535 tiles of 128 rows", fn, (long long)M);
  if (!c) return fail(QSG_ERR_ARG, "%s: null C", fn);
  if (ldc < N) return fail(QSG_ERR_ARG, "%s: ldc < N", fn);
  if (!aligned(c, c_dtype == QSG_BF16 ? 2 : 4)) return fail(QSG_ERR_ALIGN, "%s: C not aligned to its element size", fn);
  if (!sdec_a_dev || !sdec_b_dev) return fail(QSG_ERR_ARG, "%s: null tensor scale", fn);
  if (!aligned(sdec_a_dev, 4) || !aligned(sdec_b_dev, 4)) return fail(QSG_ERR_ALIGN, "%s: tensor scales not aligned", fn);
  if (K > 0) {
    if (!a || !b || !sa || !sb) return fail(QSG_ERR_ARG, "%s: null operand or block scales", fn);
    if (lda < K / 2 || ldb < K / 2) return fail(QSG_ERR_ARG, "%s: lda/ldb < K/2 bytes", fn);
  }
  qsg::launch_gemm_nvfp4(a, sa, sdec_a_dev, b, sb, sdec_b_dev, M, N, K, lda, ldb, c, c_dtype, ldc, as_stream(stream));
  return check_launch(fn);
}

}  // extern "C"
