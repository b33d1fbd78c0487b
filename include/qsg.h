/*
 * qsg.h - FP8 quantization and scaled FP8 GEMM for a transformer Linear
 * layer, on AMD Instinct MI355X (gfx950).  C ABI of libqsg.so.
 *
 * What is computed (the pages that define it):
 *   "Low-Precision Training Guide" (Megatron Core developer guide):
 *     - section "Recipe Reference", recipes "delayed" (scale from a rolling
 *       amax history), "tensorwise" (scale from the current tensor), "mxfp8"
 *       (one power-of-two scale per 1x32 block) and "blockwise" (1x128
 *       activation blocks with 128x128 weight blocks);
 *     - table "Numerical Stability Knobs": --fp8-margin (M bits of headroom
 *       in the scaling factor), --fp8-amax-history-len and
 *       --fp8-amax-compute-algo;
 *     - section "When to Use Low Precision": the FP8 GEMMs.
 *   "How to reduce cuda memory usage of fp8?" (TransformerEngine issue 1764):
 *     the backward pass of a Linear reads a transposed FP8 copy of its input,
 *     hence the fused cast + transpose.
 *   Outside the pages: the FP8 bit layouts of the OCP 8-bit floating point
 *   specification (E4M3 max 448, E5M2 max 57344) and the E8M0 scale byte of
 *   the OCP Microscaling v1.0 specification.
 *
 * Definitions used by every entry point:
 *   enc(v)      saturating round-to-nearest-even FP8 encode of a binary32
 *               value v: finite |v| >= max and +-inf give the signed max code
 *               (0x7E / 0x7B), NaN gives sign|0x7F, the sign of zero is kept.
 *   q = enc(fp32(x * scale))   one binary32 multiply (round to nearest even),
 *               then enc.  bf16 inputs are widened to fp32 exactly first.
 *   scale       fp32(fmax / amax) * 2^-margin; scale_inv = fp32(1 / scale).
 *               amax == 0 or not finite gives scale = 1; a quotient that
 *               overflows gives FLT_MAX.
 *
 * Conventions:
 *   - Every pointer argument named *_dev or naming a tensor is a DEVICE
 *     pointer (memory of the current HIP device).  The caller owns and
 *     allocates every buffer; the library allocates and frees nothing.
 *   - Matrices are row-major: element (r, c) of an R x C matrix with leading
 *     dimension ld is at index r * ld + c.  Inputs take an explicit ld
 *     (ld >= cols); FP8 and scale outputs are dense (ld = their column count).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream), makes no host synchronisation and reads no device value
 *     on the host, so a sequence of calls can be captured in a HIP graph.
 *   - Return value: QSG_OK (0) or a negative qsg_status.  On error nothing
 *     has been launched (argument errors) or a HIP launch error was seen
 *     (QSG_ERR_HIP).  qsg_last_error() gives a message for the calling
 *     thread's last error.
 *   - Shapes with a zero dimension are valid and launch no work except where
 *     a scalar output has to be written (amax = 0 and its scale).
 */
#ifndef QSG_H
#define QSG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSG_OK = 0,
  QSG_ERR_ARG = -1,         /* null pointer, bad enum, negative size, ld < cols */
  QSG_ERR_SHAPE = -2,       /* a shape rule of the recipe is violated */
  QSG_ERR_ALIGN = -3,       /* a pointer is not aligned as the call requires */
  QSG_ERR_UNSUPPORTED = -4, /* valid but unsupported combination */
  QSG_ERR_HIP = -5          /* the HIP runtime reported an error */
} qsg_status;

/* FP8 formats ("Low-Precision Training Guide", table "Hardware and Recipe
 * Compatibility": --fp8-format {e4m3, hybrid}; hybrid = E4M3 for forward
 * tensors and E5M2 for gradients). */
typedef enum { QSG_E4M3 = 0, QSG_E5M2 = 1 } qsg_fp8;

/* Element types of high-precision inputs and of GEMM outputs. */
typedef enum { QSG_F32 = 0, QSG_BF16 = 1 } qsg_dtype;

/* Scaling recipes ("Low-Precision Training Guide", section "Recipe
 * Reference").  For a GEMM operand this names the layout of its scales:
 *   TENSORWISE, DELAYED  one fp32 scale_inv (device pointer to 1 float);
 *   MXFP8                uint8 E8M0 bytes, rows x (K/32), byte = e + 127;
 *   BLOCK_1X128          fp32 scale_inv, rows x (K/128);
 *   BLOCK_128X128        fp32 scale_inv, ceil(rows/128) x (K/128). */
typedef enum {
  QSG_TENSORWISE = 0,
  QSG_DELAYED = 1,
  QSG_MXFP8 = 2,
  QSG_BLOCK_1X128 = 3,
  QSG_BLOCK_128X128 = 4
} qsg_scaling;

/* MXFP8 block-exponent rule.  CEIL (default): the smallest power of two
 * 2^e with block_amax * 2^-e <= fmax, so no element saturates.
 * OCP_FLOOR: e = floor(log2(block_amax)) - emax_elem (OCP MX v1.0), which
 * can saturate elements. */
typedef enum { QSG_MX_CEIL = 0, QSG_MX_OCP_FLOOR = 1 } qsg_mx_rule;

/* amax-history reduction ("--fp8-amax-compute-algo"; only "max" is named). */
typedef enum { QSG_AMAX_MAX = 0 } qsg_amax_algo;

/* A recipe for qsg_quantize.  margin: integer in [0, 64]. */
typedef struct {
  int32_t scaling; /* qsg_scaling */
  int32_t fmt;     /* qsg_fp8 */
  int32_t margin;  /* --fp8-margin */
  int32_t mx_rule; /* qsg_mx_rule, used by QSG_MXFP8 only */
} qsg_recipe;

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int qsg_version(void);

/* Text of a status code (static storage). */
const char* qsg_status_string(int status);

/* Message of the calling thread's last failing call (static per thread). */
const char* qsg_last_error(void);

/* Per-tensor amax ("Low-Precision Training Guide", recipe "tensorwise": the
 * scale is computed from the current tensor).
 *   x        rows x cols, dtype QSG_F32 or QSG_BF16, leading dimension ld;
 *            aligned to its element size (16-byte alignment of x and of
 *            ld * element size selects the vector path).
 *   amax_dev out: 1 float, max |x| (-0 counts as 0; any NaN gives the NaN
 *            0x7FC00000; an empty tensor gives 0).  Written on `stream`. */
int qsg_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
             float* amax_dev, void* stream);

/* Scale from an amax (recipe "tensorwise"; knob --fp8-margin).
 *   amax_dev       in: 1 float.
 *   scale_dev      out: 1 float, scale as defined above.
 *   scale_inv_dev  out: 1 float, fp32(1/scale). */
int qsg_compute_scale(const float* amax_dev, int fmt, int margin, float* scale_dev,
                      float* scale_inv_dev, void* stream);

/* Cast + transpose with a given per-tensor scale ("How to reduce cuda memory
 * usage of fp8?": the transposed FP8 copy that backward reads; recipe
 * "delayed": the amax of the raw tensor is recorded for the next step).
 *   x             rows x cols (dtype, ld), aligned to its element size; the
 *                 vector path needs x and ld * element size 16-byte aligned,
 *                 q 8-byte aligned with cols % 8 == 0, qt 16-byte aligned with
 *                 rows % 16 == 0; otherwise an element-wise path is used.
 *   scale_dev     in: 1 float.
 *   q             out: rows x cols FP8 bytes, or NULL to skip.
 *   qt            out: cols x rows FP8 bytes (qt[c*rows + r] = q[r*cols + c]),
 *                 or NULL to skip.
 *   amax_out_dev  out: 1 float, max |x| of this call (as qsg_amax), or NULL.
 * Either output may be skipped; q and qt may not both be NULL unless the
 * tensor is empty. */
int qsg_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       int fmt, const float* scale_dev, uint8_t* q, uint8_t* qt,
                       float* amax_out_dev, void* stream);

/* Delayed-scaling update ("Low-Precision Training Guide", recipe "delayed":
 * the scaling factor comes from a rolling amax history; knobs
 * --fp8-amax-history-len, --fp8-amax-compute-algo max, --fp8-margin).
 *   history_dev   in/out: hist_len floats (hist_len >= 1); the caller zeroes
 *                 it once before step 0.
 *   step          host counter; amax is written into slot step mod hist_len.
 *   amax_dev      in: 1 float (the amax of the tensor quantized at `step`).
 *   scale_dev, scale_inv_dev  in/out: the scale in force; replaced by the
 *                 scale of max(history), or left unchanged when that max is 0
 *                 or not finite.  The caller sets them to 1 before step 0. */
int qsg_amax_update(float* history_dev, int64_t hist_len, int64_t step,
                    const float* amax_dev, int algo, int fmt, int margin,
                    float* scale_dev, float* scale_inv_dev, void* stream);

/* Bytes of the workspace qsg_cast_transpose_delayed needs (33 lines of 128
 * bytes: per-group maxima and arrival counts, and one common counter). */
#define QSG_DELAYED_WORKSPACE_BYTES 4224

/* One step of delayed scaling for one tensor, in a single kernel launch
 * ("Low-Precision Training Guide", recipe "delayed": the tensor is quantized
 * with the scale derived from earlier steps' amaxes, and its own amax enters a
 * rolling history; knobs --fp8-amax-history-len, --fp8-amax-compute-algo max,
 * --fp8-margin; "How to reduce cuda memory usage of fp8?": the transposed copy
 * that backward reads).  The result is that of
 *     qsg_cast_transpose(x, ..., fmt, scale_dev, q, qt, amax_out_dev)
 *     qsg_amax_update(history_dev, hist_len, step, amax, QSG_AMAX_MAX, fmt,
 *                     margin, scale_dev, scale_inv_dev)
 * with the amax passed between the two kept in `workspace`:
 *   x, dtype, rows, cols, ld, fmt, q, qt   as qsg_cast_transpose (q, qt may
 *                 not both be NULL unless the tensor is empty); q and qt are
 *                 written with the scale in force at entry.
 *   margin        --fp8-margin, in [0, 64].
 *   history_dev, hist_len, step, scale_dev, scale_inv_dev   as
 *                 qsg_amax_update: on return *scale_dev / *scale_inv_dev hold
 *                 the scale for the next step (unchanged when the window max
 *                 is 0 or not finite).
 *   amax_out_dev  out: 1 float, max |x| of this call (as qsg_amax), or NULL.
 *   workspace     device memory of QSG_DELAYED_WORKSPACE_BYTES bytes, 4-byte
 *                 aligned (128-byte alignment keeps each counter on its own
 *                 cache line), owned by the caller, zero before its first use;
 *                 every call leaves it zero again.  Calls that share one
 *                 workspace must not overlap (same stream, or ordered).
 * The last workgroup of the launch does the history update, so no second
 * kernel and no host synchronisation is needed. */
int qsg_cast_transpose_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                               int margin, float* history_dev, int64_t hist_len, int64_t step,
                               float* scale_dev, float* scale_inv_dev, uint8_t* q, uint8_t* qt,
                               float* amax_out_dev, void* workspace, void* stream);

/* qsg_cast_transpose_delayed for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without `workspace`.  The
 * library keeps the workspace in a file-scope device array of
 * QSG_DELAYED_WORKSPACE_BYTES bytes, one copy per GPU, held until the process
 * ends; its address is looked up on the first call on each device (that call
 * also clears it), and every call leaves it zero.  The workspace need does not
 * grow with the tensor, so no size is rejected for lack of scratch.  Calls on
 * one GPU share the array: calls that overlap in time on one GPU (different
 * streams without ordering) race and must not be issued.  Nothing is
 * allocated or freed; a failed address lookup returns QSG_ERR_HIP. */
int qsg_cast_transpose_delayed_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                       int margin, float* history_dev, int64_t hist_len, int64_t step,
                                       float* scale_dev, float* scale_inv_dev, uint8_t* q, uint8_t* qt,
                                       float* amax_out_dev, void* stream);

/* FP8 store of the MLP activation's input, forward ("Benefits of Using FP8
 * Precision with MegaDLMs and Required Hardware", configuration field
 * activation_func_fp8_input_store: the activation's input is kept in FP8 for
 * backpropagation).  The activation is GeLU, gelu(h) = h * Phi(h) with Phi the
 * standard normal CDF (erf form; the pages do not name the function).
 *   h             rows x cols bf16, leading dimension ld (2-byte aligned; the
 *                 vector path needs h, a 16-byte and q 8-byte aligned with ld
 *                 and cols multiples of 8).
 *   scale_dev     in: 1 float, the per-tensor scale of the stored input.
 *   a             out: rows x cols bf16 (dense), bf16(gelu(h)) rounded to
 *                 nearest even from a binary32 evaluation.
 *   q             out: rows x cols FP8 bytes (dense), enc(fp32(h * scale)).
 *   amax_out_dev  out: 1 float, max |h| (as qsg_amax, for delayed scaling of
 *                 the stored input), or NULL.
 * The caller owns every buffer; nothing is allocated. */
int qsg_act_fp8_store_fwd(const void* h, int64_t rows, int64_t cols, int64_t ld, int fmt,
                          const float* scale_dev, void* a, uint8_t* q, float* amax_out_dev,
                          void* stream);

/* Backward of the above: the activation's gradient from the stored FP8 input.
 *   da            rows x cols bf16 (ld), the gradient of a.
 *   q             rows x cols FP8 bytes (dense) in format fmt, as written by
 *                 qsg_act_fp8_store_fwd.
 *   scale_inv_dev in: 1 float; the input is recovered as h' = fp32(dec(q) * scale_inv).
 *   dh            out: rows x cols bf16 (dense), bf16(da * gelu'(h')) with
 *                 gelu'(h) = Phi(h) + h phi(h), phi the standard normal density. */
int qsg_act_fp8_store_bwd(const void* da, int64_t rows, int64_t cols, int64_t ld, int fmt,
                          const uint8_t* q, const float* scale_inv_dev, void* dh, void* stream);

/* Weight-gradient GEMM kept in bf16 ("Low-Precision Training Guide", knob
 * --fp8-wgrad False: wgrad in higher precision while fprop and dgrad use FP8):
 *
 *     C[n, k] = sum_t dY[t, n] * X[t, k]      (accumulate = 0)
 *     C[n, k] = fp32(C[n, k] + sum_t ...)     (accumulate = 1, fp32 C only:
 *                                              the fp32 main gradient)
 *
 *   dy  T x N bf16 (tokens x output features), leading dimension lddy;
 *   x   T x K bf16 (tokens x input features), leading dimension ldx; both
 *       2-byte aligned.  The fast path needs 16-byte aligned rows (bases
 *       16-byte aligned, lddy and ldx multiples of 8 and below 2^24) and N,
 *       K multiples of 8; other operands take a slower general path with the
 *       same results;
 *   c   N x K, ldc, c_dtype QSG_BF16 (rounded to nearest even) or QSG_F32,
 *       aligned to its element size; products of bf16 values are exact in
 *       fp32 and are summed in fp32.
 * T == 0 writes zeros (or adds +0).  Accumulation into bf16 returns
 * QSG_ERR_UNSUPPORTED. */
int qsg_wgrad_bf16(const void* dy, int64_t T, int64_t N, int64_t lddy, const void* x, int64_t K,
                   int64_t ldx, void* c, int c_dtype, int64_t ldc, int accumulate, void* stream);

/* Quantize one tensor under a recipe, producing the row-wise copy (blocks run
 * along cols, the GEMM contraction dimension of the tensor as stored) and/or
 * the column-wise copy (blocks run along rows, stored transposed so that it
 * is the row-wise quantization of x^T).
 *
 *   QSG_TENSORWISE  amax, scale and cast + transpose in one call.
 *                   s  out: 3 floats {amax, scale, scale_inv}; st unused.
 *   QSG_MXFP8       ("mxfp8": 1x32 blocks, power-of-two E8M0 scales)
 *                   q  rows x cols, s  uint8 rows x (cols/32);   cols % 32 == 0
 *                   qt cols x rows, st uint8 cols x (rows/32);   rows % 32 == 0
 *   QSG_BLOCK_1X128 ("blockwise" activations)
 *                   q  rows x cols, s  fp32 rows x (cols/128);   cols % 128 == 0
 *                   qt cols x rows, st fp32 cols x (rows/128);   rows % 128 == 0
 *   QSG_BLOCK_128X128 ("blockwise" weights)
 *                   q  rows x cols, s  fp32 (rows/128) x (cols/128);
 *                   qt = q^T, st = s^T;  rows % 128 == 0, cols % 128 == 0
 * Scale tensors hold scale_inv (what the GEMM multiplies by) except MXFP8,
 * which holds E8M0 bytes.  Pass NULL for (q, s) or (qt, st) to skip that
 * copy.  QSG_DELAYED is not accepted here (use qsg_cast_transpose and
 * qsg_amax_update). */
int qsg_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 const qsg_recipe* recipe, uint8_t* q, void* s, uint8_t* qt, void* st,
                 void* stream);

/* Scaled FP8 GEMM ("Low-Precision Training Guide", section "When to Use Low
 * Precision": the FP8 GEMMs of a Linear; recipes "mxfp8" and "blockwise" for
 * the scale granularity):
 *
 *     C[m, n] = sum_k (A[m, k] * sa(m, k)) * (B[n, k] * sb(n, k))
 *
 * A is M x K (lda), B is N x K (ldb): both K-contiguous FP8 bytes in formats
 * fa / fb.  C is M x N (ldc) in c_dtype (QSG_BF16, rounded to nearest even,
 * or QSG_F32), accumulated in fp32.  fprop, dgrad and wgrad all take this
 * form by passing the transposed FP8 copies (dgrad: A = Q(dY), B = Q(W)^T;
 * wgrad: A = Q(dY)^T, B = Q(X)^T).
 * Scale kinds (ka, kb) and their pointers (see qsg_scaling):
 *   (TENSORWISE|DELAYED, TENSORWISE|DELAYED)  1 float each
 *   (MXFP8, MXFP8)                            K % 32 == 0
 *   (BLOCK_1X128, BLOCK_128X128)              fprop / dgrad, K % 128 == 0
 *   (BLOCK_1X128, BLOCK_1X128)                wgrad, K % 128 == 0
 * Other pairs return QSG_ERR_UNSUPPORTED.  C must be aligned to its element
 * size.  The vector path needs A and B 16-byte aligned with lda and ldb
 * multiples of 16 (else A and B are read byte by byte), and C 8-byte (bf16)
 * or 16-byte (fp32) aligned with ldc a multiple of 4 (else C is written
 * element by element). */
int qsg_scaled_gemm(const uint8_t* a, int fa, int ka, const void* sa,
                    const uint8_t* b, int fb, int kb, const void* sb,
                    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                    void* c, int c_dtype, int64_t ldc, void* stream);

/* Scaled FP8 GEMM accumulated into an fp32 matrix: the weight-gradient
 * accumulation into fp32 main gradients ("Low-Precision Training Guide",
 * precision-aware optimizer knob --main-grads-dtype fp32; --fp8-wgrad keeps
 * the wgrad GEMM itself in FP8):
 *
 *     C[m, n] = fp32(C[m, n] + r[m, n]),
 *     r[m, n] = the fp32 result qsg_scaled_gemm would write (before any
 *               output rounding to bf16),
 *
 * one binary32 addition per element, so micro-batch after micro-batch the
 * gradient accumulates in C.  Arguments, scale kinds, shapes and alignment
 * rules are those of qsg_scaled_gemm with c_dtype = QSG_F32; C (M x N, ldc,
 * 4-byte aligned, caller-owned) is read and written in place.  K == 0 adds
 * +0.  C must not overlap A, B or the scales. */
int qsg_scaled_gemm_accumulate(const uint8_t* a, int fa, int ka, const void* sa,
                               const uint8_t* b, int fb, int kb, const void* sb,
                               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                               float* c, int64_t ldc, void* stream);

/* NVFP4 block scaling ("Low-Precision Training Guide": recipe "nvfp4",
 * "NVFP4 block scaling", --fp4-format e2m1; table "Hardware and Recipe
 * Compatibility", row nvfp4).  The pages name the element format only; the
 * block size and the scale formats follow NVIDIA's NVFP4 definition, outside
 * the pages: 16 consecutive elements along a row share one E4M3 decode scale
 * byte, and the tensor has one fp32 scale
 *     s_enc = fp32(448 * 6 / amax)   (1 for amax 0 or not finite, FLT_MAX
 *                                      when the quotient overflows),
 *     s_dec = fp32(1 / s_enc).
 * A block with maximum |x| = b is quantized with one binary32 operation per
 * step, each rounded to nearest even:
 *     S    = dec(E4M3(fp32(fp32(b / 6) * s_enc)))   (saturating RNE E4M3)
 *     m    = fp32(s_enc / S), or 0 when S is 0 or the scale byte is NaN
 *     code = E2M1(fp32(x * m))
 * E2M1 (OCP FP4): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit;
 * saturating round to nearest, a midpoint going to the even code; the sign
 * of zero is kept; NaN gives sign | 6.  The value represented is
 * dec(code) * S * s_dec.
 *
 * tensor_scale_dev  out: 3 floats {amax, s_enc, s_dec} (device).
 * q   rows x (cols/2) bytes, two codes per byte along the row, element 2i in
 *     the low nibble;  s  rows x (cols/16) E4M3 bytes;       cols % 16 == 0.
 * qt  cols x (rows/2) bytes: the column-wise copy (blocks of 16 rows, stored
 *     transposed, same packing);  st  cols x (rows/16);      rows % 16 == 0.
 * Pass NULL for (q, s) or (qt, st) to skip a copy.  q and qt must be 4-byte
 * aligned.  An empty matrix writes {0, 1, 1} to tensor_scale_dev only. */
int qsg_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       float* tensor_scale_dev, uint8_t* q, uint8_t* s, uint8_t* qt, uint8_t* st,
                       void* stream);

/* GEMM on NVFP4 operands (same pages and definition as qsg_quantize_nvfp4):
 *
 *     C[m, n] = (s_dec_a * s_dec_b) * sum_k (dec(A[m, k]) * Sa(m, k / 16))
 *                                         * (dec(B[n, k]) * Sb(n, k / 16))
 *
 * A is M x K codes packed as qsg_quantize_nvfp4 writes them (lda bytes per
 * row, lda >= K/2), B is N x K (ldb); sa (M x K/16) and sb (N x K/16) are
 * their dense E4M3 block-scale bytes; sdec_a_dev / sdec_b_dev point at the
 * s_dec float of each operand (element 2 of its tensor_scale).  K % 16 == 0.
 * Each block-scaled value is exact in bfloat16; products are exact and are
 * summed in fp32.  C is M x N (ldc) in c_dtype (QSG_BF16 rounded to nearest
 * even, or QSG_F32), aligned to its element size; fprop, dgrad and wgrad take
 * this form with the row-wise or column-wise copies as for qsg_scaled_gemm.
 * The vector path needs A and B 16-byte aligned with lda, ldb multiples of
 * 16 (else bytes are read one by one).  K == 0 writes zeros. */
int qsg_gemm_nvfp4(const uint8_t* a, const uint8_t* sa, const float* sdec_a_dev,
                   const uint8_t* b, const uint8_t* sb, const float* sdec_b_dev,
                   int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                   void* c, int c_dtype, int64_t ldc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSG_H */
