// Internal launchers behind the C ABI.  Arguments have been validated by the
// caller (qsg_api.hip); every launcher only enqueues work on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsg {

void launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t st);
void launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* amax,
                 hipStream_t st);
void launch_compute_scale(const float* amax, int fmt, int margin, float* scale, float* scale_inv,
                          hipStream_t st);
void launch_amax_update(float* history, int64_t L, int64_t step, const float* amax, int fmt,
                        int margin, float* scale, float* scale_inv, hipStream_t st);
void launch_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                           int fmt, const float* scale, uint8_t* q, uint8_t* qt, float* amax_out,
                           hipStream_t st);
// One delayed-scaling step of one tensor in a single launch: cast +
// transpose with *scale, amax, history[step mod L] = amax and the next scale.
// ws: two words, zero on entry, zero again on return.
void launch_cast_transpose_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                   int margin, float* history, int64_t L, int64_t step, float* scale,
                                   float* scale_inv, uint8_t* q, uint8_t* qt, float* amax_out, uint32_t* ws,
                                   hipStream_t st);
// Device address of this GPU's file-scope workspace for the allocation-free
// delayed step (looked up once per device; the first lookup also clears it on
// `st`).  Returns 0, or a negative code when the lookup fails.
int delayed_scratch(uint32_t** out, hipStream_t st);
void launch_quantize_blocked(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int scaling, int fmt, int margin, bool mx_ceil, uint8_t* q, void* s,
                             uint8_t* qt, void* st_, hipStream_t st);
// 256x256x128 direct-to-LDS kernel for per-tensor (mx = false) and MXFP8
// scales; returns false (and launches nothing) when the problem is not
// eligible, in which case the general kernel is used.  accumulate (fp32 C
// only): C = fp32(C + result) instead of C = result.
bool launch_scaled_gemm_fast(const uint8_t* a, int fa, bool mx, const void* sa, const uint8_t* b, int fb,
                             const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st);
// 128x128 two-workgroups-per-CU kernel for blockwise scales with 128x128
// weight blocks (w128; 1x128 activation blocks on A); returns false (and
// launches nothing) when the problem is not eligible.
bool launch_scaled_gemm_block_fast(const uint8_t* a, int fa, const float* sa, const uint8_t* b, int fb,
                                   const float* sb, bool w128, int64_t M, int64_t N, int64_t K, int64_t lda,
                                   int64_t ldb, void* c, int c_dtype, int64_t ldc, hipStream_t st);
// 256x256 eight-wave kernel for blockwise scales (16x16x128 instructions, one
// per 128-K block and 16 x 16 tile): w128 = 128 x 128 weight blocks on B
// (fprop, dgrad), else 1 x 128 blocks on both operands (wgrad); returns false
// (and launches nothing) when the problem is not eligible.
bool launch_scaled_gemm_block2(const uint8_t* a, int fa, const float* sa, const uint8_t* b, int fb, const float* sb,
                               bool w128, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                               int c_dtype, int64_t ldc, hipStream_t st);
// GeLU of h with the FP8 store of h (forward) and the GeLU gradient from the
// stored FP8 input (backward); bf16 h / da with leading dimension ld, dense
// a / dh / q.
void launch_act_fp8_store_fwd(const void* h, int64_t rows, int64_t cols, int64_t ld, int fmt, const float* scale,
                              void* a, uint8_t* q, float* amax_out, hipStream_t st);
void launch_act_fp8_store_bwd(const void* da, int64_t rows, int64_t cols, int64_t ld, int fmt, const uint8_t* q,
                              const float* scale_inv, void* dh, hipStream_t st);
// bf16 weight gradient C[N x K] (=, +=) dY^T X over T tokens (dY T x N, X T x K,
// row-major bf16); accumulate for fp32 C only.
void launch_wgrad_bf16(const void* dy, int64_t T, int64_t N, int64_t lddy, const void* x, int64_t K, int64_t ldx,
                       void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st);
// NVFP4: ts = {amax, s_enc, s_dec} written on `st`; row-wise (q, s) and/or
// column-wise (qt, st_) copies with E4M3 scales per 16 elements.
void launch_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* q, uint8_t* s,
                           uint8_t* qt, uint8_t* st_, float* ts, hipStream_t st);
// C = (s_dec_a s_dec_b) * sum of block-scaled E2M1 products; A M x K and B
// N x K packed (lda, ldb in bytes), sa / sb dense E4M3 bytes (K / 16 per row).
void launch_gemm_nvfp4(const uint8_t* a, const uint8_t* sa, const float* ta, const uint8_t* b, const uint8_t* sb,
                       const float* tb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                       int c_dtype, int64_t ldc, hipStream_t st);
// 256x256 persistent kernel for NVFP4 (f16 MFMA on exactly decoded values);
// returns false (and launches nothing) when the problem is not eligible.
bool launch_gemm_nvfp4_fast(const uint8_t* a, const uint8_t* sa, const float* ta, const uint8_t* b, const uint8_t* sb,
                            const float* tb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                            int c_dtype, int64_t ldc, hipStream_t st);
void launch_scaled_gemm(const uint8_t* a, int fa, int ka, const void* sa, const uint8_t* b, int fb,
                        int kb, const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda,
                        int64_t ldb, void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st);

}  // namespace qsg
