// NVFP4 block scaling for gfx950: quantization to E2M1 with one E4M3 scale
// per 1 x 16 block and one fp32 scale per tensor, and the GEMM on such
// operands.  ("Low-Precision Training Guide": recipe "nvfp4", NVFP4 block
// scaling, --fp4-format e2m1.  The pages give neither the block size nor the
// scale formats; they follow NVIDIA's NVFP4 definition: 16-element blocks
// along the contraction dimension, an E4M3 decode scale per block and an
// fp32 per-tensor scale s_enc = 448 * 6 / amax.)
//
// Quantization of a block with maximum b, each step one binary32 operation:
//   sdec = b / 6;  code = E4M3(sdec * s_enc) (saturating RNE);  S = dec(code);
//   m = s_enc / S (0 when S is 0 or NaN);  q = E2M1(x * m) (saturating RNE,
//   ties to the even code).
// Two codes per byte along the row, element 2i in the low nibble.  The
// column-wise copy (blocks of 16 rows, stored transposed) shares s_enc.
//
// Design for MI355X.
//   * Quantize: amax pass, a one-thread tensor-scale kernel, then one pass in
//     128 x 128 tiles (thread = 8 x 8 values, all 16-byte loads of a full tile
//     in flight together): a row block is a lane pair (xor 1), a column block
//     the two row groups of a lane pair (xor 16), so both copies come from one
//     read of the input.  Element codes come from the hardware E2M1
//     conversion (scale 1), two values per instruction; the column codes
//     leave through an LDS tile as 16-byte pieces.
//   * GEMM (this file: the general kernel for any K % 16 == 0 and any
//     alignment; the persistent 256 x 256 kernel for large aligned problems
//     is gemm_nvfp4_fast_kernel in gemm_fast.hip): an NVFP4 value times its
//     block scale has at most 6 significant bits, so it is exact in bfloat16;
//     operands are decoded to bf16 (block scale applied) on their way into LDS
//     and multiplied with v_mfma_f32_32x32x16_bf16, whose 16-K step is exactly
//     one NVFP4 block.  The per-tensor factors s_dec_a * s_dec_b are applied
//     in the epilogue.  (gfx950's FP4 matrix instructions take power-of-two
//     scales per 32 elements, which cannot express an E4M3 scale per 16.)
//     128 x 128 x 64 tiles, 4 waves of 64 x 64, register-staged: the next K
//     tile's FP4 bytes are loaded while the current one is multiplied.
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// OCP E4M3 byte -> binary32 (software: the GEMM's general path).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float v = e == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -v : v;
}

// Eight binary32 values times m -> eight E2M1 codes, value i in nibble i.
// v_cvt_scalef32_pk_fp4_f32 with scale 1 is the saturating RNE encode of the
// recipe (nearest of 0, 0.5, ..., 6, a midpoint to the even code, the sign
// of zero kept, NaN to sign | 6); the products are rounded to binary32 first.
__device__ __forceinline__ uint32_t e2m1x8(float v0, float v1, float v2, float v3, float v4, float v5, float v6,
                                           float v7, float m) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0 * m, v1 * m, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v2 * m, v3 * m, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v4 * m, v5 * m, 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v6 * m, v7 * m, 1.0f, 3);
}

// Element multiplier of an E4M3 block-scale code: fp32(s_enc / S), 0 when S
// is 0 or NaN (code 0x7F; a NaN block).  The codes of the non-negative block
// scales are 0..127, so a workgroup tabulates the 128 quotients once.
__device__ __forceinline__ float mult_of_code(uint32_t code, float s_enc) {
  const float S = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
  return S > 0.0f ? __fdiv_rn(s_enc, S) : 0.0f;
}

// Block scale code of a block with maximum |x| pattern bmax (non-negative
// binary32 bits; NaN canonical) and its element multiplier from the table.
__device__ __forceinline__ void block_scale(uint32_t bmax, float s_enc, const float* mult_table, uint32_t& code,
                                            float& mult) {
  const float sdec = __fdiv_rn(__uint_as_float(bmax), 6.0f);
  code = cvt_pk<kE4M3, false>(sdec * s_enc, 0.0f, 0u) & 0xFFu;
  mult = mult_table[code & 0x7Fu];
}

// ---------------------------------------------------------------------------
// tensor scale and quantization
// ---------------------------------------------------------------------------
__global__ void nvfp4_tensor_scale_kernel(float* ts) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const float a = ts[0];
    const uint32_t ab = __float_as_uint(a) & 0x7FFFFFFFu;
    float s = 1.0f;
    if (ab != 0u && ab < 0x7F800000u) {
      s = __fdiv_rn(448.0f * 6.0f, a);
      if (__float_as_uint(s) == 0x7F800000u) s = __uint_as_float(0x7F7FFFFFu);
    }
    ts[1] = s;
    ts[2] = __fdiv_rn(1.0f, s);
  }
}

struct NvQuantArgs {
  const void* x;
  int64_t rows, cols, ld;
  bool vec_ok;
  const float* ts;  // {amax, s_enc, s_dec}
  uint8_t* q;       // rows x cols/2, or null
  uint8_t* s;       // rows x cols/16
  uint8_t* qt;      // cols x rows/2, or null
  uint8_t* st;      // cols x rows/16
  bool qt_vec;      // QT rows of 16-byte aligned runs (qt 16-byte aligned, rows % 32 == 0)
  bool st_vec;      // 8-byte scale runs aligned (st 8-byte aligned, rows % 128 == 0)
  int64_t tiles_c, ntiles;
};

// The thread's 8 x 8 values as binary32.  A full tile issues all 16-byte
// loads before the first use (one wait); a partial tile reads element by
// element with bounds checks (zeros outside).
template <typename In>
__device__ __forceinline__ void load8x8(const NvQuantArgs& a, int64_t r, int64_t c, bool full, float (&v)[8][8]) {
  const In* x = reinterpret_cast<const In*>(a.x);
  if (full) {
    constexpr int NV = sizeof(In) == 2 ? 1 : 2;  // 16-byte loads per row
    u32x4 u[8][NV];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < NV; ++k) u[j][k] = ld_stream16(x + (r + j) * a.ld + c + 4 * k);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (sizeof(In) == 2) {
        const uint32_t w[4] = {u[j][0].x, u[j][0].y, u[j][0].z, u[j][0].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[j][2 * k] = bf16lo(w[k]);
          v[j][2 * k + 1] = bf16hi(w[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          v[j][4 * k + 0] = __uint_as_float(u[j][k].x);
          v[j][4 * k + 1] = __uint_as_float(u[j][k].y);
          v[j][4 * k + 2] = __uint_as_float(u[j][k].z);
          v[j][4 * k + 3] = __uint_as_float(u[j][k].w);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float f = 0.0f;
        if (r + j < a.rows && c + i < a.cols) {
          if constexpr (sizeof(In) == 2)
            f = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[(r + j) * a.ld + c + i] << 16);
          else
            f = x[(r + j) * a.ld + c + i];
        }
        v[j][i] = f;
      }
    }
  }
}

__device__ __forceinline__ uint32_t absbits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

constexpr int QT_STRIDE = 17;  // words per column of the LDS tile of column codes

template <typename In>
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(NvQuantArgs a) {
  __shared__ uint32_t lds_qt[128 * QT_STRIDE];
  __shared__ __attribute__((aligned(8))) uint8_t lds_st[128 * 8];
  __shared__ float lds_mult[128];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float s_enc = a.ts[1];
  if (tid < 128) lds_mult[tid] = mult_of_code((uint32_t)tid, s_enc);
  __syncthreads();
  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / a.tiles_c) * 128, c0 = (tile % a.tiles_c) * 128;
    const int64_t r = r0 + ty * 8, c = c0 + tx * 8;
    const bool full = a.vec_ok && r0 + 128 <= a.rows && c0 + 128 <= a.cols;
    float v[8][8];
    load8x8<In>(a, r, c, full, v);
    if (a.q) {
      // row blocks: this lane's 8 columns and its pair lane's (xor 1)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = umax(m, absbits(v[j][i]));
        m = umax(m, dpp_u32<kDppXor1>(m));
        uint32_t code;
        float mult;
        block_scale(m > 0x7F800000u ? 0x7FC00000u : m, s_enc, lds_mult, code, mult);
        const uint32_t w = e2m1x8(v[j][0], v[j][1], v[j][2], v[j][3], v[j][4], v[j][5], v[j][6], v[j][7], mult);
        if (r + j < a.rows && c < a.cols) {
          *reinterpret_cast<uint32_t*>(a.q + (r + j) * (a.cols / 2) + c / 2) = w;
          if ((tx & 1) == 0) a.s[(r + j) * (a.cols / 16) + c / 16] = (uint8_t)code;
        }
      }
    }
    if (a.qt) {
      // column blocks: this lane's 8 rows and its pair row group's (xor 16).
      // Inside the matrix the codes go through LDS, [column][64 bytes] with
      // a 4-byte pad per column, and leave as 16-byte pieces, 4 lanes per
      // 64-byte run of a QT row; the 8 scale bytes of a column leave as one
      // 8-byte store.
      const bool staged = a.qt_vec && r0 + 128 <= a.rows && c0 + 128 <= a.cols;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = umax(m, absbits(v[j][i]));
        m = max_xor16(m);
        uint32_t code;
        float mult;
        block_scale(m > 0x7F800000u ? 0x7FC00000u : m, s_enc, lds_mult, code, mult);
        const uint32_t w = e2m1x8(v[0][i], v[1][i], v[2][i], v[3][i], v[4][i], v[5][i], v[6][i], v[7][i], mult);
        if (staged) {
          lds_qt[(tx * 8 + i) * QT_STRIDE + ty] = w;
          if ((ty & 1) == 0) lds_st[(tx * 8 + i) * 8 + (ty >> 1)] = (uint8_t)code;
        } else if (c + i < a.cols && r < a.rows) {
          *reinterpret_cast<uint32_t*>(a.qt + (c + i) * (a.rows / 2) + r / 2) = w;
          if ((ty & 1) == 0) a.st[(c + i) * (a.rows / 16) + r / 16] = (uint8_t)code;
        }
      }
      if (staged) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int q = tid + 256 * k, col = q >> 2, part = q & 3;
          const uint32_t* src = lds_qt + col * QT_STRIDE + part * 4;
          const u32x4 piece = {src[0], src[1], src[2], src[3]};
          *reinterpret_cast<u32x4*>(a.qt + (c0 + col) * (a.rows / 2) + r0 / 2 + part * 16) = piece;
        }
        if (tid < 128) {
          const uint2 sc = *reinterpret_cast<const uint2*>(lds_st + tid * 8);
          uint8_t* dst = a.st + (c0 + tid) * (a.rows / 16) + r0 / 16;
          if (a.st_vec) {
            *reinterpret_cast<uint2*>(dst) = sc;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = (uint8_t)((e < 4 ? sc.x : sc.y) >> (8 * (e & 3)));
          }
        }
        __syncthreads();  // the LDS tile is reused by the next tile
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------
constexpr int NBM = 128, NBN = 128, NBK = 64;  // elements; a K tile is 32 bytes of codes per row
constexpr int NROWB = NBK * 2;                 // bytes per LDS row (bf16)

struct NvGemmArgs {
  const uint8_t* a;   // M x K/2
  const uint8_t* b;   // N x K/2
  const uint8_t* sa;  // M x K/16 E4M3
  const uint8_t* sb;  // N x K/16
  const float* ta;    // s_dec of A
  const float* tb;    // s_dec of B
  int64_t M, N, K, lda, ldb, ldc;
  void* c;
  bool vec_ab, vec_c;
};

__device__ __forceinline__ int nv_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// The 32 codes (16 bytes) a thread stages per operand and K tile, with the
// two block-scale bytes that cover them.
struct Stage {
  u32x4 codes;
  uint32_t scales;  // byte 0: first block, byte 1: second
};

__device__ __forceinline__ Stage nv_load(const uint8_t* base, const uint8_t* sbase, int64_t ld, int64_t nrows,
                                         int64_t K, int64_t row, int64_t k0, bool vec) {
  Stage s;
  s.codes = u32x4{0u, 0u, 0u, 0u};
  s.scales = 0u;
  if (row < nrows && k0 < K) {  // K % 16 == 0: each 16-element block is all in or all out
    const bool two = k0 + 32 <= K;
    const uint8_t* p = base + row * ld + k0 / 2;
    if (vec && two) {
      s.codes = *reinterpret_cast<const u32x4*>(p);
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      const int nb = two ? 16 : 8;
      for (int q = 0; q < nb; ++q) w[q >> 2] |= (uint32_t)p[q] << (8 * (q & 3));
      s.codes = u32x4{w[0], w[1], w[2], w[3]};
    }
    const uint8_t* ps = sbase + row * (K / 16) + k0 / 16;
    s.scales = (uint32_t)ps[0] | (two ? ((uint32_t)ps[1] << 8) : 0u);
  }
  return s;
}

// Decode 32 codes to bf16 (each times its block's E4M3 scale: exact) and
// write them to the thread's 64 bytes of its LDS row: chunks 4 h .. 4 h + 3.
__device__ __forceinline__ void nv_store(uint8_t* lds, int row, int h, const Stage& s) {
  const uint32_t w[4] = {s.codes.x, s.codes.y, s.codes.z, s.codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // 8 codes = one 16-byte chunk of bf16
    const float S = e4m3_to_f32((s.scales >> (8 * (q >> 1))) & 0xFFu);
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3);
    const uint32_t pk[4] = {pack_bf16x2(f0[0] * S, f0[1] * S), pack_bf16x2(f1[0] * S, f1[1] * S),
                            pack_bf16x2(f2[0] * S, f2[1] * S), pack_bf16x2(f3[0] * S, f3[1] * S)};
    const int chunk = 4 * h + q;
    *reinterpret_cast<uint4*>(lds + row * NROWB + ((chunk ^ nv_swizzle(row)) << 4)) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void nvfp4_gemm_kernel(NvGemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[NBM * NROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[NBN * NROWB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * NBM, n0 = (int64_t)blockIdx.x * NBN;
  const int srow = tid >> 1, sh = tid & 1;  // staging: row and half of the K tile
  const int64_t nkt = g.K / NBK + (g.K % NBK ? 1 : 0);

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  Stage ra = nv_load(g.a, g.sa, g.lda, g.M, g.K, m0 + srow, sh * 32, g.vec_ab);
  Stage rb = nv_load(g.b, g.sb, g.ldb, g.N, g.K, n0 + srow, sh * 32, g.vec_ab);
  for (int64_t kt = 0; kt < nkt; ++kt) {
    __syncthreads();  // the previous K tile's fragments are read
    nv_store(lds_a, srow, sh, ra);
    nv_store(lds_b, srow, sh, rb);
    __syncthreads();
    if (kt + 1 < nkt) {
      ra = nv_load(g.a, g.sa, g.lda, g.M, g.K, m0 + srow, (kt + 1) * NBK + sh * 32, g.vec_ab);
      rb = nv_load(g.b, g.sb, g.ldb, g.N, g.K, n0 + srow, (kt + 1) * NBK + sh * 32, g.vec_ab);
    }
#pragma unroll
    for (int ks = 0; ks < NBK / 16; ++ks) {
      const int chunk = 2 * ks + (lane >> 5);  // 16 K per step: lane half h holds 8 of them
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const bf16x8*>(lds_a + row * NROWB + ((chunk ^ nv_swizzle(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + (lane & 31);
        fb[j] = *reinterpret_cast<const bf16x8*>(lds_b + row * NROWB + ((chunk ^ nv_swizzle(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane l of tile (i, j) holds row 32 i + l % 32 of the wave's
  // block and, for group q = 0..3, the 4 columns 32 j + 8 q + 4 (l / 32) + 0..3
  const float alpha = *g.ta * *g.tb;
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 64 + i * 32 + (lane & 31);
    if (m >= g.M) continue;
    uint8_t* rowp = reinterpret_cast<uint8_t*>(g.c) + m * g.ldc * ESZ;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 64 + j * 32 + q * 8 + (lane >> 5) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][q * 4 + e] * alpha;
        if (g.vec_c && n + 4 <= g.N) {
          if constexpr (OUT_BF16)
            *reinterpret_cast<uint2*>(rowp + n * ESZ) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          else
            *reinterpret_cast<uint4*>(rowp + n * ESZ) =
                make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e < g.N) {
              if constexpr (OUT_BF16)
                reinterpret_cast<uint16_t*>(rowp)[n + e] = f32_to_bf16_rne(v[e]);
              else
                reinterpret_cast<float*>(rowp)[n + e] = v[e];
            }
          }
        }
      }
    }
  }
}

int nv_num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) n = p.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

}  // namespace

void launch_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, uint8_t* q, uint8_t* s,
                           uint8_t* qt, uint8_t* st, float* ts, hipStream_t stream) {
  launch_amax(x, dtype, rows, cols, ld, ts, stream);  // ts[0] = amax (0 for an empty tensor)
  hipLaunchKernelGGL(nvfp4_tensor_scale_kernel, dim3(1), dim3(64), 0, stream, ts);
  if (rows == 0 || cols == 0) return;
  NvQuantArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.ld = ld;
  const int esz = dtype == 1 ? 2 : 4;
  a.vec_ok = ((uintptr_t)x % 16 == 0) && ((ld * esz) % 16 == 0);
  a.ts = ts; a.q = q; a.s = s; a.qt = qt; a.st = st;
  a.qt_vec = qt && ((uintptr_t)qt % 16 == 0) && (rows % 32 == 0);
  a.st_vec = st && ((uintptr_t)st % 8 == 0) && (rows % 128 == 0);
  a.tiles_c = (cols + 127) / 128;
  a.ntiles = ((rows + 127) / 128) * a.tiles_c;
  int64_t grid = a.ntiles, cap = (int64_t)nv_num_cus() * 128;  // one tile per workgroup up to 128 per CU
  if (grid > cap) grid = cap;
  if (dtype == 1)
    hipLaunchKernelGGL(nvfp4_quant_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(nvfp4_quant_kernel<float>, dim3((unsigned)grid), dim3(256), 0, stream, a);
}

void launch_gemm_nvfp4(const uint8_t* a, const uint8_t* sa, const float* ta, const uint8_t* b, const uint8_t* sb,
                       const float* tb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                       int c_dtype, int64_t ldc, hipStream_t stream) {
  if (launch_gemm_nvfp4_fast(a, sa, ta, b, sb, tb, M, N, K, lda, ldb, c, c_dtype, ldc, stream)) return;
  NvGemmArgs g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb; g.ta = ta; g.tb = tb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  g.vec_ab = ((uintptr_t)a % 16 == 0) && ((uintptr_t)b % 16 == 0) && (lda % 16 == 0) && (ldb % 16 == 0);
  const bool out_bf16 = c_dtype == 1;
  g.vec_c = out_bf16 ? (((uintptr_t)c % 8 == 0) && (ldc % 4 == 0)) : (((uintptr_t)c % 16 == 0) && (ldc % 4 == 0));
  const dim3 grid((unsigned)((N + NBN - 1) / NBN), (unsigned)((M + NBM - 1) / NBM));
  if (out_bf16)
    hipLaunchKernelGGL(nvfp4_gemm_kernel<true>, grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(nvfp4_gemm_kernel<false>, grid, dim3(256), 0, stream, g);
}

}  // namespace qsg
