// Scaled FP8 GEMM for gfx950:  C[m,n] = sum_k (A[m,k] sa) (B[n,k] sb), A M x K
// and B N x K, both K-contiguous FP8 ("Low-Precision Training Guide", section
// "When to Use Low Precision": the FP8 GEMMs; recipes "mxfp8" and "blockwise"
// for the scale granularity).
//
// Design.
//   * Workgroup tile BM x BN x 128 (K), 256 threads = 4 wave64s in a 2 x 2
//     grid; each wave computes (BM/2) x (BN/2) with 32x32x64 f8f6f4 MFMAs
//     (v_mfma_f32_32x32x64_f8f6f4 unscaled, v_mfma_scale_... for MXFP8 with
//     the E8M0 bytes fed natively).
//   * MFMA operand layout (measured on gfx950 with block-scaled probes): lane
//     l holds row (l & 31) of a 32-row slice; with h = l >> 5 its 8 VGPRs hold
//     K [16h, 16h + 16) of the 64-K step in bytes 0..15 and K [32 + 16h,
//     48 + 16h) in bytes 16..31.  The scale byte of lanes 0..31 applies to K
//     0..31 of the step and that of lanes 32..63 to K 32..63, so lane half h
//     passes the E8M0 byte of 32-K block h.  The MFMA is issued as (B
//     fragment, A fragment), so the
//     accumulator of lane l holds one output row m = l & 31 and four runs of
//     four consecutive columns; the epilogue stores 8 bytes (4 bf16) per run.
//   * Global -> LDS: each thread moves 16-byte chunks (8 lanes = one 128-byte
//     K row of the tile); LDS rows are 128 bytes with the 16-byte chunk index
//     XOR-swizzled by row (see swz), so the 16-byte fragment reads of 16
//     consecutive rows hit all 64 banks.  Two LDS stages; the next K tile is
//     fetched into registers while the current one is multiplied.
//   * Scales: per-tensor scales multiply the fp32 accumulator in the epilogue;
//     MXFP8 scales go to the MFMA; blockwise scales multiply the fp32 partial
//     sum of each 128-K block (one K tile) before it is added to the
//     accumulator.
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 128;

enum ScaleMode { SM_TENSOR = 0, SM_MX = 1, SM_BLOCK_W = 2, SM_BLOCK_A = 3 };

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  int64_t M, N, K, lda, ldb, ldc;
  void* c;
  bool vec_ab;   // 16-byte loads of A and B allowed
  bool vec_c;    // vector stores of C allowed
  bool accumulate;  // fp32 C only: C = fp32(C + result)
  int64_t tiles_m, tiles_n;
};

template <int BM, int BN>
struct Smem {
  uint8_t a[2][BM * BK];
  uint8_t b[2][BN * BK];
  uint32_t sa[2][BM];  // MX: 4 E8M0 bytes (the tile's 4 K blocks) per row; block: fp32 bits
  uint32_t sb[2][BN];
};

// 16-byte chunk c of LDS row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1):
// 16 consecutive rows read at one chunk cover all 64 LDS banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

// Load a (ROWS x 128) K tile of an operand into registers: ROWS*8 chunks of 16 B.
template <int ROWS>
struct TileRegs {
  static constexpr int N = ROWS * 8 / 256;
  uint4 v[N];
};

template <int ROWS>
__device__ __forceinline__ void g_load(TileRegs<ROWS>& t, const uint8_t* __restrict__ p, int64_t ld,
                                       int64_t row0, int64_t nrows, int64_t k0, int64_t K, bool vec) {
#pragma unroll
  for (int i = 0; i < TileRegs<ROWS>::N; ++i) {
    const int id = i * 256 + threadIdx.x;
    const int row = id >> 3, chunk = id & 7;
    const int64_t gr = row0 + row, gk = k0 + chunk * 16;
    if (gr < nrows && vec && gk + 16 <= K) {
      t.v[i] = *reinterpret_cast<const uint4*>(p + gr * ld + gk);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
      if (gr < nrows) {
#pragma unroll
        for (int bb = 0; bb < 16; ++bb)
          if (gk + bb < K) w[bb >> 2] |= (uint32_t)p[gr * ld + gk + bb] << (8 * (bb & 3));
      }
      t.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int ROWS>
__device__ __forceinline__ void s_store(const TileRegs<ROWS>& t, uint8_t* lds) {
#pragma unroll
  for (int i = 0; i < TileRegs<ROWS>::N; ++i) {
    const int id = i * 256 + threadIdx.x;
    const int row = id >> 3, chunk = id & 7;
    *reinterpret_cast<uint4*>(lds + swz(row, chunk)) = t.v[i];
  }
}

// One 32-row MFMA operand fragment for K step kk (0 or 1) of the tile: lane
// half h takes the 16-byte chunks h and 2 + h of the step.
__device__ __forceinline__ v8i frag(const uint8_t* lds, int row0, int kk, int lane) {
  const int row = row0 + (lane & 31);
  const int c0 = kk * 4 + (lane >> 5);
  uint4 lo = *reinterpret_cast<const uint4*>(lds + swz(row, c0));
  uint4 hi = *reinterpret_cast<const uint4*>(lds + swz(row, c0 + 2));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Scale words of one K tile for rows [row0, row0 + ROWS) of an operand.
//   SM_MX:      4 E8M0 bytes (K blocks 4kt .. 4kt+3), missing blocks = 127
//   SM_BLOCK_*: fp32 bits of the tile's scale_inv for the row (or row block)
template <int MODE>
__device__ __forceinline__ uint32_t load_scale_word(const void* s, int64_t row, int64_t nrows,
                                                    int64_t kt, int64_t K, bool per_128_rows) {
  if constexpr (MODE == SM_MX) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(s);
    const int64_t nb = K / 32;  // E8M0 bytes per row
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t blk = kt * 4 + j;
      uint32_t byte = 127u;
      if (row < nrows && blk < nb) byte = p[row * nb + blk];
      w |= byte << (8 * j);
    }
    return w;
  } else {
    const float* p = reinterpret_cast<const float*>(s);
    const int64_t nb = K / 128;
    if (row >= nrows) return 0u;
    const int64_t r = per_128_rows ? row / 128 : row;
    return __float_as_uint(p[r * nb + kt]);
  }
}

template <int BM, int BN, int MODE, int FA, int FB, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) Smem<BM, BN> sm;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile order: groups of 8 tile-rows walk along N together (L2 reuse of B)
  const int64_t bid = blockIdx.x;
  constexpr int64_t GROUP = 8;
  const int64_t per_group = GROUP * g.tiles_n;
  const int64_t group = bid / per_group;
  const int64_t first_m = group * GROUP;
  const int64_t gsize = (g.tiles_m - first_m) < GROUP ? (g.tiles_m - first_m) : GROUP;
  const int64_t tm_idx = first_m + (bid % per_group) % gsize;
  const int64_t tn_idx = (bid % per_group) / gsize;
  const int64_t m0 = tm_idx * BM, n0 = tn_idx * BN;

  const int64_t nk = (g.K + BK - 1) / BK;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  TileRegs<BM> ra;
  TileRegs<BN> rb;
  uint32_t rsa = 0, rsb = 0;  // this thread's scale word for the next tile
  const bool w128 = (MODE == SM_BLOCK_W);

  auto fetch = [&](int64_t kt) {
    g_load<BM>(ra, g.a, g.lda, m0, g.M, kt * BK, g.K, g.vec_ab);
    g_load<BN>(rb, g.b, g.ldb, n0, g.N, kt * BK, g.K, g.vec_ab);
    if constexpr (MODE != SM_TENSOR) {
      if (tid < BM) rsa = load_scale_word<MODE>(g.sa, m0 + tid, g.M, kt, g.K, false);
      if (tid < BN) rsb = load_scale_word<MODE>(g.sb, n0 + tid, g.N, kt, g.K, w128);
    }
  };
  auto stash = [&](int buf) {
    s_store<BM>(ra, sm.a[buf]);
    s_store<BN>(rb, sm.b[buf]);
    if constexpr (MODE != SM_TENSOR) {
      if (tid < BM) sm.sa[buf][tid] = rsa;
      if (tid < BN) sm.sb[buf][tid] = rsb;
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) fetch(kt + 1);

    if constexpr (MODE == SM_BLOCK_W || MODE == SM_BLOCK_A) {
      v16f part[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) part[i][j][v] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v8i fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = frag(sm.a[buf], wm * WM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = frag(sm.b[buf], wn * WN + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], part[i][j], FB, FA, 0, 0, 0, 0);
      }
      // acc += part * sa[m] * sb[n]
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float s_a = __uint_as_float(sm.sa[buf][wm * WM + i * 32 + (lane & 31)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int nl = wn * WN + j * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const float s_b = __uint_as_float(sm.sb[buf][nl]);
            acc[i][j][v] += part[i][j][v] * (s_a * s_b);
          }
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v8i fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = frag(sm.a[buf], wm * WM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = frag(sm.b[buf], wn * WN + j * 32, kk, lane);
        if constexpr (MODE == SM_MX) {
          const int sh = 8 * (kk * 2 + (lane >> 5));
          int sca[TM], scb[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) sca[i] = (int)((sm.sa[buf][wm * WM + i * 32 + (lane & 31)] >> sh) & 0xFFu);
#pragma unroll
          for (int j = 0; j < TN; ++j) scb[j] = (int)((sm.sb[buf][wn * WN + j * 32 + (lane & 31)] >> sh) & 0xFFu);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], FB, FA, 0, scb[j], 0, sca[i]);
        } else {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], FB, FA, 0, 0, 0, 0);
        }
      }
    }

    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  float alpha = 1.0f;
  if constexpr (MODE == SM_TENSOR)
    alpha = *reinterpret_cast<const float*>(g.sa) * *reinterpret_cast<const float*>(g.sb);

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * WM + i * 32 + (lane & 31);
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int64_t n = n0 + wn * WN + j * 32 + grp * 8 + (lane >> 5) * 4;
        float v0 = acc[i][j][grp * 4 + 0] * alpha, v1 = acc[i][j][grp * 4 + 1] * alpha;
        float v2 = acc[i][j][grp * 4 + 2] * alpha, v3 = acc[i][j][grp * 4 + 3] * alpha;
        if constexpr (OUT_BF16) {
          uint16_t* c = reinterpret_cast<uint16_t*>(g.c) + m * g.ldc + n;
          uint16_t h0 = f32_to_bf16_rne(v0), h1 = f32_to_bf16_rne(v1);
          uint16_t h2 = f32_to_bf16_rne(v2), h3 = f32_to_bf16_rne(v3);
          if (g.vec_c && n + 3 < g.N) {
            *reinterpret_cast<uint2*>(c) = make_uint2((uint32_t)h0 | ((uint32_t)h1 << 16),
                                                      (uint32_t)h2 | ((uint32_t)h3 << 16));
          } else {
            if (n + 0 < g.N) c[0] = h0;
            if (n + 1 < g.N) c[1] = h1;
            if (n + 2 < g.N) c[2] = h2;
            if (n + 3 < g.N) c[3] = h3;
          }
        } else {
          float* c = reinterpret_cast<float*>(g.c) + m * g.ldc + n;
          if (g.vec_c && n + 3 < g.N) {
            if (g.accumulate) {
              const float4 o = *reinterpret_cast<const float4*>(c);
              v0 += o.x; v1 += o.y; v2 += o.z; v3 += o.w;
            }
            *reinterpret_cast<float4*>(c) = make_float4(v0, v1, v2, v3);
          } else {
            if (n + 0 < g.N) c[0] = g.accumulate ? c[0] + v0 : v0;
            if (n + 1 < g.N) c[1] = g.accumulate ? c[1] + v1 : v1;
            if (n + 2 < g.N) c[2] = g.accumulate ? c[2] + v2 : v2;
            if (n + 3 < g.N) c[3] = g.accumulate ? c[3] + v3 : v3;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int MODE, int FA, int FB>
void launch_cfg(const GemmArgs& g, bool out_bf16, hipStream_t st) {
  const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, FA, FB, true>), dim3(grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, FA, FB, false>), dim3(grid), dim3(256), 0, st, g);
}

template <int BM, int BN, int MODE>
void launch_fmt(const GemmArgs& g, int fa, int fb, bool out_bf16, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_cfg<BM, BN, MODE, kE4M3, kE4M3>(g, out_bf16, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_cfg<BM, BN, MODE, kE5M2, kE4M3>(g, out_bf16, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_cfg<BM, BN, MODE, kE4M3, kE5M2>(g, out_bf16, st);
  else launch_cfg<BM, BN, MODE, kE5M2, kE5M2>(g, out_bf16, st);
}

}  // namespace

void launch_scaled_gemm(const uint8_t* a, int fa, int ka, const void* sa, const uint8_t* b, int fb,
                        int kb, const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda,
                        int64_t ldb, void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st) {
  const bool per_tensor = (ka == 0 || ka == 1) && (kb == 0 || kb == 1);
  if ((per_tensor || ka == 2) &&
      launch_scaled_gemm_fast(a, fa, ka == 2, sa, b, fb, sb, M, N, K, lda, ldb, c, c_dtype, ldc, accumulate, st))
    return;
  // (the blockwise large-tile kernels only write C; accumulation uses the general kernel)
  if (ka == 3 && (kb == 4 || kb == 3) && !accumulate &&
      launch_scaled_gemm_block2(a, fa, reinterpret_cast<const float*>(sa), b, fb, reinterpret_cast<const float*>(sb),
                                kb == 4, M, N, K, lda, ldb, c, c_dtype, ldc, st))
    return;
  if (ka == 3 && kb == 4 && !accumulate &&
      launch_scaled_gemm_block_fast(a, fa, reinterpret_cast<const float*>(sa), b, fb,
                                    reinterpret_cast<const float*>(sb), true, M, N, K, lda, ldb, c, c_dtype, ldc,
                                    st))
    return;
  constexpr int BM = 128, BN = 128;
  GemmArgs g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  g.accumulate = accumulate && c_dtype == 0;
  g.vec_ab = ((uintptr_t)a % 16 == 0) && ((uintptr_t)b % 16 == 0) && (lda % 16 == 0) && (ldb % 16 == 0);
  const bool out_bf16 = (c_dtype == 1);
  g.vec_c = out_bf16 ? (((uintptr_t)c % 8 == 0) && (ldc % 4 == 0)) : (((uintptr_t)c % 16 == 0) && (ldc % 4 == 0));
  g.tiles_m = (M + BM - 1) / BM;
  g.tiles_n = (N + BN - 1) / BN;
  int mode = SM_TENSOR;
  if (ka == 2) mode = SM_MX;
  else if (ka == 3 && kb == 4) mode = SM_BLOCK_W;
  else if (ka == 3 && kb == 3) mode = SM_BLOCK_A;
  switch (mode) {
    case SM_MX: launch_fmt<BM, BN, SM_MX>(g, fa, fb, out_bf16, st); break;
    case SM_BLOCK_W: launch_fmt<BM, BN, SM_BLOCK_W>(g, fa, fb, out_bf16, st); break;
    case SM_BLOCK_A: launch_fmt<BM, BN, SM_BLOCK_A>(g, fa, fb, out_bf16, st); break;
    default: launch_fmt<BM, BN, SM_TENSOR>(g, fa, fb, out_bf16, st); break;
  }
}

}  // namespace qsg
