// Large-tile FP8 GEMM with blockwise scales for gfx950:
//   C[m,n] = sum_kb (sum_{k in kb} A[m,k] B[n,k]) * sa[m,kb] * sb[., kb]
// with 128-wide K blocks kb; sb is indexed by n / 128 (128 x 128 weight
// blocks, fprop / dgrad) or by n (1 x 128 blocks on both operands, wgrad).
// ("Low-Precision Training Guide", recipe "blockwise": 1 x 128 activation and
// 128 x 128 weight blocks with an fp32 scale each; the partial sum of every
// K block is scaled and added in fp32.)
//
// Design for MI355X.
//   * The per-block scale is applied by the VALU to each K block's MFMA
//     partial sum, so every lane holds its running sums and the block's
//     partial sums: a 128 x 128 wave tile would need 512 registers for the
//     two.  The wave tile is 64 x 64 (2 x 2 MFMA tiles), the workgroup tile
//     128 x 128 (2 x 2 waves), and two workgroups share a CU (at most 256
//     registers per lane), so one workgroup's barriers and fetch waits are
//     covered by the other's MFMAs.
//   * Per 128-K block and wave: 4 MFMA tiles x 2 K steps of
//     v_mfma_f32_32x32x64_f8f6f4 (the first from a zero accumulator), then
//     acc = fma(part, sa * sb, acc) for the 16 values of each tile, sb being
//     the one scale of the tile's 128-column weight block.  The update of
//     tile q for block t is issued just before the MFMA that starts tile q
//     of block t+1 (which overwrites its partial sum), so the VALU work runs
//     beside the matrix core.
//   * Operands go global -> LDS directly (global_load_lds_dwordx4) into two
//     stages (A 16 KB + B 16 KB + the block's scales), with the fragment
//     swizzle and the three-phase fetch schedule of the 256 x 256 kernel;
//     XCD-aware tile order; the epilogue stages each wave's 64 x 64 block
//     through an idle stage buffer and stores whole 128-byte row segments.
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BBM = 128, BBN = 128, BBK = 128;
constexpr int CH = BBK / 16;                    // 16-byte chunks per LDS row
constexpr int NCA = BBM * CH / 256, NCB = BBN * CH / 256;  // fetches per thread per tile
constexpr int WM = BBM / 2, WN = BBN / 2;       // wave tile 64 x 64
constexpr int TMW = WM / 32, TNW = WN / 32;     // 2 x 2 MFMA tiles per wave
constexpr int NT = TMW * TNW;

struct BlockArgs {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;  // M x (K/128)
  const float* sb;  // ceil(N/128) x (K/128)
  int64_t M, N, K, lda, ldb, ldc;
  void* c;
  bool vec_c;
  int64_t tiles_m, tiles_n;
};

// 16-byte chunk c of LDS row r sits at position c ^ row_swizzle(r): the
// 16-byte fragment reads of 16 consecutive rows then cover all 64 banks.
__device__ __forceinline__ int row_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int ROWS>
__device__ __forceinline__ void chunk_offsets(uint32_t (&off)[ROWS * CH / 256], int64_t row0, int64_t nrows,
                                              int64_t ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < ROWS * CH / 256; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int row = slot / CH, pc = slot % CH;
    const int c = pc ^ row_swizzle(row);
    int64_t gr = row0 + row;
    if (gr > nrows - 1) gr = nrows - 1;
    off[i] = (uint32_t)(gr * ld + c * 16);
  }
}

template <int ROWS>
__device__ __forceinline__ void issue_tile(const uint8_t* base, const uint32_t (&off)[ROWS * CH / 256],
                                           int64_t k0, uint8_t* lds) {
  const int wave = threadIdx.x >> 6;
  const uint8_t* p = base + k0;
#pragma unroll
  for (int i = 0; i < ROWS * CH / 256; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(p + off[i]), (lds_ptr_t)(lds + (i * 4 + wave) * 1024), 16, 0, 0);
}

__device__ __forceinline__ v8i ffrag(const uint8_t* lds, int row_off, int slice, int c_lo, int c_hi) {
  const uint8_t* p = lds + row_off + slice * 32 * BBK;
  uint4 lo = *reinterpret_cast<const uint4*>(p + c_lo);
  uint4 hi = *reinterpret_cast<const uint4*>(p + c_hi);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

struct Frags {
  v8i a[TMW], b[TNW];
};

__shared__ __attribute__((aligned(1024))) uint8_t blk_a0[BBM * BBK];
__shared__ __attribute__((aligned(1024))) uint8_t blk_a1[BBM * BBK];
__shared__ __attribute__((aligned(1024))) uint8_t blk_b0[BBN * BBK];
__shared__ __attribute__((aligned(1024))) uint8_t blk_b1[BBN * BBK];
// scale slots: 64 per wave (waves 2-3 repeat the rows / block of waves 0-1)
__shared__ __attribute__((aligned(256))) float blk_sa0[256];
__shared__ __attribute__((aligned(256))) float blk_sa1[256];
__shared__ __attribute__((aligned(256))) float blk_sb0[256];
__shared__ __attribute__((aligned(256))) float blk_sb1[256];

template <int S>
__device__ __forceinline__ uint8_t* st_a() { return S ? blk_a1 : blk_a0; }
template <int S>
__device__ __forceinline__ uint8_t* st_b() { return S ? blk_b1 : blk_b0; }
template <int S>
__device__ __forceinline__ float* st_sa() { return S ? blk_sa1 : blk_sa0; }
template <int S>
__device__ __forceinline__ float* st_sb() { return S ? blk_sb1 : blk_sb0; }

// Scale rows of one 128 x 128 tile: thread t fetches sa of tile row t % 128
// and the scale of the tile's 128-column weight block.
struct ScaleRows {
  const float* sa_row;  // &sa[row * nkb]
  const float* sb_row;  // &sb[(n0 / 128) * nkb]
};

// Part 0 of a K tile's fetch: the A tile and the scales; part 1: the B tile.
template <int S, int PART>
__device__ __forceinline__ void issue_part(const BlockArgs& g, const uint32_t (&offa)[NCA], const uint32_t (&offb)[NCB],
                                           const ScaleRows& sr, int64_t kt) {
  const int wave = threadIdx.x >> 6;
  if constexpr (PART == 0) {
    issue_tile<BBM>(g.a, offa, kt * BBK, st_a<S>());
    __builtin_amdgcn_global_load_lds((const void*)(sr.sa_row + kt), (lds_ptr_t)(st_sa<S>() + wave * 64), 4, 0, 0);
    // every wave issues the same number of fetches (waves 2-3 repeat what
    // waves 0-1 fetch, into slots 128..255), so the vmcnt counts hold
    __builtin_amdgcn_global_load_lds((const void*)(sr.sb_row + kt), (lds_ptr_t)(st_sb<S>() + wave * 64), 4, 0, 0);
  } else {
    issue_tile<BBN>(g.b, offb, kt * BBK, st_b<S>());
  }
}

template <int S>
__device__ __forceinline__ void issue_stage(const BlockArgs& g, const uint32_t (&offa)[NCA], const uint32_t (&offb)[NCB],
                                            const ScaleRows& sr, int64_t kt) {
  issue_part<S, 0>(g, offa, offb, sr, kt);
  issue_part<S, 1>(g, offa, offb, sr, kt);
}

template <int S>
__device__ __forceinline__ void load_frags(Frags& f, int a_row_off, int b_row_off, int c_lo, int c_hi) {
#pragma unroll
  for (int i = 0; i < TMW; ++i) f.a[i] = ffrag(st_a<S>(), a_row_off, i, c_lo, c_hi);
#pragma unroll
  for (int j = 0; j < TNW; ++j) f.b[j] = ffrag(st_b<S>(), b_row_off, j, c_lo, c_hi);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// One K block's scale factors for this lane: sa of its row in each row tile
// times the tile's weight-block scale.
struct BlockScale {
  float s[TMW];
};

template <int S>
__device__ __forceinline__ void read_scales(BlockScale& bs, int a_srow) {
  const float sb = st_sb<S>()[0];
#pragma unroll
  for (int i = 0; i < TMW; ++i) bs.s[i] = st_sa<S>()[a_srow + i * 32] * sb;
}

// acc += part * s, as one fma per value (the expression of the general kernel)
__device__ __forceinline__ void promote(v16f& acc, const v16f& part, float s) {
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = __builtin_fmaf(part[v], s, acc[v]);
}

// MFMA Q of a K block (Q < NT: first 64-K step of tile Q, from a zero
// accumulator, preceded by the promotion of that tile's previous partial
// sum; Q >= NT: second step of tile Q - NT).
template <int Q, int FA, int FB>
__device__ __forceinline__ void block_mfma(v16f (&acc)[TMW][TNW], v16f (&part)[TMW][TNW], const Frags& f0,
                                           const Frags& f1, const BlockScale& bs_prev) {
  if constexpr (Q < NT) {
    constexpr int i = Q / TNW, j = Q % TNW;
    promote(acc[i][j], part[i][j], bs_prev.s[i]);
    part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f0.b[j], f0.a[i], (v16f){}, FB, FA, 0, 0, 0, 0);
  } else {
    constexpr int i = (Q - NT) / TNW, j = (Q - NT) % TNW;
    part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f1.b[j], f1.a[i], part[i][j], FB, FA, 0, 0, 0, 0);
  }
}

template <int LO, int HI, int FA, int FB>
__device__ __forceinline__ void mfma_seq(v16f (&acc)[TMW][TNW], v16f (&part)[TMW][TNW], const Frags& f0,
                                         const Frags& f1, const BlockScale& bs_prev) {
  if constexpr (LO < HI) {
    block_mfma<LO, FA, FB>(acc, part, f0, f1, bs_prev);
    mfma_seq<LO + 1, HI, FA, FB>(acc, part, f0, f1, bs_prev);
  }
}

template <int FA, int FB, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void gemm_block_kernel(BlockArgs g) {
  // the wave index in an SGPR: the per-wave offsets derived from it then need
  // no VGPR held across the K loop
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile coordinates: XCD-contiguous ranges, groups of 4 tile-rows
  const int64_t T = g.tiles_m * g.tiles_n;
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % 8, local = bid / 8;
  const int64_t per = T / 8, rem = T % 8;
  const int64_t logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  constexpr int64_t GM = 4;
  const int64_t per_group = GM * g.tiles_n;
  const int64_t first_m = (logical / per_group) * GM;
  const int64_t gsize = (g.tiles_m - first_m) < GM ? (g.tiles_m - first_m) : GM;
  const int64_t m0 = (first_m + (logical % per_group) % gsize) * BBM;
  const int64_t n0 = ((logical % per_group) / gsize) * BBN;
  const int64_t nk = g.K / BBK;  // even (checked by the launcher)

  const int a_row_off = (wm * WM + (lane & 31)) * BBK;
  const int b_row_off = (wn * WN + (lane & 31)) * BBK;
  const int h = lane >> 5, x7 = row_swizzle(lane & 31);
  const int c00 = ((0 + h) ^ x7) << 4, c01 = ((2 + h) ^ x7) << 4;
  const int c10 = ((4 + h) ^ x7) << 4, c11 = ((6 + h) ^ x7) << 4;
  const int a_srow = wm * WM + (lane & 31);

  uint32_t offa[NCA], offb[NCB];
  chunk_offsets<BBM>(offa, m0, g.M, g.lda);
  chunk_offsets<BBN>(offb, n0, g.N, g.ldb);
  ScaleRows sr;
  {
    int64_t ra = m0 + (threadIdx.x & (BBM - 1));
    if (ra > g.M - 1) ra = g.M - 1;
    sr.sa_row = g.sa + ra * nk;
    sr.sb_row = g.sb + (n0 / 128) * nk;
  }
  constexpr int P1 = 2, P2 = 4;  // MFMA split of the three phases (8 per K block)
  constexpr int NA = NCA + 2;    // fetch instructions of a part-0 issue
  constexpr int NS = NCA + NCB + 2;
  issue_stage<0>(g, offa, offb, sr, 0);
  issue_stage<1>(g, offa, offb, sr, 1);
  wait_vm_lgkm0<NS>();  // stage 0 landed

  v16f acc[TMW][TNW], part[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = part[i][j][v] = 0.0f;
  BlockScale bs_prev, bs_cur;
#pragma unroll
  for (int i = 0; i < TMW; ++i) bs_prev.s[i] = 0.0f;
  Frags f0, f1;
  lds_barrier();  // stage 0 is complete for every wave
  load_frags<0>(f0, a_row_off, b_row_off, c00, c01);

  // K block KT in stage S, as MFMAs 0..2*NT-1 (see block_mfma):
  //   phase 1: MFMAs 0..P1-1; second-step fragments and this block's scales
  //            read from S.
  //   phase 2: barrier; MFMAs P1..P1+P2-1; A tile and scales of KT+2 fetched
  //            into S.
  //   phase 3: wait for KT+1, barrier; the other MFMAs; first-step fragments
  //            of KT+1 read from S^1, B tile of KT+2 fetched into S.
  // Past the last block the fetch repeats the last block and is unused.
#define QSG_BLOCK_STEP(S, KT)                                                                   \
  {                                                                                             \
    load_frags<S>(f1, a_row_off, b_row_off, c10, c11);                                          \
    read_scales<S>(bs_cur, a_srow);                                                             \
    mfma_seq<0, P1, FA, FB>(acc, part, f0, f1, bs_prev);                                        \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    wait_vm_lgkm0<63>();                                                                        \
    lds_barrier();                                                                              \
    const int64_t nxt = (KT) + 2 < nk ? (KT) + 2 : nk - 1;                                      \
    issue_part<S, 0>(g, offa, offb, sr, nxt);                                                   \
    mfma_seq<P1, P1 + P2, FA, FB>(acc, part, f0, f1, bs_prev);                                  \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    wait_vm_lgkm0<NA>();                                                                        \
    lds_barrier();                                                                              \
    load_frags<S ^ 1>(f0, a_row_off, b_row_off, c00, c01);                                      \
    issue_part<S, 1>(g, offa, offb, sr, nxt);                                                   \
    mfma_seq<P1 + P2, 2 * NT, FA, FB>(acc, part, f0, f1, bs_prev);                              \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    bs_prev = bs_cur;                                                                           \
  }

  for (int64_t kt = 0; kt < nk; kt += 2) {
    QSG_BLOCK_STEP(0, kt)
    QSG_BLOCK_STEP(1, kt + 1)
  }
#undef QSG_BLOCK_STEP
  // the last block's partial sums
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) promote(acc[i][j], part[i][j], bs_prev.s[i]);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();  // every wave is done with the stages

  // ---- epilogue: each wave converts its 64 x 64 block into bands of 32
  // rows x 128 bytes in an idle stage buffer (padded row stride: bf16 136 B,
  // fp32 144 B, conflict-free accumulator writes), then stores 8 whole
  // 128-byte row segments per instruction.
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  constexpr int STRIDE = OUT_BF16 ? 136 : 144;
  constexpr int BCOLS = 128 / ESZ;
  constexpr int JPB = BCOLS / 32;
  static_assert(32 * STRIDE <= BBN * BBK, "band must fit a stage buffer");
  uint8_t* band = (wave == 0) ? blk_a0 : (wave == 1) ? blk_a1 : (wave == 2) ? blk_b0 : blk_b1;
  const int64_t bm0 = m0 + wm * WM, bn0 = n0 + wn * WN;
  const int sl = lane % 8, srw = lane / 8;
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
#pragma unroll
    for (int jb = 0; jb < TNW / JPB; ++jb) {
      const int r = lane & 31;
#pragma unroll
      for (int jj = 0; jj < JPB; ++jj) {
        const int j = jb * JPB + jj;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int col = jj * 32 + grp * 8 + (lane >> 5) * 4;
          const float v0 = acc[i][j][grp * 4 + 0], v1 = acc[i][j][grp * 4 + 1];
          const float v2 = acc[i][j][grp * 4 + 2], v3 = acc[i][j][grp * 4 + 3];
          uint8_t* dst = band + r * STRIDE + col * ESZ;
          if constexpr (OUT_BF16)
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          else
            *reinterpret_cast<uint4*>(dst) =
                make_uint4(__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's band writes are done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rr = 0; rr < 32; rr += 8) {
        const int rw = rr + srw;
        const int64_t m = bm0 + i * 32 + rw;
        const int64_t n = bn0 + jb * BCOLS + sl * (16 / ESZ);
        const uint4 v = *reinterpret_cast<const uint4*>(band + rw * STRIDE + sl * 16);
        if (m < g.M) {
          uint8_t* cp = reinterpret_cast<uint8_t*>(g.c) + (m * g.ldc + n) * ESZ;
          if (g.vec_c && n + 16 / ESZ <= g.N) {
            *reinterpret_cast<uint4*>(cp) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16 / ESZ; ++e) {
              if (n + e < g.N) {
                if constexpr (OUT_BF16)
                  reinterpret_cast<uint16_t*>(cp)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                else
                  reinterpret_cast<uint32_t*>(cp)[e] = w[e];
              }
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // band reads done before the next band overwrites it
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <int FA, int FB>
void launch_block_cfg(const BlockArgs& g, bool out_bf16, hipStream_t st) {
  const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_block_kernel<FA, FB, true>), dim3(grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_block_kernel<FA, FB, false>), dim3(grid), dim3(256), 0, st, g);
}

}  // namespace

bool launch_scaled_gemm_block_fast(const uint8_t* a, int fa, const float* sa, const uint8_t* b, int fb,
                                   const float* sb, bool w128, int64_t M, int64_t N, int64_t K, int64_t lda,
                                   int64_t ldb, void* c, int c_dtype, int64_t ldc, hipStream_t st) {
  // eligibility: 128 x 128 weight blocks, an even number of 128-K blocks,
  // 16-byte rows, 32-bit chunk offsets, 4-byte aligned scales, enough tiles
  // to fill the chip
  if (!w128) return false;
  if (K <= 0 || K % (2 * BBK) != 0) return false;
  if ((uintptr_t)a % 16 || (uintptr_t)b % 16 || lda % 16 || ldb % 16) return false;
  if (M * lda >= (int64_t)1 << 32 || N * ldb >= (int64_t)1 << 32) return false;
  if ((uintptr_t)sa % 4 || (uintptr_t)sb % 4) return false;
  const int64_t tiles_m = (M + BBM - 1) / BBM, tiles_n = (N + BBN - 1) / BBN;
  if (tiles_m * tiles_n < 512) return false;
  BlockArgs g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  const bool out_bf16 = (c_dtype == 1);
  g.vec_c = ((uintptr_t)c % 16 == 0) && ((ldc * (out_bf16 ? 2 : 4)) % 16 == 0);
  g.tiles_m = tiles_m;
  g.tiles_n = tiles_n;
  if (fa == kE4M3 && fb == kE4M3) launch_block_cfg<kE4M3, kE4M3>(g, out_bf16, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_block_cfg<kE5M2, kE4M3>(g, out_bf16, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_block_cfg<kE4M3, kE5M2>(g, out_bf16, st);
  else launch_block_cfg<kE5M2, kE5M2>(g, out_bf16, st);
  return true;
}

}  // namespace qsg
