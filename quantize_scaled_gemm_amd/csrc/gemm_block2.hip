// Large-tile FP8 GEMM with blockwise scales for gfx950, 16x16x128 matrix
// instructions:
//   C[m,n] = sum_kb (sum_{k in kb} A[m,k] B[n,k]) * sa[m,kb] * sb(n,kb)
// with 128-wide K blocks kb; sb(n,kb) = sb[n / 128, kb] (128 x 128 weight
// blocks: fprop, dgrad) or sb[n, kb] (1 x 128 blocks on both operands:
// wgrad along the tokens).  ("Low-Precision Training Guide", recipe
// "blockwise": 1 x 128 activation and 128 x 128 weight blocks with an fp32
// scale each; each K block's partial sum is scaled and added in fp32.)
//
// Design for MI355X.
//   * One v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-K scale block of a
//     16 x 16 output tile, so its result is the block's partial sum: it
//     starts from zero and is promoted at once (acc = fma(part, sa * sb,
//     acc)), so partial sums live only for the few instructions between the
//     MFMA and its fma and the running sums are the only per-tile state (4
//     VGPRs per 16 x 16 tile).  The promotion fma runs on the VALU beside the
//     matrix core, about half of the MFMA time.
//   * 256 x 256 x 128 workgroup tile, 512 threads = 8 wave64s (two per SIMD,
//     each one's VALU work and waits covered by the other's MFMAs), wave w
//     owning 64 A rows (w % 4) x 128 B rows (w / 4): 4 x 8 MFMA tiles, 128
//     accumulator VGPRs.  A K tile costs 64 KB of operand fetch and 192 KB of
//     fragment reads per 2048 MFMA cycles per SIMD.
//   * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds) into
//     two stages, with a row swizzle that keeps the 16 x 16 x 128 fragment
//     reads free of bank conflicts (see row_swizzle); one barrier per K tile,
//     after which K tile t + 1 is fetched into the stage tile t - 1 used (the
//     last K tile of an output tile fetches the next output tile's first).
//   * Scales: 16 bytes per row (4 K blocks of fp32 scale_inv) per group of 4
//     K tiles, one load instruction per wave, into two alternating group
//     buffers, one group ahead.  Waves 0-3 fetch the 256 A rows' sa, waves
//     4-7 the B rows' sb (1 x 128) or the two weight blocks' sb (128 x 128).
//   * Persistent workgroups in the XCD-aware tile order of the per-tensor
//     kernel; the results are stored straight from registers (8 bytes of
//     bf16 or 16 bytes of fp32 per lane and tile).
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTH = 512, NW = 8;                 // threads and waves per workgroup
constexpr int TI = 4, TJ = 8;                    // 16 x 16 MFMA tiles per wave (A rows x B rows)
constexpr int NCK = BM * (BK / 16) / NTH;        // 16-byte fetches per thread per operand tile (4)
constexpr int GROUP = 4;                         // K tiles per scale group

struct Block2Args {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;  // M x (K/128)
  const float* sb;  // W128: ceil(N/128) x (K/128); else N x (K/128)
  int64_t M, N, K, lda, ldb, ldc;
  void* c;
  bool vec_c;
  int64_t tiles_m, tiles_n;
};

// 16-byte chunk c of LDS row r sits at position c ^ row_swizzle(r), with the
// swizzle's bits 0, 1, 2 taken from row bits 1, 3, 2.  A fragment read
// (lane l: row l % 16, chunk l / 16 or 4 + l / 16) then hits 16 distinct
// 16-byte bank groups both within lanes 0-15 (all even or all odd rows get
// all 8 swizzle values) and within lanes {8p .. 8p + 7} u {8p + 32 .. 8p + 39},
// whose chunks differ by 2 (the 8 rows' swizzle values lie in distinct
// classes {x, x ^ 2}).
__device__ __forceinline__ int row_swizzle(int row) {
  return ((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 2) & 1) << 2);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t row0, int64_t nrows,
                                                           int64_t ld) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + row0 * ld;
  const int64_t n = nrows > row0 ? (nrows - row0) * ld : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)n, 0x00020000);
}

__shared__ __attribute__((aligned(1024))) uint8_t b2_a0[BM * BK];
__shared__ __attribute__((aligned(1024))) uint8_t b2_a1[BM * BK];
__shared__ __attribute__((aligned(1024))) uint8_t b2_b0[BN * BK];
__shared__ __attribute__((aligned(1024))) uint8_t b2_b1[BN * BK];
// scale groups: row r's 4 floats (K tiles 4g .. 4g + 3) at floats 4r .. 4r + 3
__shared__ __attribute__((aligned(1024))) float b2_sa0[BM * GROUP];
__shared__ __attribute__((aligned(1024))) float b2_sa1[BM * GROUP];
__shared__ __attribute__((aligned(1024))) float b2_sb0[BN * GROUP];
__shared__ __attribute__((aligned(1024))) float b2_sb1[BN * GROUP];

template <int S>
__device__ __forceinline__ uint8_t* st_a() { return S ? b2_a1 : b2_a0; }
template <int S>
__device__ __forceinline__ uint8_t* st_b() { return S ? b2_b1 : b2_b0; }
template <int G>
__device__ __forceinline__ float* gr_sa() { return G ? b2_sa1 : b2_sa0; }
template <int G>
__device__ __forceinline__ float* gr_sb() { return G ? b2_sb1 : b2_sb0; }

// Per-thread byte offsets (within a tile) of the chunks this thread fetches:
// instruction i of wave w fills 1 KB block i * 8 + w of the operand tile,
// lane L its 16-byte position L, i.e. tile row (i*8+w)*8 + L/8 at swizzled
// chunk L%8.
__device__ __forceinline__ void chunk_offsets(uint32_t (&off)[NCK], int64_t ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NCK; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int row = slot / 8, pc = slot % 8;
    off[i] = (uint32_t)(row * ld + ((pc ^ row_swizzle(row)) * 16));
  }
}

struct Res {
  __amdgpu_buffer_rsrc_t ra, rb, rs;  // A rows, B rows, this wave's scale rows
};

template <int S>
__device__ __forceinline__ void issue_tile(const Res& r, const uint32_t (&voa)[NCK], const uint32_t (&vob)[NCK],
                                           uint32_t wl, uint32_t kt) {
#pragma unroll
  for (int i = 0; i < NCK; ++i) dma16(r.ra, voa[i], kt * BK, st_a<S>() + i * NW * 1024 + wl);
#pragma unroll
  for (int i = 0; i < NCK; ++i) dma16(r.rb, vob[i], kt * BK, st_b<S>() + i * NW * 1024 + wl);
}

// Scale group g: waves 0-3 the A rows' 16 bytes, waves 4-7 the B side's.
template <int G>
__device__ __forceinline__ void issue_group(const Res& r, uint32_t vos, uint32_t wl, uint32_t g) {
  uint8_t* dst = (threadIdx.x >> 6) < 4 ? reinterpret_cast<uint8_t*>(gr_sa<G>()) + wl
                                        : reinterpret_cast<uint8_t*>(gr_sb<G>()) + wl - 4 * 1024;
  dma16(r.rs, vos, g * 16, dst);
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

// A 16-row fragment of the 16x16x128 instruction: lane l takes row l % 16 of
// the tile and the 16-byte chunks g and 4 + g of its 128-byte K row, g =
// l / 16 (both operands use the same K order, so the dot product is the
// block's sum).
__device__ __forceinline__ v8i frag16(const uint8_t* lds, int row_off, int c_lo, int c_hi) {
  const uint8_t* p = lds + row_off;
  const uint4 lo = *reinterpret_cast<const uint4*>(p + c_lo);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + c_hi);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int TN_>
__device__ __forceinline__ void tile_coords(const Block2Args& g, uint32_t logical, uint32_t& m0, uint32_t& n0) {
  constexpr uint32_t GM = 4;
  const uint32_t tm = (uint32_t)g.tiles_m, tn = (uint32_t)g.tiles_n;
  const uint32_t per_group = GM * tn;
  const uint32_t first_m = (logical / per_group) * GM;
  const uint32_t gsize = (tm - first_m) < GM ? (tm - first_m) : GM;
  m0 = (first_m + (logical % per_group) % gsize) * BM;
  n0 = ((logical % per_group) / gsize) * BN;
}

template <int FA, int FB, bool OUT_BF16, bool W128>
__global__ __launch_bounds__(NTH, 1) void gemm_block2_kernel(Block2Args g) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 3, wn = wave >> 2;

  // persistent workgroups over each XCD's contiguous range of tiles
  const uint32_t T = (uint32_t)(g.tiles_m * g.tiles_n);
  const uint32_t G = gridDim.x;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t per = T / 8, rem = T % 8;
  const uint32_t x_begin = xcd * per + (xcd < rem ? xcd : rem);
  const uint32_t x_end = x_begin + per + (xcd < rem ? 1 : 0);
  const uint32_t x_wgs = G / 8 + (xcd < G % 8 ? 1 : 0);
  uint32_t logical = x_begin + local;
  if (logical >= x_end) return;
  const uint32_t nk = (uint32_t)(g.K / BK);  // a multiple of 8 (checked by the launcher)
  const uint32_t ngrp = nk / GROUP;
  // B fragments are read PF fragments ahead of their MFMAs (the 1 x 128
  // layout holds 4 more scale factors per fragment and has no room for 2)
  constexpr int PF = W128 ? 2 : 1;
  // Fetch schedule: one barrier per K tile.  After it the other stage is
  // free (every wave has read its fragments), and the K tile's first
  // instructions fetch the next K tile into it; the wait before the barrier
  // at the end of the K tile completes it.
  const int64_t sstride = (g.K / BK) * 4;   // bytes per scale row

  // fragment addressing
  const int r16 = lane & 15, grp = lane >> 4, xs = row_swizzle(r16);
  const int c_lo = (grp ^ xs) << 4, c_hi = ((4 + grp) ^ xs) << 4;
  const int a_off = (wm * 64 + r16) * BK;    // + i * 16 * BK
  const int b_off = (wn * 128 + r16) * BK;   // + j * 16 * BK
  // scale rows of this lane: A row wm*64 + 16 i + r16; B rows (1 x 128)
  // wn*128 + 16 j + 4 grp + v, or weight block wn (128 x 128)
  const int sa_idx = (wm * 64 + r16) * GROUP;
  const int sb_idx = W128 ? wn * GROUP : (wn * 128 + 4 * grp) * GROUP;

  uint32_t voa[NCK], vob[NCK];
  chunk_offsets(voa, g.lda);
  chunk_offsets(vob, g.ldb);
  const uint32_t wl = (uint32_t)wave * 1024u;
  const uint32_t vos = (uint32_t)(((threadIdx.x & 255)) * sstride);  // scale row of this lane
  auto resources = [&](uint32_t tm0, uint32_t tn0) {
    Res r;
    r.ra = rows_rsrc(g.a, tm0, g.M, g.lda);
    r.rb = rows_rsrc(g.b, tn0, g.N, g.ldb);
    if (wave < 4) {
      r.rs = rows_rsrc(g.sa, tm0, g.M, sstride);
    } else if constexpr (W128) {
      const int64_t nb0 = tn0 / 128, nbl = (g.N + 127) / 128;
      r.rs = rows_rsrc(g.sb, nb0, nb0 + 2 < nbl ? nb0 + 2 : nbl, sstride);
    } else {
      r.rs = rows_rsrc(g.sb, tn0, g.N, sstride);
    }
    return r;
  };

  uint32_t m0, n0;
  tile_coords<0>(g, logical, m0, n0);
  Res cur = resources(m0, n0);
  issue_group<0>(cur, vos, wl, 0);
  issue_tile<0>(cur, voa, vob, wl, 0);
  wait_vm_lgkm0<0>();  // group 0 and K tile 0 landed (this wave's part)
  lds_barrier();

  v4f acc[TI][TJ];
  while (true) {
    const uint32_t nlogical = logical + x_wgs;
    const bool more = nlogical < x_end;
    uint32_t nm0 = m0, nn0 = n0;
    if (more) tile_coords<0>(g, nlogical, nm0, nn0);
    const Res nxt = resources(nm0, nn0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    // The partial sums of the previous B fragment (pp) and their scale
    // factors (pfa: A-row factors of their K tile; pfb: their B factors) are
    // promoted while the next fragment's MFMAs run: MFMA i of fragment j is
    // followed by the 4 fmas of pp[i], which read results 4 MFMAs old, so no
    // fma waits on the matrix core and the VALU work issues in the MFMAs'
    // shadow.  The first promotion of a tile adds 0 * 0.
    v4f pp[TI];
    float pfa[TI], pfb[4];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      pp[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
      pfa[i] = 0.0f;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) pfb[v] = 0.0f;

    // K tile KT in stage S; its scales are word KI of group buffer GB.
    //   1. the fetch of K tile KT + 1 into S ^ 1 (and, at KI == 1, of the
    //      next scale group), issued before any fragment read: issued after
    //      them, the global -> LDS loads wait for every read in flight;
    //   2. scale factors and the 4 A fragments; the B fragments PF ahead of
    //      their 4 MFMAs; the previous fragment's partial sums promoted
    //      between them;
    //   3. wait for this wave's fetches, barrier.
#define QSG_B2_STEP(S, KT, GB, KI)                                                                         \
  {                                                                                                        \
    {                                                                                                      \
      /* the next K tile into the other stage (free since the last barrier) */                             \
      const bool own = (KT) + 1 < nk;                                                                      \
      Res RES = own ? cur : nxt;                                                                           \
      uint32_t FK = own ? (KT) + 1 : 0;                                                                    \
      asm volatile("" : "+s"(RES.ra), "+s"(RES.rb), "+s"(FK));                                             \
      issue_tile<(S) ^ 1>(RES, voa, vob, wl, FK);                                                          \
      if constexpr ((KI) == 1) {                                                                           \
        const uint32_t ng = (KT) / GROUP + 1;                                                              \
        const bool sown = ng < ngrp;                                                                       \
        Res SR = sown ? cur : nxt;                                                                         \
        uint32_t SG = sown ? ng : 0;                                                                       \
        issue_group<(GB) ^ 1>(SR, vos, wl, SG);                                                            \
      }                                                                                                    \
    }                                                                                                      \
    float fa_[TI];                                                                                         \
    _Pragma("unroll") for (int i = 0; i < TI; ++i) fa_[i] = gr_sa<GB>()[sa_idx + i * 16 * GROUP + (KI)];   \
    float fb_w = 0.0f;                                                                                     \
    if constexpr (W128) fb_w = gr_sb<GB>()[sb_idx + (KI)];                                                 \
    v8i af[TI];                                                                                            \
    _Pragma("unroll") for (int i = 0; i < TI; ++i) af[i] = frag16(st_a<S>(), a_off + i * 16 * BK, c_lo, c_hi); \
    v8i bf = frag16(st_b<S>(), b_off, c_lo, c_hi);                                                         \
    v8i bn = bf;                                                                                           \
    if constexpr (PF == 2) bn = frag16(st_b<S>(), b_off + 16 * BK, c_lo, c_hi);                            \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j) {                                                       \
      v8i bnn = bn;                                                                                        \
      if (j + PF < TJ) bnn = frag16(st_b<S>(), b_off + (j + PF) * 16 * BK, c_lo, c_hi);                    \
      float fbv[4];                                                                                        \
      if constexpr (W128) {                                                                                \
        _Pragma("unroll") for (int v = 0; v < 4; ++v) fbv[v] = fb_w;                                       \
      } else {                                                                                             \
        _Pragma("unroll") for (int v = 0; v < 4; ++v)                                                      \
          fbv[v] = gr_sb<GB>()[sb_idx + (j * 16 + v) * GROUP + (KI)];                                      \
      }                                                                                                    \
      v4f part[TI];                                                                                        \
      _Pragma("unroll") for (int i = 0; i < TI; ++i) {                                                     \
        part[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], (v4f){0.0f, 0.0f, 0.0f, 0.0f}, \
                                                                   FB, FA, 0, 0, 0, 0);                    \
        if constexpr (W128) {                                                                              \
          const float f = pfa[i] * pfb[0];                                                                 \
          _Pragma("unroll") for (int v = 0; v < 4; ++v) acc[i][(j + TJ - 1) % TJ][v] = __builtin_fmaf(pp[i][v], f, acc[i][(j + TJ - 1) % TJ][v]); \
        } else {                                                                                           \
          _Pragma("unroll") for (int v = 0; v < 4; ++v)                                                    \
            acc[i][(j + TJ - 1) % TJ][v] = __builtin_fmaf(pp[i][v], pfa[i] * pfb[v], acc[i][(j + TJ - 1) % TJ][v]);                    \
        }                                                                                                  \
      }                                                                                                    \
      _Pragma("unroll") for (int q = 0; q < TI; ++q) {                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                 \
        __builtin_amdgcn_sched_group_barrier(0x002, W128 ? 5 : 8, 0);                                      \
      }                                                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                                                   \
      _Pragma("unroll") for (int i = 0; i < TI; ++i) {                                                     \
        pp[i] = part[i];                                                                                   \
        pfa[i] = fa_[i];                                                                                   \
      }                                                                                                    \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) pfb[v] = fbv[v];                                       \
      if constexpr (PF == 2) {                                                                             \
        bf = bn;                                                                                           \
        bn = bnn;                                                                                          \
      } else {                                                                                             \
        bf = bnn;                                                                                          \
      }                                                                                                    \
    }                                                                                                      \
    wait_vm_lgkm0<0>();                                                                                    \
    lds_barrier();                                                                                         \
  }

    uint32_t kt = 0;
    do {
      QSG_B2_STEP(0, kt, 0, 0)
      QSG_B2_STEP(1, kt + 1, 0, 1)
      QSG_B2_STEP(0, kt + 2, 0, 2)
      QSG_B2_STEP(1, kt + 3, 0, 3)
      QSG_B2_STEP(0, kt + 4, 1, 0)
      QSG_B2_STEP(1, kt + 5, 1, 1)
      QSG_B2_STEP(0, kt + 6, 1, 2)
      QSG_B2_STEP(1, kt + 7, 1, 3)
      kt += 8;
    } while (kt < nk);
#undef QSG_B2_STEP
    // the last fragment's partial sums
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][TJ - 1][v] = __builtin_fmaf(pp[i][v], pfa[i] * pfb[v], acc[i][TJ - 1][v]);

    // ---- epilogue: lane l of tile (i, j) holds row 16 i + l % 16 and the 4
    // columns 16 j + 4 (l / 16) .. + 3 of the wave's block ----
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    uint32_t em0 = m0, en0 = n0;
    int64_t ldc = g.ldc;
    uint8_t* cbase = reinterpret_cast<uint8_t*>(g.c);
    asm volatile("" : "+s"(em0), "+s"(en0), "+s"(ldc), "+s"(cbase));
    const int64_t rm = (int64_t)em0 + wm * 64 + r16;
    const int64_t cn = (int64_t)en0 + wn * 128 + 4 * grp;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t m = rm + i * 16;
      if (m < g.M) {
        uint8_t* rowp = cbase + m * ldc * ESZ;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int64_t n = cn + j * 16;
          const v4f v = acc[i][j];
          if (g.vec_c && n + 4 <= g.N) {
            if constexpr (OUT_BF16) {
              *reinterpret_cast<uint2*>(rowp + n * ESZ) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            } else {
              *reinterpret_cast<uint4*>(rowp + n * ESZ) =
                  make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
            }
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
    if (!more) {
      wait_vm_lgkm0<0>();  // the repeated fetches of the last step land before the workgroup ends
      break;
    }
    logical = nlogical;
    m0 = nm0;
    n0 = nn0;
    cur = nxt;
  }
}

int b2_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int FA, bool W128>
void launch_b2(const Block2Args& g, bool out_bf16, unsigned grid, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((gemm_block2_kernel<FA, kE4M3, true, W128>), dim3(grid), dim3(NTH), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_block2_kernel<FA, kE4M3, false, W128>), dim3(grid), dim3(NTH), 0, st, g);
}

}  // namespace

bool launch_scaled_gemm_block2(const uint8_t* a, int fa, const float* sa, const uint8_t* b, int fb, const float* sb,
                               bool w128, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                               int c_dtype, int64_t ldc, hipStream_t st) {
  // eligibility: E4M3 weights (B), whole pairs of scale groups (K % 1024),
  // 16-byte rows, 32-bit buffer offsets, 16-byte aligned scale rows, enough
  // tiles to fill the chip
  if (fb != kE4M3) return false;
  if (K <= 0 || K % (2 * GROUP * BK) != 0) return false;
  if ((uintptr_t)a % 16 || (uintptr_t)b % 16 || lda % 16 || ldb % 16) return false;
  if (M * lda >= (int64_t)1 << 32 || N * ldb >= (int64_t)1 << 32) return false;
  if ((uintptr_t)sa % 16 || (uintptr_t)sb % 16) return false;
  const int64_t sstride = (K / BK) * 4;
  if (M * sstride >= (int64_t)1 << 31 || N * sstride >= (int64_t)1 << 31) return false;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  if (tiles_m * tiles_n < 128) return false;
  Block2Args g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  const bool out_bf16 = (c_dtype == 1);
  g.vec_c = out_bf16 ? (((uintptr_t)c % 8 == 0) && (ldc % 4 == 0)) : (((uintptr_t)c % 16 == 0) && (ldc % 4 == 0));
  g.tiles_m = tiles_m;
  g.tiles_n = tiles_n;
  const int64_t T = tiles_m * tiles_n, cus = b2_cu_count();
  const unsigned grid = (unsigned)(T < cus ? T : cus);
  if (fa == kE4M3) {
    if (w128) launch_b2<kE4M3, true>(g, out_bf16, grid, st);
    else launch_b2<kE4M3, false>(g, out_bf16, grid, st);
  } else {
    if (w128) launch_b2<kE5M2, true>(g, out_bf16, grid, st);
    else launch_b2<kE5M2, false>(g, out_bf16, grid, st);
  }
  return true;
}

}  // namespace qsg
