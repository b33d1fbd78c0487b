// Large-tile scaled FP8 GEMM for gfx950 (per-tensor and MXFP8 scales):
//   C[m,n] = sum_k (A[m,k] sa) (B[n,k] sb),  A M x K, B N x K, K-contiguous.
// ("Low-Precision Training Guide", section "When to Use Low Precision": the
// FP8 GEMMs of a Linear; recipe "mxfp8": E8M0 scale per 1 x 32 block.)
//
// Design for MI355X.
//   * 256 x 256 x 128 workgroup tile, 256 threads = 4 wave64s in 2 x 2, each
//     wave 128 x 128 = 4 x 4 MFMA tiles of v_mfma(_scale)_f32_32x32x64_f8f6f4
//     (256 fp32 accumulators per lane).  At this tile size a workgroup needs
//     64 KB of operand data per 128-K step for 2048 MFMA cycles per SIMD, i.e.
//     32 B/clk/CU from L2, half of what a 128 x 128 tile needs.
//   * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds),
//     without passing through VGPRs.  Such a load writes lane L's 16 bytes to
//     LDS slot L of a 1 KB block, so the swizzled LDS layout (see
//     row_swizzle: the 16-byte fragment reads of 16 consecutive rows are
//     conflict-free) is produced by choosing, per lane, which (row, chunk) of
//     global memory it fetches; every load instruction covers 8 whole
//     128-byte row segments.  The buffer resource of a tile ends at the
//     matrix's last row, so rows past M / N read as zero (never stored).
//   * Two LDS stages (2 x 64 KB).  The vector-memory path moves ~60 B/clk/CU,
//     so a K tile's 64 KB occupies it for more than half of the tile's MFMA
//     time: the fetch of tile t+2 is spread over the middle and last phase of
//     tile t (three phases around two barriers per K tile, see the main
//     loop) instead of being issued in a burst, which would stall the
//     in-order wave behind a full load queue.
//   * MXFP8: the 4 E8M0 bytes of a row for the tile's 4 K blocks travel with
//     the tile (buffer_load_dword ... lds), or, where K allows, 16 bytes per
//     row for groups of 4 K tiles, read into registers once per group (see
//     GroupWords); lane half h shifts its row's word by
//     8h so that op_sel 0 / 2 pick the bytes of K blocks h / 2+h for the two
//     64-K MFMA steps (the MFMA operand K order: lane half h holds K
//     [16h, 16h+16) and [32+16h, 48+16h) of a step; the scale of lanes 0..31
//     covers K 0..31 and that of lanes 32..63 covers K 32..63).
//   * Persistent workgroups, one per CU.  Workgroup ids are dispatched
//     round-robin over the 8 XCDs; the workgroups of an XCD take turns over a
//     contiguous range of the tile order, walked in groups of 4 (or 8, see
//     tile_group_rows) tile-rows x all tile-columns, so the 32 tiles an XCD
//     runs at once share 4 A panels and 8 B panels (8 and 4) in its L2.  The
//     operand stream runs across tile boundaries: the last two K steps of a
//     tile fetch the next tile's first two K tiles, and the results are
//     stored straight from registers without waiting for any fetch, so the
//     next tile starts on operands that are already in LDS.
//   * A last round of tiles that would leave at least half the CUs idle runs
//     as a second launch of 256 x 128 tiles (each wave 128 x 64), twice as
//     many work items of half the size.
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int FBM = 256, FBN = 256, FBK = 128;
constexpr int CH = FBK / 16;  // 16-byte chunks per LDS row

struct FastArgs {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  int64_t M, N, K, lda, ldb, ldc;
  void* c;
  bool vec_c;
  bool accumulate;  // fp32 C only: C = fp32(C + result)
  int64_t tiles_m, tiles_n;
  int64_t max_wgs;  // persistent grid: one workgroup per CU
  uint32_t gm;      // tile-rows per group of the tile order
  const float* ta;  // NVFP4: the operands' per-tensor decode scales
  const float* tb;
};

// 16-byte chunk c of LDS row r is stored at position c ^ row_swizzle(r).  A
// 128-byte row covers half of the 64 four-byte banks, so rows r and r + 2
// share banks.  The LDS serves a 16-byte read for 16 lanes at a time, lanes
// 8p .. 8p+7 together with 8p+32 .. 8p+39 [measured with the bank-conflict
// counter]; in a fragment read those are rows 8p' .. 8p'+7 at chunk 2q
// (lanes < 32) and 2q + 1, which the swizzle puts on 16 distinct 16-byte
// bank groups.  (It also spreads any 16 consecutive rows at one chunk over
// all 64 banks.)
__device__ __forceinline__ int row_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }


// global -> LDS loads through buffer resources: lane L's 16 (or 4) bytes go
// to position L of the LDS block at `lds` (wave-uniform).  The resource of a
// tile starts at its first row and ends at the matrix's last row, so rows
// past M / N read as zero (their results are never stored) and the
// per-thread offsets do not depend on the tile.  The stages are distinct
// __shared__ objects, so the compiler needs no wait before reading one stage
// while loads into the other are in flight; the kernel orders the loads with
// counted vmcnt waits and barriers.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

constexpr int NCHUNK = FBM * CH / 256;  // fetch instructions per wave per operand tile
static_assert(FBM == FBN, "A and B tiles share the chunk mapping");

// Per-thread byte offsets, within a tile, of the chunks this thread fetches:
// instruction i of wave w fills 1 KB block i * 4 + w of a stage, lane L its
// 16-byte position L, i.e. tile row (i*4+w)*8 + L/8 at swizzled chunk L%8.
__device__ __forceinline__ void chunk_offsets(uint32_t (&off)[NCHUNK], int64_t ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NCHUNK; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int row = slot / CH, pc = slot % CH;
    off[i] = (uint32_t)(row * ld + ((pc ^ row_swizzle(row)) * 16));
  }
}

// The buffers of one 256 x 256 tile (A rows, B rows, and for MXFP8 their
// E8M0 rows).
struct TileRes {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
};

// Materializes a step's fetch resources where it starts (the selection is
// then scheduled with the first phase's MFMAs, not between the fetches).
template <bool MX>
__device__ __forceinline__ void pin_res(TileRes& t, uint32_t& k) {
  if constexpr (MX)
    asm volatile("" : "+s"(t.ra), "+s"(t.rb), "+s"(t.rsa), "+s"(t.rsb), "+s"(k));
  else
    asm volatile("" : "+s"(t.ra), "+s"(t.rb), "+s"(k));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t row0, int64_t nrows, int64_t ld) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + row0 * ld;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)((nrows - row0) * ld), 0x00020000);
}
// A 32-row fragment: `row_off` is the byte offset of this lane's row of the
// first 32-row slice, `c_lo` / `c_hi` the swizzled byte offsets of its two
// 16-byte chunks (the swizzle only depends on row & 7, which is the same for
// every 32-row slice), and slice i adds i * 32 rows as an immediate.
__device__ __forceinline__ v8i ffrag(const uint8_t* lds, int row_off, int slice, int c_lo, int c_hi) {
  const uint8_t* p = lds + row_off + slice * 32 * FBK;
  uint4 lo = *reinterpret_cast<const uint4*>(p + c_lo);
  uint4 hi = *reinterpret_cast<const uint4*>(p + c_hi);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// MFMA tiles per wave: TMW rows; TN columns (4: 256 x 256 workgroup tile,
// 2: 256 x 128, for the last partial round of tiles)
constexpr int TMW = FBM / 2 / 32;

template <int TN>
struct Frags {
  v8i a[TMW], b[TN];
  int sa[TMW], sb[TN];  // MX: E8M0 words (byte 0: first 64-K step, byte 2: second)
};

// The operand tiles of the two LDS stages are distinct __shared__ objects so
// that the compiler can tell reads of one stage from the in-flight
// global->LDS loads into the other (it then needs no vmcnt wait before them).
__shared__ __attribute__((aligned(1024))) uint8_t lds_a0[FBM * FBK];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a1[FBM * FBK];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b0[FBN * FBK];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b1[FBN * FBK];
__shared__ __attribute__((aligned(256))) uint32_t lds_sa0[FBM];
__shared__ __attribute__((aligned(256))) uint32_t lds_sa1[FBM];
__shared__ __attribute__((aligned(256))) uint32_t lds_sb0[FBN];
__shared__ __attribute__((aligned(256))) uint32_t lds_sb1[FBN];
// MXFP8 with grouped scale fetches: 16 bytes (4 K tiles) per row, two groups
// in flight; row r's word for K tile k of the group is word 4r + k
__shared__ __attribute__((aligned(1024))) uint32_t lds_gsa0[FBM * 4];
__shared__ __attribute__((aligned(1024))) uint32_t lds_gsa1[FBM * 4];
__shared__ __attribute__((aligned(1024))) uint32_t lds_gsb0[FBN * 4];
__shared__ __attribute__((aligned(1024))) uint32_t lds_gsb1[FBN * 4];

template <int S>
__device__ __forceinline__ uint8_t* stage_a() { return S ? lds_a1 : lds_a0; }
template <int S>
__device__ __forceinline__ uint8_t* stage_b() { return S ? lds_b1 : lds_b0; }
template <int S>
__device__ __forceinline__ uint32_t* stage_sa() { return S ? lds_sa1 : lds_sa0; }
template <int S>
__device__ __forceinline__ uint32_t* stage_sb() { return S ? lds_sb1 : lds_sb0; }
template <int GB>
__device__ __forceinline__ uint32_t* group_sa() { return GB ? lds_gsa1 : lds_gsa0; }
template <int GB>
__device__ __forceinline__ uint32_t* group_sb() { return GB ? lds_gsb1 : lds_gsb0; }

// Scale handling of a kernel instance: SC_NONE per-tensor (one scale pair in
// the epilogue); SC_MX E8M0 bytes fetched with every K tile (4 bytes per row);
// SC_MXG E8M0 bytes fetched once per group of 4 K tiles (16 bytes per row,
// a quarter of the fetch instructions, each covering 64 rows).
constexpr int SC_NONE = 0, SC_MX = 1, SC_MXG = 2;

// Fetch of K tile kt of a tile into stage S: part 0 = the A tile (+ MX
// scale words), part 1 = the B tile; `wl` is this wave's 1 KB block offset.
template <int S, int PART, int SC, int TN>
__device__ __forceinline__ void issue_part(const TileRes& t, const uint32_t (&voa)[NCHUNK],
                                           const uint32_t (&vob)[NCHUNK], uint32_t vos, uint32_t wl, uint32_t kt) {
  if constexpr (PART == 0) {
#pragma unroll
    for (int i = 0; i < NCHUNK; ++i) dma16(t.ra, voa[i], kt * FBK, stage_a<S>() + i * 4096 + wl);
    if constexpr (SC == SC_MX) {
      dma4(t.rsa, vos, kt * 4, stage_sa<S>() + wl / 16);
      dma4(t.rsb, vos, kt * 4, stage_sb<S>() + wl / 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NCHUNK * TN / 4; ++i) dma16(t.rb, vob[i], kt * FBK, stage_b<S>() + i * 4096 + wl);
  }
}

template <int S, int SC, int TN>
__device__ __forceinline__ void issue_stage(const TileRes& t, const uint32_t (&voa)[NCHUNK],
                                            const uint32_t (&vob)[NCHUNK], uint32_t vos, uint32_t wl, uint32_t kt) {
  issue_part<S, 0, SC, TN>(t, voa, vob, vos, wl, kt);
  issue_part<S, 1, SC, TN>(t, voa, vob, vos, wl, kt);
}

// SC_MXG: the E8M0 bytes of scale group grp (K tiles 4 grp .. 4 grp + 3) of
// the tile's 256 A rows and 256 B rows into group buffer GB: lane L of wave w
// fills slot 64 w + L with the 16 bytes of row grp_slot(64 w + L) (`vos`).
template <int GB>
__device__ __forceinline__ void issue_scale_group(const TileRes& t, uint32_t vos, uint32_t wl, uint32_t grp) {
  dma16(t.rsa, vos, grp * 16, reinterpret_cast<uint8_t*>(group_sa<GB>()) + wl);
  dma16(t.rsb, vos, grp * 16, reinterpret_cast<uint8_t*>(group_sb<GB>()) + wl);
}
// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence (a fence would also wait for the
// global->LDS loads in flight); the waits it needs are explicit.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// SC_MXG: the scale words of the current group, in registers.  The group
// buffers hold row r in 16-byte slot grp_slot(r), which swaps bit 3 of the
// row for rows with bit 5 set, so that one 16-byte read per lane of rows
// base + 32 h + (l & 31) (lane half h) meets 16 distinct bank groups in every
// set of lanes the LDS serves together (lanes 8p .. 8p+7 with 8p+32 .. 8p+39,
// and 16 consecutive lanes).  a[p] / b[p] hold, in lane half h, the 4 words
// (K tiles of the group) of row block 2p + h; a swap of the wave halves
// (v_permlane32_swap) gives every lane the words of blocks 2p and 2p + 1.
// (Reading one word per row and K tile instead puts rows r and r + 16 on one
// bank: a 2-way conflict on every scale read.)
__device__ __forceinline__ int grp_slot(int row) { return row ^ (((row >> 5) & 1) << 3); }

template <int TN>
struct GroupWords {
  u32x4 a[TMW / 2], b[(TN + 1) / 2];
};

// Fragments of one 64-K step from stage S, and for MXFP8 the scale words of
// the step's rows: from the stage's per-K-tile buffers (SC_MX) or word KI of
// the group's words (SC_MXG; read from group buffer GB at KI == 0).
template <int S, int SC, int GB, int KI, int TN>
__device__ __forceinline__ void load_frags(Frags<TN>& f, GroupWords<TN>& gw, int kk, int a_row_off, int b_row_off,
                                           int c_lo, int c_hi, int a_srow, int b_srow, int a_gs, int b_gs, int sh) {
  if constexpr (SC == SC_MXG) {
    // step 0 only: the word shifted by 8h serves both 64-K steps (op_sel 0
    // and 2 pick bytes h and 2 + h); step 1 copies it (mfma_range<..., 2>)
    if (kk == 0) {
      if constexpr (KI == 0) {
#pragma unroll
        for (int p = 0; p < TMW / 2; ++p)
          gw.a[p] = *reinterpret_cast<const u32x4*>(group_sa<GB>() + (a_gs + p * 64) * 4);
#pragma unroll
        for (int p = 0; p < (TN + 1) / 2; ++p)
          gw.b[p] = *reinterpret_cast<const u32x4*>(group_sb<GB>() + (b_gs + p * 64) * 4);
      }
#pragma unroll
      for (int p = 0; p < TMW / 2; ++p) {
        const auto w = __builtin_amdgcn_permlane32_swap(gw.a[p][KI], gw.a[p][KI], false, false);
        f.sa[2 * p] = (int)(w[0] >> sh);
        f.sa[2 * p + 1] = (int)(w[1] >> sh);
      }
#pragma unroll
      for (int p = 0; p < (TN + 1) / 2; ++p) {
        const auto w = __builtin_amdgcn_permlane32_swap(gw.b[p][KI], gw.b[p][KI], false, false);
        f.sb[2 * p] = (int)(w[0] >> sh);
        if (2 * p + 1 < TN) f.sb[2 * p + 1] = (int)(w[1] >> sh);
      }
    }
  } else if constexpr (SC == SC_MX) {
#pragma unroll
    for (int i = 0; i < TMW; ++i) f.sa[i] = (int)(stage_sa<S>()[a_srow + i * 32] >> sh);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.sb[j] = (int)(stage_sb<S>()[b_srow + j * 32] >> sh);
  }
  // the scale words first: the first MFMA needs them and the LDS returns reads in order
#pragma unroll
  for (int i = 0; i < TMW; ++i) f.a[i] = ffrag(stage_a<S>(), a_row_off, i, c_lo, c_hi);
#pragma unroll
  for (int j = 0; j < TN; ++j) f.b[j] = ffrag(stage_b<S>(), b_row_off, j, c_lo, c_hi);
}

// MFMAs LO..HI-1 of one 64-K step, MFMA q updating accumulator tile
// (q / TN, q % TN); OPS: the byte of the scale words (op_sel).
template <bool MX, int FA, int FB, int LO, int HI, int TN, int OPS = 0>
__device__ __forceinline__ void mfma_range(v16f (&acc)[TMW][TN], const Frags<TN>& f) {
#pragma unroll
  for (int q = LO; q < HI; ++q) {
    const int i = q / TN, j = q % TN;
    if constexpr (MX)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], FB, FA, OPS, f.sb[j], OPS, f.sa[i]);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], FB, FA, 0, 0, 0, 0);
  }
}

// The 16 accumulators of one 32 x 32 tile copied to VGPRs (keeps the
// accumulators in AGPRs for the register allocator).  The reads come as one
// block into 16 distinct registers, so the multiplies that follow find their
// inputs ready instead of each waiting for the read just before it.
__device__ __forceinline__ void acc_read16(const v16f& a, float (&o)[16]) {
#pragma unroll
  for (int q = 0; q < 16; q += 4)
    asm("v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\t"
        "v_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
        : "=v"(o[q]), "=v"(o[q + 1]), "=v"(o[q + 2]), "=v"(o[q + 3])
        : "a"(a[q]), "a"(a[q + 1]), "a"(a[q + 2]), "a"(a[q + 3]));
}

typedef __attribute__((address_space(1))) uint8_t gbyte;

// One 32 x 32 accumulator tile scaled by alpha and rearranged for 64-byte
// row stores.  In the tile, lane l holds row l % 32 and, for group g = 0..3,
// columns 8g + 4(l / 32) + 0..3.  For bf16 a swap between the lane halves
// (v_permlane32_swap) of groups 2p and 2p + 1 gives every lane 8 consecutive
// columns (16 bytes); fp32 groups are 16 bytes already.  A second swap
// between lanes l and l + 16 (v_permlane16_swap) of two such pieces makes 4
// lanes hold 64 contiguous bytes of one row: xs[pr] holds rows 0..15 and
// ys[pr] rows 16..31 of the 64-byte column pair pr (bf16: one pair, fp32:
// two).  All 16 reads come first, then all multiplies, then the conversions,
// so each stage uses results issued several instructions earlier.
template <bool OUT_BF16>
__device__ __forceinline__ void tile_pieces(const v16f& acc, float alpha, u32x4 (&xs)[OUT_BF16 ? 1 : 2],
                                            u32x4 (&ys)[OUT_BF16 ? 1 : 2]) {
  float v[16];
  acc_read16(acc, v);
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] *= alpha;
  constexpr int NPAIR = OUT_BF16 ? 1 : 2;
  u32x4 lo[2], hi[2];  // per pair: the 16-byte pieces before the row swap
  if constexpr (OUT_BF16) {
    uint32_t pk[4][2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      pk[gq][0] = pack_bf16x2(v[gq * 4 + 0], v[gq * 4 + 1]);
      pk[gq][1] = pack_bf16x2(v[gq * 4 + 2], v[gq * 4 + 3]);
    }
    // lane halves: lane l gets columns 8h .. 8h+7 (lo) and 16 + 8h .. (hi)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * p][0], pk[2 * p + 1][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * p][1], pk[2 * p + 1][1], false, false);
      (p == 0 ? lo[0] : hi[0]) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
  } else {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const u32x4 w = {__float_as_uint(v[gq * 4 + 0]), __float_as_uint(v[gq * 4 + 1]),
                       __float_as_uint(v[gq * 4 + 2]), __float_as_uint(v[gq * 4 + 3])};
      ((gq & 1) ? hi[gq >> 1] : lo[gq >> 1]) = w;
    }
  }
  // row swap: lanes 0-15 give their hi piece to lanes 16-31 for their lo
  // piece (and 32-47 / 48-63 alike), so that x holds rows 0-15 and y rows 16-31
#pragma unroll
  for (int pr = 0; pr < NPAIR; ++pr) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto sw = __builtin_amdgcn_permlane16_swap(lo[pr][d], hi[pr][d], false, false);
      xs[pr][d] = sw[0];
      ys[pr][d] = sw[1];
    }
  }
}

// Tile t of the XCD-aware order: workgroup ids are dispatched round-robin
// over the 8 XCDs, each XCD owns a contiguous range of the logical tile
// order, walked in groups of g.gm tile-rows x all tile-columns.
template <int TN>
__device__ __forceinline__ void tile_coords(const FastArgs& g, uint32_t logical, uint32_t& m0, uint32_t& n0) {
  const uint32_t GM = g.gm;
  const uint32_t tm = (uint32_t)g.tiles_m, tn = (uint32_t)g.tiles_n;
  const uint32_t per_group = GM * tn;
  const uint32_t first_m = (logical / per_group) * GM;
  const uint32_t gsize = (tm - first_m) < GM ? (tm - first_m) : GM;
  m0 = (first_m + (logical % per_group) % gsize) * FBM;
  n0 = ((logical % per_group) / gsize) * (TN * 64);
}

// Epilogue of one workgroup tile: scale by alpha, convert, store straight
// from registers (see tile_pieces); every store writes 16 rows x 64
// contiguous bytes.  (cm0, cn0): the tile's first row and column.
template <bool OUT_BF16, int TN>
__device__ __forceinline__ void store_tile(const FastArgs& g, v16f (&acc)[TMW][TN], float alpha, int64_t cm0,
                                           int64_t cn0, int wm, int wn, int lane) {
  constexpr int WM = FBM / 2, WN = TN * 32, TBN = TN * 64;
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  // tile coordinates made opaque here, so that no address below is
  // computed ahead of the K loop and kept live across it
  uint32_t em0 = (uint32_t)cm0, en0 = (uint32_t)cn0;
  int64_t ldc = g.ldc;
  gbyte* cbase = (gbyte*)g.c;
  asm volatile("" : "+s"(em0), "+s"(en0), "+s"(ldc), "+s"(cbase));
  const int64_t bm0 = (int64_t)em0 + wm * WM, bn0 = (int64_t)en0 + wn * WN;
  int elane = lane;
  asm volatile("" : "+v"(elane));
  const int eh = elane >> 5;
  const bool interior = g.vec_c && bm0 - wm * WM + FBM <= g.M && bn0 - wn * WN + TBN <= g.N;
  gbyte* const cw = cbase + (bm0 * ldc + bn0) * ESZ;  // wave-uniform
  // After the swaps below, a store writes 16 rows x 64 contiguous bytes:
  // lane l holds row (l % 16) (+16 for the second store of a pair) and the
  // 16-byte piece pidx = l / 32 + 2 ((l / 16) % 2) of the pair's 64 bytes.
  const int r16 = elane & 15, pidx = eh + 2 * ((elane >> 4) & 1);
  const uint32_t loff = ((uint32_t)r16 * (uint32_t)ldc * ESZ) + (uint32_t)pidx * 16;
  constexpr int NPAIR = OUT_BF16 ? 1 : 2;  // 64-byte column pairs per 32 x 32 tile
  if (interior) {
    // every piece of the workgroup's tile is inside C: straight-line code
    // with no per-tile branch, one scheduling region per accumulator tile
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 xs[NPAIR], ys[NPAIR];
        tile_pieces<OUT_BF16>(acc[i][j], alpha, xs, ys);
#pragma unroll
        for (int pr = 0; pr < NPAIR; ++pr) {
          const int cb = j * 32 * ESZ + pr * 64;  // byte column of the pair in the wave's block
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w = half ? ys[pr] : xs[pr];
            gbyte* const cp = cw + (int64_t)(i * 32 + 16 * half) * ldc * ESZ + cb + loff;
            if constexpr (!OUT_BF16) {
              if (g.accumulate) {
                const u32x4 o = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(cp);
#pragma unroll
                for (int d = 0; d < 4; ++d) w[d] = __float_as_uint(__uint_as_float(w[d]) + __uint_as_float(o[d]));
              }
            }
            *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(cp) = w;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 xs[NPAIR], ys[NPAIR];
        tile_pieces<OUT_BF16>(acc[i][j], alpha, xs, ys);
#pragma unroll
        for (int pr = 0; pr < NPAIR; ++pr) {
          const int cb = j * 32 * ESZ + pr * 64;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 w = half ? ys[pr] : xs[pr];
            gbyte* const cp = cw + (int64_t)(i * 32 + 16 * half) * ldc * ESZ + cb + loff;
            constexpr int PE = 16 / ESZ;  // elements per piece
            const int m = (int)bm0 + i * 32 + 16 * half + r16;
            const int n = (int)bn0 + cb / ESZ + pidx * PE;
            if (m < g.M) {
              if (g.vec_c && n + PE <= g.N) {
                if constexpr (!OUT_BF16) {
                  if (g.accumulate) {
                    const u32x4 o = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(cp);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                      w[d] = __float_as_uint(__uint_as_float(w[d]) + __uint_as_float(o[d]));
                  }
                }
                *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(cp) = w;
              } else {
#pragma unroll
                for (int e = 0; e < PE; ++e) {
                  if (n + e < g.N) {
                    if constexpr (OUT_BF16) {
                      reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(cp)[e] =
                          (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    } else {
                      auto* ce = reinterpret_cast<__attribute__((address_space(1))) float*>(cp) + e;
                      *ce = g.accumulate ? *ce + __uint_as_float(w[e]) : __uint_as_float(w[e]);
                    }
                  }
                }
              }
            }
          }
        }
      }
    }
  }
}

template <int SC, int FA, int FB, bool OUT_BF16, int TN>
__global__ __launch_bounds__(256, 1) void gemm_fast_kernel(FastArgs g) {
  constexpr bool MX = SC != SC_NONE;
  constexpr int WM = FBM / 2, WN = TN * 32;
  constexpr int NQ = TMW * TN;  // MFMAs per 64-K step
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Persistent workgroups: the ones on XCD x (ids x, x+8, ...) take turns
  // over XCD x's contiguous range of logical tiles.
  const uint32_t T = (uint32_t)(g.tiles_m * g.tiles_n);
  const uint32_t G = gridDim.x;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t per = T / 8, rem = T % 8;
  const uint32_t x_begin = xcd * per + (xcd < rem ? xcd : rem);
  const uint32_t x_end = x_begin + per + (xcd < rem ? 1 : 0);
  const uint32_t x_wgs = G / 8 + (xcd < G % 8 ? 1 : 0);
  uint32_t logical = x_begin + local;
  if (logical >= x_end) return;
  const uint32_t nk = (uint32_t)(g.K / FBK);  // even; SC_MXG: a multiple of 8 (checked by the launcher)
  const uint32_t nb = (uint32_t)(g.K / 32);   // MX: E8M0 bytes per row

  // fragment addressing: lane half h reads chunks kk*4 + h and kk*4 + 2 + h
  const int a_row_off = (wm * WM + (lane & 31)) * FBK;
  const int b_row_off = (wn * WN + (lane & 31)) * FBK;
  const int h = lane >> 5, x7 = row_swizzle(lane & 31);
  const int c00 = ((0 + h) ^ x7) << 4, c01 = ((2 + h) ^ x7) << 4;
  const int c10 = ((4 + h) ^ x7) << 4, c11 = ((6 + h) ^ x7) << 4;
  const int a_srow = wm * WM + (lane & 31), b_srow = wn * WN + (lane & 31);
  // SC_MXG: group-buffer slots of the rows of block h (lane half h)
  const int a_gs = grp_slot(a_srow + 32 * h), b_gs = grp_slot(b_srow + 32 * h);
  // MX: bytes h (first 64-K step) and 2 + h (second) of the row's word
  const int sh0 = 8 * h, sh1 = 8 * h + 16;
  constexpr int OPS1 = SC == SC_MXG ? 2 : 0;  // scale byte of the second 64-K step
  float alpha = 1.0f;
  if constexpr (!MX) alpha = *reinterpret_cast<const float*>(g.sa) * *reinterpret_cast<const float*>(g.sb);

  uint32_t voa[NCHUNK], vob[NCHUNK];
  chunk_offsets(voa, g.lda);
  chunk_offsets(vob, g.ldb);
  // scale row of this thread's fetch (SC_MXG: the row held by slot threadIdx.x)
  const uint32_t vos = (uint32_t)((SC == SC_MXG ? grp_slot(threadIdx.x) : (int)threadIdx.x) * nb);
  const uint32_t wl = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  auto resources = [&](uint32_t tm0, uint32_t tn0) {
    TileRes t;
    t.ra = rows_rsrc(g.a, tm0, g.M, g.lda);
    t.rb = rows_rsrc(g.b, tn0, g.N, g.ldb);
    if constexpr (MX) {
      t.rsa = rows_rsrc(g.sa, tm0, g.M, nb);
      t.rsb = rows_rsrc(g.sb, tn0, g.N, nb);
    }
    return t;
  };

  uint32_t m0, n0;
  tile_coords<TN>(g, logical, m0, n0);
  TileRes cur = resources(m0, n0);
  constexpr int P1 = TN == 4 ? 8 : 5, P2 = TN == 4 ? 8 : 3;
  constexpr int NA = NCHUNK + (SC == SC_MX ? 2 : 0);                 // fetches in a part-0 issue
  constexpr int NS = NCHUNK * (4 + TN) / 4 + (SC == SC_MX ? 2 : 0);  // fetches of a whole stage
  if constexpr (SC == SC_MXG) issue_scale_group<0>(cur, vos, wl, 0);  // lands with stage 0
  issue_stage<0, SC, TN>(cur, voa, vob, vos, wl, 0);
  issue_stage<1, SC, TN>(cur, voa, vob, vos, wl, 1);
  wait_vm_lgkm0<NS>();  // stage 0 landed
  lds_barrier();

  v16f acc[TMW][TN];
  Frags<TN> f0, f1;
  GroupWords<TN> gw;
  load_frags<0, SC, 0, 0, TN>(f0, gw, 0, a_row_off, b_row_off, c00, c01, a_srow, b_srow, a_gs, b_gs, sh0);
  while (true) {
    // The next tile's resources: the fetches of the last two K steps go to
    // its first two K tiles (or repeat this tile's, past the last tile), so
    // the operand stream runs on across the tile boundary.
    const int64_t cm0 = m0, cn0 = n0;
    const uint32_t nlogical = logical + x_wgs;
    const bool more = nlogical < x_end;
    uint32_t nm0 = m0, nn0 = n0;
    if (more) tile_coords<TN>(g, nlogical, nm0, nn0);
    const TileRes nxt_t = resources(nm0, nn0);
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // One K tile KT in stage S (f0 holds its first 64-K fragments), in three
  // phases around two barriers:
  //   1. MFMAs 0..P1-1 of f0; the second-step fragments f1 are read from S.
  //   2. barrier (every wave is done reading S); MFMAs P1..15 of f0 and
  //      0..P2-1 of f1; the A half of the K tile two ahead is fetched into S.
  //   3. wait for this wave's fetches of the next K tile, barrier (it is
  //      complete in S^1); MFMAs P2..15 of f1; the next K tile's first-step
  //      fragments are read from S^1 and the B half of the K tile two ahead
  //      is fetched into S.
  // Two ahead of the last K tiles are the next tile's first two.
#define QSG_FAST_STEP(S, KT, GB, KI)                                                           \
  {                                                                                            \
    const bool own = (KT) + 2 < nk;                                                            \
    TileRes RES = own ? cur : nxt_t;                                                           \
    uint32_t FK = own ? (KT) + 2 : (KT) + 2 - nk;                                              \
    pin_res<MX>(RES, FK);                                                                      \
    constexpr bool SGF = SC == SC_MXG && (KI) == 1;  /* this step fetches the next scale group */ \
    constexpr int NAS = NA + (SGF ? 2 : 0);                                                    \
    load_frags<S, SC, GB, KI, TN>(f1, gw, 1, a_row_off, b_row_off, c10, c11, a_srow, b_srow, a_gs, b_gs, sh1); \
    if constexpr (SC == SC_MXG) {                                                              \
      _Pragma("unroll") for (int i = 0; i < TMW; ++i) f1.sa[i] = f0.sa[i];                     \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) f1.sb[j] = f0.sb[j];                      \
    }                                                                                          \
    mfma_range<MX, FA, FB, 0, P1>(acc, f0);                                                    \
    _Pragma("unroll") for (int q = 0; q < P1 - 1; ++q) {                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TMW + TN) / (P1 - 1), 0);               \
    }                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    wait_vm_lgkm0<63>();                                                                       \
    lds_barrier();                                                                             \
    issue_part<S, 0, SC, TN>(RES, voa, vob, vos, wl, FK);                                      \
    if constexpr (SGF) {                                                                       \
      /* the next group of this tile, or the next tile's first group */                        \
      const uint32_t ng = (KT) / 4 + 1;                                                        \
      const bool sown = ng < nk / 4;                                                           \
      TileRes SRES = sown ? cur : nxt_t;                                                       \
      uint32_t SG = sown ? ng : 0;                                                             \
      pin_res<MX>(SRES, SG);                                                                   \
      issue_scale_group<(GB) ^ 1>(SRES, vos, wl, SG);                                          \
    }                                                                                          \
    mfma_range<MX, FA, FB, P1, NQ>(acc, f0);                                                   \
    mfma_range<MX, FA, FB, 0, P2, TN, OPS1>(acc, f1);                                          \
    _Pragma("unroll") for (int q = 0; q < (NAS < NQ - P1 + P2 ? NAS : NQ - P1 + P2); ++q) {    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);                                       \
      __builtin_amdgcn_sched_group_barrier(0x001, 3, 1);                                       \
    }                                                                                          \
    if constexpr (NQ - P1 + P2 > NAS)                                                          \
      __builtin_amdgcn_sched_group_barrier(0x008, NQ - P1 + P2 - NAS, 1);                      \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    wait_vm_lgkm0<NAS>();                                                                      \
    lds_barrier();                                                                             \
    load_frags<S ^ 1, SC, ((KI) == 3 ? (GB) ^ 1 : (GB)), (((KI) + 1) & 3), TN>(                \
        f0, gw, 0, a_row_off, b_row_off, c00, c01, a_srow, b_srow, a_gs, b_gs, sh0);          \
    issue_part<S, 1, SC, TN>(RES, voa, vob, vos, wl, FK);                                      \
    mfma_range<MX, FA, FB, P2, NQ, TN, OPS1>(acc, f1);                                         \
    _Pragma("unroll") for (int q = 0; q < NQ - P2 - 1; ++q) {                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TMW + TN) / (NQ - P2 - 1), 2);          \
      __builtin_amdgcn_sched_group_barrier(0x001, 3, 2);                                       \
    }                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);                                         \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }

    // nk >= 2: a do-while leaves the compiler no path that skips the loop
    // (merging the zeroed accumulators of such a path with the loop's costs
    // accumulator copies and spills in the epilogue).  With grouped scale
    // fetches one iteration covers two scale groups (8 K tiles), so the group
    // buffer of every step is a compile-time choice.
    uint32_t kt = 0;
    if constexpr (SC == SC_MXG) {
      do {
        QSG_FAST_STEP(0, kt, 0, 0)
        QSG_FAST_STEP(1, kt + 1, 0, 1)
        QSG_FAST_STEP(0, kt + 2, 0, 2)
        QSG_FAST_STEP(1, kt + 3, 0, 3)
        QSG_FAST_STEP(0, kt + 4, 1, 0)
        QSG_FAST_STEP(1, kt + 5, 1, 1)
        QSG_FAST_STEP(0, kt + 6, 1, 2)
        QSG_FAST_STEP(1, kt + 7, 1, 3)
        kt += 8;
      } while (kt < nk);
    } else {
      do {
        QSG_FAST_STEP(0, kt, 0, 0)
        QSG_FAST_STEP(1, kt + 1, 0, 0)
        kt += 2;
      } while (kt < nk);
    }
#undef QSG_FAST_STEP
    // The next tile's first K tile is in stage 0, its second on the way to
    // stage 1.  The epilogue stores from registers and waits for no fetch.
    // (The last step's reads of f0 are repeated after it, so that the
    // fragments are not held through the epilogue.)

    store_tile<OUT_BF16, TN>(g, acc, alpha, cm0, cn0, wm, wn, lane);
    if (!more) {
      wait_vm_lgkm0<0>();  // the repeated fetches of the last step land before the workgroup ends
      break;
    }
    logical = nlogical;
    m0 = nm0;
    n0 = nn0;
    cur = nxt_t;
    load_frags<0, SC, 0, 0, TN>(f0, gw, 0, a_row_off, b_row_off, c00, c01, a_srow, b_srow, a_gs, b_gs, sh0);
  }
}

// ---------------------------------------------------------------------------
// NVFP4 operands ("Low-Precision Training Guide": recipe "nvfp4", E2M1
// elements; NVIDIA's NVFP4 definition: one E4M3 decode scale per 16 elements
// along K and an fp32 decode scale per tensor):
//   C[m,n] = ta tb sum_k (dec(A[m,k]) Sa(m,k/16)) (dec(B[n,k]) Sb(n,k/16)).
// A block-scaled value dec(code) * S has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in f16; the products are exact in the
// f32 accumulation of v_mfma_f32_32x32x16_f16.  (gfx950's FP4 matrix
// instructions take power-of-two scales per 32 elements, which cannot carry
// an E4M3 scale per 16, and its scaled FP4 conversions use only the scale's
// exponent: the conversion runs with scale 1 and the block scale is applied
// by v_pk_mul_f16.)
//   * The same 256 x 256 workgroup tile, waves and LDS stages as the FP8
//     kernel: a K tile is 256 elements = 128 bytes of codes per row, fetched
//     global -> LDS with the FP8 chunk mapping and swizzle; the tile's 16
//     scale bytes per row travel to the group buffers (16 B per row, in the
//     slot order of GroupWords) and are read into registers once per K tile.
//   * Each wave decodes its own fragments from LDS.  For a 64-K chunk of a
//     K tile, lane half h reads the 16 bytes (32 codes) of K [32h, 32h + 32)
//     of its row with one ds_read_b128; step s = 0..3 of the chunk feeds
//     codes 8s .. 8s + 7 of them to the 16-K MFMA.  A and B lanes of the same
//     half see the same K, so the chunk's 64 K values are each multiplied
//     once; the steps' K order differs from the plain one, which only
//     changes the order of the f32 sums.  The two blocks a lane half covers
//     per chunk are scale bytes 2h (steps 0, 1) and 2h + 1 (steps 2, 3) of
//     the row's chunk word.
//   * Decoding step t + 1 (4 conversions + 4 packed multiplies per 8 values)
//     is interleaved with the 16 MFMAs of step t.  One barrier per K tile:
//     at step 12 every wave has read the tile's last chunk, the next K tile
//     has landed, the stage is refilled with the K tile two ahead, and the
//     next K tile's first chunk is read.
// ---------------------------------------------------------------------------
typedef _Float16 nv_h2 __attribute__((ext_vector_type(2)));
typedef _Float16 nv_h8 __attribute__((ext_vector_type(8)));

constexpr int NV_KT = 256;          // elements per K tile (FBK bytes of codes per row)
constexpr int NV_FETCHES = 2 * NCHUNK + 2;  // global -> LDS loads per thread per K tile

// 8 codes (element 2i in the low nibble of byte i) times the scale pair s2.
__device__ __forceinline__ nv_h8 nv_decode8(uint32_t w, nv_h2 s2) {
  const nv_h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const nv_h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const nv_h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const nv_h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return nv_h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The raw data of one 64-K chunk for this lane: 16 bytes of codes per
// fragment row, and the row's scale word shifted so that byte 0 / 1 are the
// blocks of steps 0-1 / 2-3.
struct NvChunk {
  u32x4 a[TMW], b[4];
  uint32_t sa[TMW], sb[4];
};

// Per-lane addressing of the NVFP4 kernel.
struct NvAddr {
  int slot[4];  // swizzled byte offset of chunk c's 16 bytes for this lane half
  int a_row_off, b_row_off, sh;
  int a_gs, b_gs;  // group-buffer slots of the rows of block h (lane half h)
};

// The row scale words of chunk c (0..3) come from the K tile's 16 scale bytes
// per row, read into gw at chunk 0 (two 16-byte reads per operand: lane half h
// takes row block 2p + h, from the bank-spread slot order of GroupWords) and
// exchanged between the wave halves per chunk.
template <int S>
__device__ __forceinline__ void nv_read_chunk(NvChunk& r, GroupWords<4>& gw, int c, int slot, const NvAddr& ad) {
#pragma unroll
  for (int i = 0; i < TMW; ++i)
    r.a[i] = *reinterpret_cast<const u32x4*>(stage_a<S>() + ad.a_row_off + i * 32 * FBK + slot);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r.b[j] = *reinterpret_cast<const u32x4*>(stage_b<S>() + ad.b_row_off + j * 32 * FBK + slot);
  if (c == 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      gw.a[p] = *reinterpret_cast<const u32x4*>(group_sa<S>() + (ad.a_gs + p * 64) * 4);
      gw.b[p] = *reinterpret_cast<const u32x4*>(group_sb<S>() + (ad.b_gs + p * 64) * 4);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const auto wa = __builtin_amdgcn_permlane32_swap(gw.a[p][c], gw.a[p][c], false, false);
    r.sa[2 * p] = wa[0] >> ad.sh;
    r.sa[2 * p + 1] = wa[1] >> ad.sh;
    const auto wb = __builtin_amdgcn_permlane32_swap(gw.b[p][c], gw.b[p][c], false, false);
    r.sb[2 * p] = wb[0] >> ad.sh;
    r.sb[2 * p + 1] = wb[1] >> ad.sh;
  }
}

// Fragments of step s (0..3) of a chunk.
__device__ __forceinline__ void nv_frags(const NvChunk& r, int s, nv_h8 (&fa)[TMW], nv_h8 (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
    const nv_h2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sa[i], 1.0f, false);
    const nv_h2 s2 = s < 2 ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
    fa[i] = nv_decode8(r.a[i][s], s2);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const nv_h2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sb[j], 1.0f, false);
    const nv_h2 s2 = s < 2 ? __builtin_shufflevector(sp, sp, 0, 0) : __builtin_shufflevector(sp, sp, 1, 1);
    fb[j] = nv_decode8(r.b[j][s], s2);
  }
}

// K tile kt of a tile into stage S: codes of A and B, then the 16 scale bytes
// of each row (lane L of wave w: row 64 w + L).
template <int S>
__device__ __forceinline__ void nv_issue(const TileRes& t, const uint32_t (&voa)[NCHUNK], const uint32_t (&vob)[NCHUNK],
                                         uint32_t vos, uint32_t wl, uint32_t kt) {
#pragma unroll
  for (int i = 0; i < NCHUNK; ++i) dma16(t.ra, voa[i], kt * FBK, stage_a<S>() + i * 4096 + wl);
#pragma unroll
  for (int i = 0; i < NCHUNK; ++i) dma16(t.rb, vob[i], kt * FBK, stage_b<S>() + i * 4096 + wl);
  dma16(t.rsa, vos, kt * 16, reinterpret_cast<uint8_t*>(group_sa<S>()) + wl);
  dma16(t.rsb, vos, kt * 16, reinterpret_cast<uint8_t*>(group_sb<S>()) + wl);
}

// One K tile in stage S.  On entry r0 holds its first chunk and (fa, fb) the
// fragments of its first step; on return r0 holds the next K tile's first
// chunk (stage S ^ 1) and (fa, fb) that K tile's first-step fragments.  At
// step 12 the stage is refilled with K tile fk of `res`.
template <int S>
__device__ __forceinline__ void nv_ktile(v16f (&acc)[TMW][4], NvChunk& r0, GroupWords<4>& gw, nv_h8 (&fa)[TMW],
                                         nv_h8 (&fb)[4], const NvAddr& ad, TileRes res, uint32_t fk, const uint32_t (&voa)[NCHUNK],
                                         const uint32_t (&vob)[NCHUNK], uint32_t vos, uint32_t wl) {
  NvChunk rc = r0, rn;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int c = t / 4, s = t % 4;
    if (s == 1 && c < 3) nv_read_chunk<S>(rn, gw, c + 1, ad.slot[c + 1], ad);
    if (t == 12) {
      pin_res<true>(res, fk);
      wait_vm_lgkm0<0>();
      lds_barrier();
      nv_issue<S>(res, voa, vob, vos, wl, fk);
      nv_read_chunk<S ^ 1>(r0, gw, 0, ad.slot[0], ad);
    }
    nv_h8 na[TMW], nb[4];
    if (t < 15)
      nv_frags((t + 1) % 4 == 0 ? rn : rc, (t + 1) % 4, na, nb);
    else
      nv_frags(r0, 0, na, nb);
#pragma unroll
    for (int q = 0; q < TMW * 4; ++q) {
      const int i = q / 4, j = q % 4;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < TMW * 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if ((t + 1) % 4 == 0 && t < 15) rc = rn;
#pragma unroll
    for (int i = 0; i < TMW; ++i) fa[i] = na[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = nb[j];
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_nvfp4_fast_kernel(FastArgs g) {
  constexpr int TN = 4, WM = FBM / 2, WN = TN * 32;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // persistent, XCD-aware tile order (as the FP8 kernel)
  const uint32_t T = (uint32_t)(g.tiles_m * g.tiles_n);
  const uint32_t G = gridDim.x;
  const uint32_t xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const uint32_t per = T / 8, rem = T % 8;
  const uint32_t x_begin = xcd * per + (xcd < rem ? xcd : rem);
  const uint32_t x_end = x_begin + per + (xcd < rem ? 1 : 0);
  const uint32_t x_wgs = G / 8 + (xcd < G % 8 ? 1 : 0);
  uint32_t logical = x_begin + local;
  if (logical >= x_end) return;
  const uint32_t nk = (uint32_t)(g.K / NV_KT);  // even (checked by the launcher)
  const uint32_t nsb = (uint32_t)(g.K / 16);    // scale bytes per row

  NvAddr ad;
  const int h = lane >> 5, x7 = row_swizzle(lane & 31);
#pragma unroll
  for (int c = 0; c < 4; ++c) ad.slot[c] = ((2 * c + h) ^ x7) << 4;
  ad.a_row_off = (wm * WM + (lane & 31)) * FBK;
  ad.b_row_off = (wn * WN + (lane & 31)) * FBK;
  ad.a_gs = grp_slot(wm * WM + 32 * h + (lane & 31));
  ad.b_gs = grp_slot(wn * WN + 32 * h + (lane & 31));
  ad.sh = 16 * h;
  const float alpha = *g.ta * *g.tb;

  uint32_t voa[NCHUNK], vob[NCHUNK];
  chunk_offsets(voa, g.lda);
  chunk_offsets(vob, g.ldb);
  const uint32_t vos = (uint32_t)(grp_slot(threadIdx.x) * nsb);  // the row held by slot threadIdx.x
  const uint32_t wl = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  auto resources = [&](uint32_t tm0, uint32_t tn0) {
    TileRes t;
    t.ra = rows_rsrc(g.a, tm0, g.M, g.lda);
    t.rb = rows_rsrc(g.b, tn0, g.N, g.ldb);
    t.rsa = rows_rsrc(g.sa, tm0, g.M, nsb);
    t.rsb = rows_rsrc(g.sb, tn0, g.N, nsb);
    return t;
  };

  uint32_t m0, n0;
  tile_coords<TN>(g, logical, m0, n0);
  TileRes cur = resources(m0, n0);
  nv_issue<0>(cur, voa, vob, vos, wl, 0);
  nv_issue<1>(cur, voa, vob, vos, wl, 1);
  wait_vm_lgkm0<NV_FETCHES>();  // stage 0 landed
  lds_barrier();

  v16f acc[TMW][TN];
  NvChunk r0;
  GroupWords<4> gw;
  nv_h8 fa[TMW], fb[TN];
  nv_read_chunk<0>(r0, gw, 0, ad.slot[0], ad);
  nv_frags(r0, 0, fa, fb);
  while (true) {
    const int64_t cm0 = m0, cn0 = n0;
    const uint32_t nlogical = logical + x_wgs;
    const bool more = nlogical < x_end;
    uint32_t nm0 = m0, nn0 = n0;
    if (more) tile_coords<TN>(g, nlogical, nm0, nn0);
    const TileRes nxt_t = resources(nm0, nn0);
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // K tiles kt (stage 0) and kt + 1 (stage 1); each refills its stage with
    // the K tile two ahead, which past the last one is the next tile's
    // first or second (or this tile's again after the last tile)
    uint32_t kt = 0;
    do {
      nv_ktile<0>(acc, r0, gw, fa, fb, ad, kt + 2 < nk ? cur : nxt_t, kt + 2 < nk ? kt + 2 : kt + 2 - nk, voa, vob, vos, wl);
      nv_ktile<1>(acc, r0, gw, fa, fb, ad, kt + 3 < nk ? cur : nxt_t, kt + 3 < nk ? kt + 3 : kt + 3 - nk, voa, vob, vos, wl);
      kt += 2;
    } while (kt < nk);
    store_tile<OUT_BF16, TN>(g, acc, alpha, cm0, cn0, wm, wn, lane);
    if (!more) {
      wait_vm_lgkm0<0>();  // the repeated fetches land before the workgroup ends
      break;
    }
    logical = nlogical;
    m0 = nm0;
    n0 = nn0;
    cur = nxt_t;
  }
}

int device_cu_count() {
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

// Tile-rows per group of the tile order.  The 32 tiles an XCD runs at once
// span gm tile-rows x 32 / gm tile-columns; 4 and 8 read the same panels per
// tile.  [measured, same-box A/Bs on two boxes] 8 is 1-3 % faster than 4
// where K is short and the output narrow (32768 x 4096 x 4096 fprop and
// dgrad) and 3-4 % slower on the long-K 32768 x 4096 x 14336 dgrad; 4
// elsewhere.
uint32_t tile_group_rows(int64_t K, int64_t tiles_n) { return (K <= 4096 && tiles_n <= 16) ? 8u : 4u; }

template <int SC, int FA, int FB>
void launch_fast_cfg(const FastArgs& g, bool out_bf16, int tn, hipStream_t st) {
  const int64_t tiles = g.tiles_m * g.tiles_n;
  const unsigned grid = (unsigned)(tiles < g.max_wgs ? tiles : g.max_wgs);
  if (tn == 4) {
    if (out_bf16)
      hipLaunchKernelGGL((gemm_fast_kernel<SC, FA, FB, true, 4>), dim3(grid), dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_fast_kernel<SC, FA, FB, false, 4>), dim3(grid), dim3(256), 0, st, g);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((gemm_fast_kernel<SC, FA, FB, true, 2>), dim3(grid), dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_fast_kernel<SC, FA, FB, false, 2>), dim3(grid), dim3(256), 0, st, g);
  }
}

template <int SC>
void launch_fast_fmt(const FastArgs& g, int fa, int fb, bool out_bf16, int tn, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_fast_cfg<SC, kE4M3, kE4M3>(g, out_bf16, tn, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_fast_cfg<SC, kE5M2, kE4M3>(g, out_bf16, tn, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_fast_cfg<SC, kE4M3, kE5M2>(g, out_bf16, tn, st);
  else launch_fast_cfg<SC, kE5M2, kE5M2>(g, out_bf16, tn, st);
}

}  // namespace

bool launch_scaled_gemm_fast(const uint8_t* a, int fa, bool mx, const void* sa, const uint8_t* b, int fb,
                             const void* sb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st) {
  // eligibility: whole 128-K tiles, 16-byte rows, 32-bit buffer offsets, enough tiles
  if (K <= 0 || K % (2 * FBK) != 0) return false;
  if ((uintptr_t)a % 16 || (uintptr_t)b % 16 || lda % 16 || ldb % 16) return false;
  if (M * lda >= (int64_t)1 << 32 || N * ldb >= (int64_t)1 << 32) return false;
  if (mx && ((uintptr_t)sa % 4 || (uintptr_t)sb % 4)) return false;
  const int64_t tiles_m = (M + FBM - 1) / FBM, tiles_n = (N + FBN - 1) / FBN;
  if (tiles_m * tiles_n < 128) return false;  // too few large tiles to fill the chip
  FastArgs g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  const bool out_bf16 = (c_dtype == 1);
  g.accumulate = accumulate && !out_bf16;
  const int esz = out_bf16 ? 2 : 4;
  // 16-byte row-segment stores need 16-byte aligned rows
  g.vec_c = ((uintptr_t)c % 16 == 0) && ((ldc * esz) % 16 == 0);
  g.tiles_m = tiles_m;
  g.tiles_n = tiles_n;
  g.max_wgs = device_cu_count();
  g.gm = tile_group_rows(K, tiles_n);
  // MXFP8 scale bytes in groups of 4 K tiles when whole pairs of groups fit
  // every tile's K (16-byte aligned rows of scale bytes)
  const bool mx_grouped = mx && K % (8 * FBK) == 0;
  auto launch = [&](const FastArgs& ga, int tn) {
    if (mx_grouped)
      launch_fast_fmt<SC_MXG>(ga, fa, fb, out_bf16, tn, st);
    else if (mx)
      launch_fast_fmt<SC_MX>(ga, fa, fb, out_bf16, tn, st);
    else
      launch_fast_fmt<SC_NONE>(ga, fa, fb, out_bf16, tn, st);
  };
  // A last round that would leave at least half of the workgroups idle, made
  // of whole tile-rows: those rows run as a second launch of 256 x 128 tiles
  // (twice as many, each half the work; every output element is computed the
  // same way, so the results do not change).
  const int64_t T = tiles_m * tiles_n, G = g.max_wgs, R = T % G;
  if (T > G && R > 0 && 2 * R <= G && R % tiles_n == 0) {
    const int64_t tail_rows = R / tiles_n;
    const int64_t m_main = (tiles_m - tail_rows) * FBM;
    FastArgs gm = g;
    gm.M = m_main;
    gm.tiles_m = tiles_m - tail_rows;
    launch(gm, 4);
    FastArgs gt = g;
    gt.a = a + m_main * lda;
    gt.c = reinterpret_cast<uint8_t*>(c) + m_main * ldc * esz;
    if (mx) gt.sa = reinterpret_cast<const uint8_t*>(sa) + m_main * (K / 32);
    gt.M = M - m_main;
    gt.tiles_m = tail_rows;
    gt.tiles_n = (N + 127) / 128;
    launch(gt, 2);
  } else {
    launch(g, 4);
  }
  return true;
}

bool launch_gemm_nvfp4_fast(const uint8_t* a, const uint8_t* sa, const float* ta, const uint8_t* b, const uint8_t* sb,
                            const float* tb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, void* c,
                            int c_dtype, int64_t ldc, hipStream_t st) {
  // eligibility: whole pairs of 256-K tiles, 16-byte rows of codes and of
  // scale bytes, 32-bit buffer offsets, enough tiles to fill the chip
  if (K <= 0 || K % (2 * NV_KT) != 0) return false;
  if ((uintptr_t)a % 16 || (uintptr_t)b % 16 || lda % 16 || ldb % 16) return false;
  if ((uintptr_t)sa % 16 || (uintptr_t)sb % 16) return false;
  if (M * lda >= (int64_t)1 << 32 || N * ldb >= (int64_t)1 << 32) return false;
  if (M * (K / 16) >= (int64_t)1 << 32 || N * (K / 16) >= (int64_t)1 << 32) return false;
  const int64_t tiles_m = (M + FBM - 1) / FBM, tiles_n = (N + FBN - 1) / FBN;
  if (tiles_m * tiles_n < 128) return false;
  FastArgs g{};
  g.a = a; g.b = b; g.sa = sa; g.sb = sb; g.ta = ta; g.tb = tb;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c = c;
  const bool out_bf16 = (c_dtype == 1);
  const int esz = out_bf16 ? 2 : 4;
  g.vec_c = ((uintptr_t)c % 16 == 0) && ((ldc * esz) % 16 == 0);
  g.tiles_m = tiles_m;
  g.tiles_n = tiles_n;
  g.max_wgs = device_cu_count();
  g.gm = 4;
  const int64_t tiles = tiles_m * tiles_n;
  const unsigned grid = (unsigned)(tiles < g.max_wgs ? tiles : g.max_wgs);
  if (out_bf16)
    hipLaunchKernelGGL(gemm_nvfp4_fast_kernel<true>, dim3(grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(gemm_nvfp4_fast_kernel<false>, dim3(grid), dim3(256), 0, st, g);
  return true;
}

}  // namespace qsg
