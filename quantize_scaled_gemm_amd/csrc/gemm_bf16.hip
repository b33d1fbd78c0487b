// Weight-gradient GEMM in bf16 ("Low-Precision Training Guide", knob
// --fp8-wgrad False: the wgrad GEMM stays in higher precision while fprop
// and dgrad run in FP8):
//
//   C[n, k] (=, +=) sum_t dY[t, n] * X[t, k],   dY T x N, X T x K, bf16, row-major,
//
// fp32 accumulation, C N x K in bf16 (rounded to nearest even) or fp32 (the
// fp32 main gradient, optionally accumulated: C = fp32(C + result)).
//
// Two kernels.  Operands with 16-byte aligned rows and N, K multiples of 8
// (every Linear layer's) take gemm_wgrad_bf16_dma_kernel further down: direct
// global -> LDS loads and LDS transpose reads.  Any other shape or alignment
// takes the general kernel below.
//
// General kernel, designed for gfx950.  The contraction runs over the tokens
// t, the slow dimension of both operands, so the kernel transposes on the way
// into LDS:
//   * 256 x 256 output tile per workgroup of 256 threads (4 waves of 128 x 128,
//     4 x 4 v_mfma_f32_32x32x16_bf16 each, 256 accumulators per lane), 64
//     tokens per K step: every 32-cycle MFMA needs 0.5 KB of fragment reads,
//     so fragment reads and the transposed writes fit in the LDS bandwidth.
//   * Threads 0-127 load dY, 128-255 load X: thread u holds the 8 x 8 blocks of
//     tokens 8 (u % 4) .. +7 and 8 (u % 4 + 4) .. +7 and features
//     8 (u / 4) .. +7 of the step's 64 x 256 tile (sixteen 16-byte loads; the
//     64 lanes of a wave cover 4 token rows x 256 contiguous bytes per load
//     instruction).  Two blocks are in flight
//     per thread, and two LDS stages: while the MFMAs of step s run, the
//     block of step s + 1 is transposed into the other stage and the block
//     of step s + 2 fetched; one barrier per step.
//   * The 8 x 8 block is transposed in registers (32 v_perm_b32, pairs of
//     16-bit halves) and written as 8 rows of 16 bytes into an LDS tile
//     [feature][64 tokens] (128-byte rows); 16-byte chunk c of row f sits at
//     position c ^ ((f >> 1) & 7), so a fragment read (16 lanes, 16
//     consecutive features, one chunk) touches all 64 banks once.
//   * MFMA operands are then 16-byte LDS reads: lane l supplies feature
//     l % 32 of its block and tokens 8 (l / 32) .. +7 of a 16-token MFMA step,
//     for both operands (any consistent split of the 16 tokens between the
//     lane halves gives the same dot products).
// Tokens past T and features past N / K are read as zero; results outside C
// are not stored.  Operands whose rows are not 16-byte aligned take an
// element-wise load path.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int WT = 256;    // output tile (features of dY x features of X)
constexpr int BT = 64;     // tokens per K step
constexpr int ROWB = BT * 2;  // bytes per LDS row (one feature, 64 tokens: 8 chunks of 16 bytes)

struct Bf16Args {
  const uint16_t* dy;
  const uint16_t* x;
  int64_t T, N, K, lddy, ldx, ldc;
  void* c;
  bool vec;         // 16-byte loads of both operands
  bool out_bf16;
  bool accumulate;  // fp32 C only
};

// chunk c of row f at position c ^ ((f >> 1) & 7): 16 lanes reading one chunk
// of 16 consecutive rows (128-byte rows: 2 rows per 64 banks) hit every bank once
__device__ __forceinline__ int swz(int f, int chunk) { return chunk ^ ((f >> 1) & 7); }

// 8 x 8 block of bf16 (rows = tokens, 16 bytes each) of operand p at token
// t0, feature f0 (row-major, leading dimension ld); out-of-range -> 0.
__device__ __forceinline__ void load_block(const uint16_t* p, int64_t ld, int64_t t0, int64_t f0, int64_t T,
                                           int64_t F, bool vec, u32x4 (&r)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + i;
    if (vec && t < T && f0 + 8 <= F) {
      r[i] = ld_stream16(p + t * ld + f0);
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (t < T) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (f0 + e < F) w[e >> 1] |= (uint32_t)p[t * ld + f0 + e] << (16 * (e & 1));
      }
      r[i] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// Transpose the 8 x 8 block (r[token] = 8 features) and store feature rows:
// row (frow + j) gets the 8 tokens of feature j as chunk `chunk`.
__device__ __forceinline__ void store_block_t(uint8_t* lds, int frow, int chunk, const u32x4 (&r)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high / low halves of the pair
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(r[2 * p + 1][j >> 1], r[2 * p][j >> 1], sel);
    const int f = frow + j;
    *reinterpret_cast<u32x4*>(lds + f * ROWB + swz(f, chunk) * 16) = o;
  }
}

__global__ __launch_bounds__(256, 1) void gemm_wgrad_bf16_kernel(Bf16Args g) {
  // two stages: step s writes stage s & 1 while slower waves may still read
  // the other, so one barrier per step suffices
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][WT * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][WT * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.y * WT, k0 = (int64_t)blockIdx.x * WT;
  // loader role: two 8-token x 8-feature blocks per step (tokens 8 tg.. and
  // 8 (tg + 4).., features 8 fg..)
  const bool is_b = tid >= 128;
  const int u = tid & 127, tg = u & 3, fg = u >> 2;
  const uint16_t* src = is_b ? g.x : g.dy;
  const int64_t ld = is_b ? g.ldx : g.lddy;
  const int64_t F = is_b ? g.K : g.N;
  const int64_t fbase = (is_b ? k0 : n0) + fg * 8;
  // MFMA role: wave (wn, wk) owns features wn*128.. of dY and wk*128.. of X
  const int wn = wave >> 1, wk = wave & 1;

  const int64_t nsteps = (g.T + BT - 1) / BT;
  v16f acc[4][4];
  // One K step s, on the block already in LDS stage s & 1: the block of step
  // s + 1 (registers RN) is transposed into the other stage and the block of
  // step s + 2 fetched into the registers RF (those of step s, stored one step
  // earlier) while the MFMAs of step s run; then one barrier.  A stage is
  // rewritten two steps after it was read, behind that barrier.  FIRST: the
  // first MFMA of each accumulator tile starts from C = 0 (the accumulators
  // get their first values from MFMAs, not from zero constants merged in at a
  // loop head, which would make the register allocator copy them through
  // VGPRs).
  auto step = [&](u32x4 (&RN)[2][8], u32x4 (&RF)[2][8], int64_t s, auto first, auto stage) {
    constexpr int ST = decltype(stage)::value;
    if (s + 1 < nsteps) {
      store_block_t(is_b ? lds_b[ST ^ 1] : lds_a[ST ^ 1], fg * 8, tg, RN[0]);
      store_block_t(is_b ? lds_b[ST ^ 1] : lds_a[ST ^ 1], fg * 8, tg + 4, RN[1]);
    }
    if (s + 2 < nsteps) {
      load_block(src, ld, (s + 2) * BT + tg * 8, fbase, g.T, F, g.vec, RF[0]);
      load_block(src, ld, (s + 2) * BT + (tg + 4) * 8, fbase, g.T, F, g.vec, RF[1]);
    }
#pragma unroll
    for (int ks = 0; ks < BT / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = wn * 128 + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const bf16x8*>(lds_a[ST] + f * ROWB + swz(f, chunk) * 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = wk * 128 + j * 32 + (lane & 31);
        fb[j] = *reinterpret_cast<const bf16x8*>(lds_b[ST] + f * ROWB + swz(f, chunk) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (decltype(first)::value && ks == 0) {
            const v16f z = {};
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], z, 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  };
  if (nsteps == 0) {
    // no tokens: the result is +0 (written, or added to the fp32 C)
    for (int e = tid; e < WT * WT; e += 256) {
      const int64_t n = n0 + e / WT, k = k0 + e % WT;
      if (n >= g.N || k >= g.K) continue;
      if (g.out_bf16) {
        reinterpret_cast<uint16_t*>(g.c)[n * g.ldc + k] = 0;
      } else {
        float* cp = reinterpret_cast<float*>(g.c) + n * g.ldc + k;
        *cp = g.accumulate ? *cp + 0.0f : 0.0f;
      }
    }
    return;
  }
  // two register blocks in flight: even steps' blocks in r0, odd steps' in r1
  u32x4 r0[2][8], r1[2][8];
  load_block(src, ld, (int64_t)tg * 8, fbase, g.T, F, g.vec, r0[0]);
  load_block(src, ld, (int64_t)(tg + 4) * 8, fbase, g.T, F, g.vec, r0[1]);
  if (nsteps > 1) {
    load_block(src, ld, BT + (int64_t)tg * 8, fbase, g.T, F, g.vec, r1[0]);
    load_block(src, ld, BT + (int64_t)(tg + 4) * 8, fbase, g.T, F, g.vec, r1[1]);
  }
  store_block_t(is_b ? lds_b[0] : lds_a[0], fg * 8, tg, r0[0]);
  store_block_t(is_b ? lds_b[0] : lds_a[0], fg * 8, tg + 4, r0[1]);
  __syncthreads();
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  step(r1, r0, 0, std::true_type{}, S0{});
  int64_t s = 1;
  while (s < nsteps) {
    step(r0, r1, s, std::false_type{}, S1{});
    if (++s >= nsteps) break;
    step(r1, r0, s, std::false_type{}, S0{});
    ++s;
  }

  // accumulator tile (i, j): lane l holds column k = l % 32 and rows
  // n = 8 (v / 4) + 4 (l / 32) + v % 4 of its 32 x 32 block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = k0 + wk * 128 + j * 32 + (lane & 31);
      if (k >= g.K) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t n = n0 + wn * 128 + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
        if (n >= g.N) continue;
        float val;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(val) : "a"(acc[i][j][v]));
        if (g.out_bf16) {
          reinterpret_cast<uint16_t*>(g.c)[n * g.ldc + k] = (uint16_t)(pack_bf16x2(val, 0.0f) & 0xFFFF);
        } else {
          float* cp = reinterpret_cast<float*>(g.c) + n * g.ldc + k;
          *cp = g.accumulate ? *cp + val : val;
        }
      }
    }
}

// ---- Aligned operands: global -> LDS directly, LDS transpose reads ----
//
// When both operands have 16-byte aligned rows and N, K are multiples of 8,
// the tiles go into LDS as they lie in memory (buffer_load_dwordx4 ... lds)
// and gfx950's LDS transpose read (ds_read_b64_tr_b16) forms the MFMA
// operands, so no VGPRs stage the loads and nothing is transposed in
// registers:
//   * 48 tokens per step, a ring of 3 LDS stages of 48 x 256 per operand
//     (512-byte token rows, 144 KB in all); the loads of step s + 2 are
//     issued while the MFMAs of step s run, and a counted vmcnt wait plus a
//     barrier at the end of step s makes step s + 1 visible.
//   * Each wave issues 12 loads per step (6 per operand), each filling a
//     1 KB block (2 token rows) of a stage; lane L fills position L % 32 of
//     row L / 32, i.e. it fetches chunk (L % 32) ^ (4 (t % 4)) of token t.
//   * Edges without branches: a step's buffer resource covers only the
//     step's token rows that exist (none past the last step), and a lane
//     whose 8 features lie past N / K gets an offset past the resource; both
//     read as zero.
//   * One ds_read_b64_tr_b16 transposes 4 x 4 blocks of 16-bit values within
//     each 16-lane group: lane 4 e + q supplies 4 features of token e, and
//     lane 4 q + r receives feature r of tokens 0..3.  Two such reads, 4
//     token rows apart, give lane l tokens 8 (l / 32) .. +7 of feature l % 32
//     of a 32-feature block: the operand layout of the 32x32x16 MFMA.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int DT = 48;                // tokens per step
constexpr int DROWB = WT * 2;         // bytes per LDS row (one token, 256 features)
constexpr int DOP = DT * DROWB;       // bytes per operand per stage
constexpr int DLOADS = DOP / 1024 / 4;  // 1 KB loads per wave per operand per step
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;  // past any step's resource (< 2^31 bytes)

// chunk c of token row t at position c ^ (4 (t % 4)): the 4 consecutive
// token rows x 4 chunks that 32 lanes of a transpose read touch land on 16
// different 16-byte bank groups
__device__ __forceinline__ int tswz(int t, int chunk) { return chunk ^ ((t & 3) << 2); }

// Byte offset, within an operand's stage, of what lane `lane` supplies to the
// transpose reads of features fblk .. fblk + 31, tokens 0 .. 15: lane
// 16 g + 4 e + q reads token 8 (g / 2) + e, features fblk + 16 (g % 2) + 4 q
// .. + 3 (and, 4 rows further, token 8 (g / 2) + 4 + e).
__device__ __forceinline__ int tr_offset(int fblk, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const int t = 8 * (g >> 1) + e;
  const int c = (fblk >> 3) + 2 * (g & 1) + (q >> 1);
  return t * DROWB + tswz(t, c) * 16 + (q & 1) * 8;
}

__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * DROWB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Resource over the token rows of step `step` that exist, starting at
// feature f0 of operand p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const uint16_t* p, int64_t ld, int64_t f0, int64_t T,
                                                            int64_t step) {
  int64_t rows = T - step * DT;
  rows = rows < 0 ? 0 : (rows > DT ? DT : rows);
  const uint16_t* b = p + step * DT * ld + f0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)b, 0, (int)(rows * ld * 2), 0x00020000);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence (a fence would also wait for the
// global -> LDS loads in flight); the waits it needs are explicit.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Output tile of workgroup b (1-D grid of nx * ny).  Workgroups go to the 8
// XCDs round-robin (b % 8), each XCD with its own L2, so XCD j is given the
// j-th eighth of a tile order that walks groups of 4 tile rows column by
// column: the 32 tiles an XCD runs at once on a 16 x 16 grid span 4 dY and
// 8 X panels (12 panels, instead of 18 in row-major order).
__device__ __forceinline__ void tile_of(int b, int nx, int ny, int& tx, int& ty) {
  constexpr int GH = 4;
  const int total = nx * ny;
  const int l = total % 8 == 0 ? (b % 8) * (total / 8) + b / 8 : b;
  const int y0 = l / (GH * nx) * GH;
  const int h = ny - y0 < GH ? ny - y0 : GH;
  const int idx = l - y0 * nx;
  ty = y0 + idx % h;
  tx = idx / h;
}

__global__ __launch_bounds__(256, 1) void gemm_wgrad_bf16_dma_kernel(Bf16Args g) {
  // three distinct stage objects, so that reads of one stage need no wait for
  // the loads in flight into the others; [0, DOP) dY, [DOP, 2 DOP) X
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * DOP];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * DOP];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * DOP];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tx, ty;
  tile_of(blockIdx.x, (int)((g.K + WT - 1) / WT), (int)((g.N + WT - 1) / WT), tx, ty);
  const int64_t n0 = (int64_t)ty * WT, k0 = (int64_t)tx * WT;

  // load j of an operand fills 1 KB block (j * 4 + wave) of its stage: token
  // rows 2 (j * 4 + wave) + L / 32, position L % 32
  uint32_t voa[DLOADS], vob[DLOADS];
#pragma unroll
  for (int j = 0; j < DLOADS; ++j) {
    const int t = 2 * (j * 4 + wave) + (lane >> 5);
    const int c = tswz(t, lane & 31);
    voa[j] = n0 + 8 * c < g.N ? (uint32_t)((t * g.lddy + 8 * c) * 2) : OUT_OF_RANGE;
    vob[j] = k0 + 8 * c < g.K ? (uint32_t)((t * g.ldx + 8 * c) * 2) : OUT_OF_RANGE;
  }
  const int wn = wave >> 1, wk = wave & 1;
  int offa[4], offb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    offa[i] = tr_offset(wn * 128 + i * 32, lane);
    offb[i] = DOP + tr_offset(wk * 128 + i * 32, lane);
  }

  const int64_t nsteps = (g.T + DT - 1) / DT;
  // the loads of step `step` into stage object `dst`
  auto issue = [&](uint8_t* dst, int64_t step) {
    const __amdgpu_buffer_rsrc_t ra = step_rsrc(g.dy, g.lddy, n0, g.T, step);
    const __amdgpu_buffer_rsrc_t rb = step_rsrc(g.x, g.ldx, k0, g.T, step);
#pragma unroll
    for (int j = 0; j < DLOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + (j * 4 + wave) * 1024), 16, voa[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < DLOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(dst + DOP + (j * 4 + wave) * 1024), 16, vob[j], 0,
                                               0, 0);
  };

  v16f acc[4][4];
  // Step s on stage `cur`: the loads of step s + 2 go into `next2` (the
  // stage of step s - 1, which every wave left before the last barrier), the
  // MFMAs run on `cur`, then the wait for step s + 1's loads (at most the
  // younger step's 2 DLOADS loads are still in flight) and a barrier.
  // FIRST: the first MFMA of each accumulator tile starts from C = 0.
  auto step = [&](const uint8_t* cur, uint8_t* next2, int64_t s, auto first) {
    issue(next2, s + 2);
#pragma unroll
    for (int ks = 0; ks < DT / 16; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = tr_frag(cur + ks * 16 * DROWB + offa[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = tr_frag(cur + ks * 16 * DROWB + offb[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (decltype(first)::value && ks == 0) {
            const v16f z = {};
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], z, 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
          }
        }
    }
    // spread this step's fetches over its MFMAs (one per 3), rather than
    // letting them issue as one burst that stalls the MFMA issue
#pragma unroll
    for (int q = 0; q < 2 * DLOADS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
    wait_vm<2 * DLOADS>();
    lds_barrier();
  };

  issue(st0, 0);
  issue(st1, 1);
  wait_vm<2 * DLOADS>();
  lds_barrier();
  step(st0, st2, 0, std::true_type{});
  int64_t s = 1;
  // whole groups of 3 steps in the loop, the rest after it (a loop with
  // exits between its steps makes the compiler drain every load at its head)
  for (; s + 3 <= nsteps; s += 3) {
    step(st1, st0, s, std::false_type{});
    step(st2, st1, s + 1, std::false_type{});
    step(st0, st2, s + 2, std::false_type{});
  }
  if (s < nsteps) step(st1, st0, s++, std::false_type{});
  if (s < nsteps) step(st2, st1, s++, std::false_type{});
  wait_vm<0>();  // the loads past the last step (empty resources) have landed

  // accumulator tile (i, j): lane l holds column k = l % 32 and rows
  // n = 8 (v / 4) + 4 (l / 32) + v % 4 of its 32 x 32 block.  A wave's store
  // of one v covers 32 consecutive columns of two rows.  Interior tiles take
  // a branch-free path, so that the 16 reads of an fp32 C being accumulated
  // are in flight together instead of one read-add-write at a time.
  if (n0 + WT <= g.N && k0 + WT <= g.K) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k = k0 + wk * 128 + j * 32 + (lane & 31);
        const int64_t nb = n0 + wn * 128 + i * 32 + 4 * (lane >> 5);
        float val[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(val[v]) : "a"(acc[i][j][v]));
        if (g.out_bf16) {
          uint16_t* cp = reinterpret_cast<uint16_t*>(g.c) + nb * g.ldc + k;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            cp[(8 * (v / 4) + v % 4) * g.ldc] = (uint16_t)(pack_bf16x2(val[v], 0.0f) & 0xFFFF);
        } else {
          float* cp = reinterpret_cast<float*>(g.c) + nb * g.ldc + k;
          if (g.accumulate) {
            float old[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) old[v] = cp[(8 * (v / 4) + v % 4) * g.ldc];
#pragma unroll
            for (int v = 0; v < 16; ++v) val[v] += old[v];
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) cp[(8 * (v / 4) + v % 4) * g.ldc] = val[v];
        }
      }
    return;
  }
  // accumulator tile (i, j): lane l holds column k = l % 32 and rows
  // n = 8 (v / 4) + 4 (l / 32) + v % 4 of its 32 x 32 block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = k0 + wk * 128 + j * 32 + (lane & 31);
      if (k >= g.K) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t n = n0 + wn * 128 + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
        if (n >= g.N) continue;
        float val;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(val) : "a"(acc[i][j][v]));
        if (g.out_bf16) {
          reinterpret_cast<uint16_t*>(g.c)[n * g.ldc + k] = (uint16_t)(pack_bf16x2(val, 0.0f) & 0xFFFF);
        } else {
          float* cp = reinterpret_cast<float*>(g.c) + n * g.ldc + k;
          *cp = g.accumulate ? *cp + val : val;
        }
      }
    }
}

}  // namespace

void launch_wgrad_bf16(const void* dy, int64_t T, int64_t N, int64_t lddy, const void* x, int64_t K, int64_t ldx,
                       void* c, int c_dtype, int64_t ldc, bool accumulate, hipStream_t st) {
  Bf16Args g{};
  g.dy = reinterpret_cast<const uint16_t*>(dy);
  g.x = reinterpret_cast<const uint16_t*>(x);
  g.T = T; g.N = N; g.K = K; g.lddy = lddy; g.ldx = ldx; g.ldc = ldc; g.c = c;
  g.vec = ((uintptr_t)dy % 16 == 0) && ((uintptr_t)x % 16 == 0) && (lddy % 8 == 0) && (ldx % 8 == 0);
  g.out_bf16 = (c_dtype == 1);
  g.accumulate = accumulate && c_dtype == 0;
  const dim3 grid((unsigned)((K + WT - 1) / WT), (unsigned)((N + WT - 1) / WT));
  // direct-to-LDS path: aligned rows, whole 16-byte chunks at the feature
  // edges, a step's rows (48 x ld x 2 bytes) within a 31-bit resource, and the
  // tiles within a 1-D grid
  const bool dma = g.vec && N % 8 == 0 && K % 8 == 0 && lddy < (1 << 24) && ldx < (1 << 24) && T > 0 &&
                   (uint64_t)grid.x * grid.y <= 0x7FFFFFFFu;
  if (dma)
    hipLaunchKernelGGL(gemm_wgrad_bf16_dma_kernel, dim3(grid.x * grid.y), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(gemm_wgrad_bf16_kernel, grid, dim3(256), 0, st, g);
}

}  // namespace qsg
