// Quantization kernels for gfx950: amax, scale, amax-history update, and one
// tiled kernel family for cast + transpose under the per-tensor, MXFP8 and
// blockwise recipes of the "Low-Precision Training Guide" (section "Recipe
// Reference").
//
// Tile kernel layout.  A workgroup of 256 threads (4 wave64s) owns a 128 x 128
// tile of the input.  Thread t has tx = t & 15 and ty = t >> 4 and holds the
// 8 x 8 sub-block at rows ty*8.., cols tx*8..; wave w holds rows 32w..32w+31.
//   * Global loads are 16-byte (8 bf16 or 4 fp32) row segments: 16 lanes
//     cover a 256-byte row of bf16, fully coalesced.
//   * The row-wise copy Q is encoded with the 8 values of a row grouped, and
//     stored straight from registers with non-temporal stores (8 bytes per
//     lane, 128 contiguous bytes per row segment).
//   * The column-wise copy is encoded with the 8 values of a column grouped,
//     which is already its transposed byte order (where both copies share
//     one scale -- per-tensor and 128x128 -- the row codes are byte-transposed
//     in registers with v_perm_b32 instead of being encoded again); each lane
//     writes two 8-byte pieces per column into an LDS tile [col][row] (stride
//     136 bytes, 8-byte slots swizzled by slot ^ tx so the writes of a
//     half-wave hit distinct banks), and the tile is read back as 16-byte chunks of 16 consecutive
//     rows of one column and stored to QT: 8 lanes cover a 128-byte run.
//   * Block maxima: 1x32 row blocks are 4 lanes (xor 1, 2); 32x1 column
//     blocks are the 4 row-groups of one wave (xor 16, 32); 1x128 row blocks
//     are 16 lanes; 128x1 column blocks and 128x128 blocks reduce across the
//     4 waves through LDS.
// The kernel walks the tiles in row-major order with a grid stride: a
// persistent grid of 2 workgroups per CU where the per-tensor path fuses the
// amax (one atomic per workgroup), otherwise one tile per workgroup (see
// launch_tile).
#include <hip/hip_runtime.h>

#include <mutex>

#include "qsg.h"
#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

constexpr int TILE = 128;
constexpr int QT_STRIDE = 136;  // bytes per column of the LDS transpose tile

// ---------------------------------------------------------------------------
// small kernels
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void compute_scale_kernel(const float* amax, float fmax, int margin, float* scale,
                                     float* scale_inv) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    float s = scale_from_amax(*amax, fmax, margin);
    *scale = s;
    *scale_inv = __fdiv_rn(1.0f, s);
  }
}

// One workgroup of 256 threads: history[slot] = amax (bits a); window max;
// next scale unless the max is 0 or not finite ("Low-Precision Training
// Guide", recipe "delayed", --fp8-amax-history-len / --fp8-amax-compute-algo
// max).  red: 4 words of LDS.
__device__ __forceinline__ void history_update_wg(float* history, int64_t L, int64_t slot, uint32_t a, float fmax,
                                                  int margin, float* scale, float* scale_inv, uint32_t* red) {
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < L; i += 256) {
    uint32_t v = (i == slot) ? a : __float_as_uint(history[i]);
    // amax values are >= 0; any NaN is reported as the canonical NaN and any
    // value with the sign bit set ranks above +inf, so both keep the scale
    v = (v > 0x7F800000u) ? 0x7FC00000u : v;
    m = m > v ? m : v;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = red[0];
    for (int i = 1; i < 4; ++i) w = w > red[i] ? w : red[i];
    history[slot] = __uint_as_float(a);
    if (w != 0u && w < 0x7F800000u) {
      float s = scale_from_amax(__uint_as_float(w), fmax, margin);
      *scale = s;
      *scale_inv = __fdiv_rn(1.0f, s);
    }
  }
}

__global__ __launch_bounds__(256) void amax_update_kernel(float* history, int64_t L, int64_t slot,
                                                          const float* amax, float fmax,
                                                          int margin, float* scale,
                                                          float* scale_inv) {
  __shared__ uint32_t red[4];
  history_update_wg(history, L, slot, __float_as_uint(*amax), fmax, margin, scale, scale_inv, red);
}

// ---------------------------------------------------------------------------
// amax reduction (per tensor)
// ---------------------------------------------------------------------------
template <typename In>
__global__ __launch_bounds__(256) void amax_kernel(const In* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld, bool vec_ok,
                                                   uint32_t* __restrict__ out) {
  constexpr int VEC = 16 / sizeof(In);
  uint32_t m = 0;
  const int64_t nvec = vec_ok ? cols / VEC : 0;
  const int64_t tail0 = nvec * VEC;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const In* row = x + r * ld;
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < nvec; i += 8 * stride) {
      u32x4 u[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) u[k] = ld_stream16(rv + i + k * stride);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (sizeof(In) == 2) {
            uint32_t lo = (w[q] << 16) & 0x7FFFFFFFu, hi = w[q] & 0x7FFF0000u;
            m = m > lo ? m : lo;
            m = m > hi ? m : hi;
          } else {
            uint32_t v = w[q] & 0x7FFFFFFFu;
            m = m > v ? m : v;
          }
        }
      }
    }
    for (; i < nvec; i += stride) {
      u32x4 u = ld_stream16(rv + i);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (sizeof(In) == 2) {
          uint32_t lo = (w[q] << 16) & 0x7FFFFFFFu, hi = w[q] & 0x7FFF0000u;
          m = m > lo ? m : lo;
          m = m > hi ? m : hi;
        } else {
          uint32_t v = w[q] & 0x7FFFFFFFu;
          m = m > v ? m : v;
        }
      }
    }
    // scalar tail (or the whole row when vector loads are not allowed)
    for (int64_t c = tail0 + (int64_t)blockIdx.x * 256 + threadIdx.x; c < cols; c += stride) {
      uint32_t v;
      if constexpr (sizeof(In) == 2)
        v = ((uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << 16) & 0x7FFFFFFFu;
      else
        v = reinterpret_cast<const uint32_t*>(row)[c] & 0x7FFFFFFFu;
      m = m > v ? m : v;
    }
  }
  __shared__ uint32_t red[4];
  block_max_to_global<256>(m, out, red);
}

// ---------------------------------------------------------------------------
// tile kernel
// ---------------------------------------------------------------------------
enum Mode { MODE_TENSOR = 0, MODE_MX = 1, MODE_B1X128 = 2, MODE_B128X128 = 3 };

struct TileArgs {
  const void* x;
  int64_t rows, cols, ld;
  bool vec_ok;           // 16-byte loads/stores allowed on full tiles
  const float* scale;    // MODE_TENSOR: device scale
  uint8_t* q;            // rows x cols or null
  uint8_t* qt;           // cols x rows or null
  void* s;               // row-wise scales (MX: u8, block: f32)
  void* st;              // column-wise scales
  uint32_t* amax_out;    // MODE_TENSOR fused amax (as uint bits) or null
  // MODE_TENSOR, one launch of a delayed-scaling step: ws[0] collects the
  // amax bits, ws[1] counts finished workgroups; the last one records the
  // amax in hist[slot], sets the next scale and clears ws again
  uint32_t* ws;
  float* hist;
  int64_t hist_len, slot;
  float* scale_w;        // the scale in force, replaced by the next one
  float* scale_inv_w;
  int margin;
  bool mx_ceil;
  // MXFP8: a full tile's E8M0 bytes leave as one 4-byte store per row (s) and
  // per column (st) when those runs are 4-byte aligned
  bool s_vec, st_vec;
  int64_t tiles_c, ntiles;
};

// Thread-private 8x8 sub-block in its input type.
template <typename In>
struct Block8;

template <>
struct Block8<uint16_t> {  // bf16 bit patterns
  uint32_t w[8][4];
  __device__ __forceinline__ float at(int j, int i) const {
    uint32_t v = w[j][i >> 1];
    return (i & 1) ? bf16hi(v) : bf16lo(v);
  }
  __device__ __forceinline__ uint32_t absbits(int j, int i) const {
    uint32_t v = w[j][i >> 1];
    return ((i & 1) ? (v & 0xFFFF0000u) : (v << 16)) & 0x7FFFFFFFu;
  }
  template <bool FULL>
  __device__ __forceinline__ void load(const TileArgs& a, int64_t r, int64_t c) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (FULL) {
        u32x4 u = ld_stream16(x + (r + j) * a.ld + c);
        w[j][0] = u.x; w[j][1] = u.y; w[j][2] = u.z; w[j][3] = u.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo = 0, hi = 0;
          if (r + j < a.rows) {
            if (c + 2 * k < a.cols) lo = x[(r + j) * a.ld + c + 2 * k];
            if (c + 2 * k + 1 < a.cols) hi = x[(r + j) * a.ld + c + 2 * k + 1];
          }
          w[j][k] = lo | (hi << 16);
        }
      }
    }
  }
};

template <>
struct Block8<float> {
  float v[8][8];
  __device__ __forceinline__ float at(int j, int i) const { return v[j][i]; }
  __device__ __forceinline__ uint32_t absbits(int j, int i) const {
    return __float_as_uint(v[j][i]) & 0x7FFFFFFFu;
  }
  template <bool FULL>
  __device__ __forceinline__ void load(const TileArgs& a, int64_t r, int64_t c) {
    const float* x = reinterpret_cast<const float*>(a.x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (FULL) {
        const float* p = x + (r + j) * a.ld + c;
        u32x4 u0 = ld_stream16(p);
        u32x4 u1 = ld_stream16(p + 4);
        v[j][0] = __uint_as_float(u0.x); v[j][1] = __uint_as_float(u0.y);
        v[j][2] = __uint_as_float(u0.z); v[j][3] = __uint_as_float(u0.w);
        v[j][4] = __uint_as_float(u1.x); v[j][5] = __uint_as_float(u1.y);
        v[j][6] = __uint_as_float(u1.z); v[j][7] = __uint_as_float(u1.w);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[j][i] = (r + j < a.rows && c + i < a.cols) ? x[(r + j) * a.ld + c + i] : 0.0f;
      }
    }
  }
};

// 4 x 4 byte transpose: a..d are four rows of four bytes (byte k = column
// k); o0..o3 are the four columns (byte k = row k).  Eight v_perm_b32: four
// interleave the rows in pairs, four gather the columns.
__device__ __forceinline__ void transpose4x4_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                   uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  // v_perm_b32(hi, lo, sel): selector byte values 0-3 pick bytes of lo, 4-7 of hi
  const uint32_t ab01 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab23 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd01 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t cd23 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o0 = __builtin_amdgcn_perm(cd01, ab01, 0x05040100u);             // a0 b0 c0 d0
  o1 = __builtin_amdgcn_perm(cd01, ab01, 0x07060302u);             // a1 b1 c1 d1
  o2 = __builtin_amdgcn_perm(cd23, ab23, 0x05040100u);             // a2 b2 c2 d2
  o3 = __builtin_amdgcn_perm(cd23, ab23, 0x07060302u);             // a3 b3 c3 d3
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t canon(uint32_t m) { return m > 0x7F800000u ? 0x7FC00000u : m; }

// End of a one-launch delayed-scaling step (TileArgs::ws set).  Workgroups
// are split into DELAYED_GROUPS groups (id mod DELAYED_GROUPS), each with its
// own 128-byte line of the workspace holding the group's amax and arrival
// count, so no address sees more than a few dozen atomics.  A workgroup
// performs its group's atomic max and waits for it to return before it
// arrives; the last arrival of a group arrives at the common counter; the
// last one there has every workgroup's maximum in the group lines, records
// the amax in the history, sets the next scale and clears the workspace.
// Device-scope atomics are performed in issue order at the coherence point,
// so no cache write-back is needed; the history, scale and FP8 outputs are
// read by later launches only (the scale in force was read by every
// workgroup before its first tile).
constexpr int DELAYED_GROUPS = 32;
constexpr int WS_LINE = 32;  // words per workspace line

__device__ __forceinline__ void delayed_finish(const TileArgs& a, uint32_t m, float fmax, uint32_t* red) {
  m = wave_max_u32(m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 4; ++i) m = m > red[i] ? m : red[i];
    m = canon(m);
    const uint32_t G = gridDim.x, grp = blockIdx.x % DELAYED_GROUPS;
    const uint32_t ngrp = G < DELAYED_GROUPS ? G : DELAYED_GROUPS;
    const uint32_t in_grp = G / DELAYED_GROUPS + (grp < G % DELAYED_GROUPS ? 1u : 0u);
    uint32_t* line = a.ws + grp * WS_LINE;
    uint32_t old = __hip_atomic_fetch_max(line, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(old) : : "memory");  // the max is performed before arriving
    uint32_t last = 0;
    if (__hip_atomic_fetch_add(line + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_grp - 1) {
      const uint32_t n = __hip_atomic_fetch_add(a.ws + DELAYED_GROUPS * WS_LINE, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      last = (n == ngrp - 1) ? 1u : 0u;
    }
    red[4] = last;
  }
  __syncthreads();
  if (red[4]) {
    // the last workgroup: one lane per group reads and clears its line
    const uint32_t G = gridDim.x;
    const uint32_t ngrp = G < DELAYED_GROUPS ? G : DELAYED_GROUPS;
    uint32_t v = 0;
    if (threadIdx.x < ngrp) {
      uint32_t* line = a.ws + threadIdx.x * WS_LINE;
      v = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(line, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(line + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    v = wave_max_u32(v);  // the group lanes are all in wave 0
    if (threadIdx.x == 0) {
      __hip_atomic_store(a.ws + DELAYED_GROUPS * WS_LINE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.amax_out) *a.amax_out = v;
      red[5] = v;
    }
    __syncthreads();
    history_update_wg(a.hist, a.hist_len, a.slot, red[5], fmax, a.margin, a.scale_w, a.scale_inv_w, red + 8);
  }
}

template <typename In, int MODE, int FMT>
__global__ __launch_bounds__(256) void tile_kernel(TileArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_qt[TILE * QT_STRIDE];
  __shared__ uint32_t lds_red[4][TILE];
  __shared__ float lds_cscale[TILE];

  constexpr float FMAX = Fp8Traits<FMT>::kMax;
  constexpr int EMAX = Fp8Traits<FMT>::kEmaxElem;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4, wave = tid >> 6;
  uint32_t amax_acc = 0;

  float tscale = 1.0f;
  if constexpr (MODE == MODE_TENSOR) tscale = *a.scale;

  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / a.tiles_c) * TILE;
    const int64_t c0 = (tile % a.tiles_c) * TILE;
    const int64_t r = r0 + ty * 8, c = c0 + tx * 8;
    const bool full = a.vec_ok && (r0 + TILE <= a.rows) && (c0 + TILE <= a.cols);

    Block8<In> b;
    if (full)
      b.template load<true>(a, r, c);
    else
      b.template load<false>(a, r, c);

    // ---- scales -----------------------------------------------------------
    float rs[8];  // row-wise multiplier for each of this thread's rows
    float cs[8];  // column-wise multiplier for each of this thread's columns
    // MXFP8 with the CEIL exponent rule on blocks with no infinity or NaN:
    // every scaled value is exactly <= max (a power-of-two scale), so the
    // encode needs no clamp and no NaN patch
    bool inrange = false;
    if constexpr (MODE == MODE_TENSOR) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = umax(m, b.absbits(j, i));
      amax_acc = umax(amax_acc, m);
#pragma unroll
      for (int k = 0; k < 8; ++k) rs[k] = cs[k] = tscale;
    } else if constexpr (MODE == MODE_MX || MODE == MODE_B1X128) {
      // row blocks: 32 columns = 4 lanes (MX) or 128 columns = 16 lanes
      uint32_t rowmax[8], colmax[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = umax(m, b.absbits(j, i));
        rowmax[j] = canon(MODE == MODE_MX ? group_max_u32<0x3>(m) : group_max_u32<0xF>(m));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = umax(m, b.absbits(j, i));
        colmax[i] = group_max_u32<0x30>(m);  // the 4 row groups of this wave
      }
      if constexpr (MODE == MODE_MX) {
        uint32_t mm = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) mm = umax(mm, umax(rowmax[k], colmax[k]));
        inrange = a.mx_ceil && mm < 0x7F800000u;
        // E8M0 bytes of a full tile: through LDS (lds_red is free in this
        // mode), row-block bytes [row][4], column-block bytes [col][4]
        const bool tile_in = (r0 + TILE <= a.rows) && (c0 + TILE <= a.cols);
        uint8_t* sbytes = reinterpret_cast<uint8_t*>(&lds_red[0][0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          int e = mx_exponent(rowmax[j], EMAX, a.mx_ceil, a.margin);
          rs[j] = pow2_neg(e);
          if (a.s && (tx & 3) == 0) {
            if (tile_in && a.s_vec)
              sbytes[(ty * 8 + j) * 4 + (tx >> 2)] = (uint8_t)(e + 127);
            else if (r + j < a.rows && c < a.cols)
              reinterpret_cast<uint8_t*>(a.s)[(r + j) * (a.cols / 32) + (c >> 5)] = (uint8_t)(e + 127);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int e = mx_exponent(canon(colmax[i]), EMAX, a.mx_ceil, a.margin);
          cs[i] = pow2_neg(e);
          if (a.st && (ty & 3) == 0) {
            if (tile_in && a.st_vec)
              sbytes[512 + (tx * 8 + i) * 4 + (ty >> 2)] = (uint8_t)(e + 127);
            else if (c + i < a.cols && r < a.rows)
              reinterpret_cast<uint8_t*>(a.st)[(c + i) * (a.rows / 32) + (r >> 5)] = (uint8_t)(e + 127);
          }
        }
        if (tile_in && ((a.s && a.s_vec) || (a.st && a.st_vec))) {
          __syncthreads();
          const uint32_t* w = reinterpret_cast<const uint32_t*>(sbytes);
          if (tid < TILE) {
            if (a.s && a.s_vec)
              *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.s) + (r0 + tid) * (a.cols / 32) + c0 / 32) =
                  w[tid];
          } else if (a.st && a.st_vec) {
            const int col = tid - TILE;
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.st) + (c0 + col) * (a.rows / 32) + r0 / 32) =
                w[TILE + col];
          }
        }
      } else {
        // 1x128: row scale per row of the tile; 128x1: column scale needs all 4 waves
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float s = scale_from_amax(__uint_as_float(rowmax[j]), FMAX, a.margin);
          rs[j] = s;
          if (a.s && tx == 0 && r + j < a.rows)
            reinterpret_cast<float*>(a.s)[(r + j) * (a.cols / TILE) + (c0 / TILE)] = __fdiv_rn(1.0f, s);
        }
        if ((tid & 0x30) == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) lds_red[wave][tx * 8 + i] = colmax[i];
        }
        __syncthreads();
        if (tid < TILE) {
          uint32_t m = umax(umax(lds_red[0][tid], lds_red[1][tid]), umax(lds_red[2][tid], lds_red[3][tid]));
          float s = scale_from_amax(__uint_as_float(canon(m)), FMAX, a.margin);
          lds_cscale[tid] = s;
          if (a.st && c0 + tid < a.cols && r0 < a.rows)
            reinterpret_cast<float*>(a.st)[(c0 + tid) * (a.rows / TILE) + (r0 / TILE)] = __fdiv_rn(1.0f, s);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) cs[i] = lds_cscale[tx * 8 + i];
      }
    } else {  // MODE_B128X128: one scale for the whole tile
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = umax(m, b.absbits(j, i));
      m = wave_max_u32(m);
      if ((tid & 63) == 0) lds_red[0][wave] = m;
      __syncthreads();
      m = umax(umax(lds_red[0][0], lds_red[0][1]), umax(lds_red[0][2], lds_red[0][3]));
      float s = scale_from_amax(__uint_as_float(canon(m)), FMAX, a.margin);
      if (tid == 0) {
        float si = __fdiv_rn(1.0f, s);
        const int64_t tr = r0 / TILE, tc = c0 / TILE;
        if (a.s) reinterpret_cast<float*>(a.s)[tr * (a.cols / TILE) + tc] = si;
        if (a.st) reinterpret_cast<float*>(a.st)[tc * (a.rows / TILE) + tr] = si;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) rs[k] = cs[k] = s;
    }

    // ---- row-wise copy ------------------------------------------------------
    // Where the row and column copies share one scale (per-tensor, 128x128),
    // the column codes are the row codes transposed, so they are computed
    // once and transposed as bytes in registers.
    constexpr bool SAME_SCALE = (MODE == MODE_TENSOR || MODE == MODE_B128X128);
    uint32_t rq[8][2];
    if (SAME_SCALE || a.q) {
      if (MODE == MODE_MX && inrange) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float s = rs[j];
          rq[j][0] = enc4_inrange<FMT>(b.at(j, 0) * s, b.at(j, 1) * s, b.at(j, 2) * s, b.at(j, 3) * s);
          rq[j][1] = enc4_inrange<FMT>(b.at(j, 4) * s, b.at(j, 5) * s, b.at(j, 6) * s, b.at(j, 7) * s);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float s = rs[j];
          rq[j][0] = enc4<FMT>(b.at(j, 0) * s, b.at(j, 1) * s, b.at(j, 2) * s, b.at(j, 3) * s);
          rq[j][1] = enc4<FMT>(b.at(j, 4) * s, b.at(j, 5) * s, b.at(j, 6) * s, b.at(j, 7) * s);
        }
      }
    }
    if (a.q) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (full) {
          st_stream8(a.q + (r + j) * a.cols + c, rq[j][0], rq[j][1]);
        } else if (r + j < a.rows) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (c + i < a.cols) a.q[(r + j) * a.cols + c + i] = (uint8_t)((rq[j][i >> 2] >> (8 * (i & 3))) & 0xFF);
        }
      }
    }

    // ---- column-wise copy through the LDS transpose tile --------------------
    if (a.qt) {
      uint32_t cq[8][2];  // column i: rows 0-3 in cq[i][0], rows 4-7 in cq[i][1]
      if constexpr (SAME_SCALE) {
        transpose4x4_bytes(rq[0][0], rq[1][0], rq[2][0], rq[3][0], cq[0][0], cq[1][0], cq[2][0], cq[3][0]);
        transpose4x4_bytes(rq[4][0], rq[5][0], rq[6][0], rq[7][0], cq[0][1], cq[1][1], cq[2][1], cq[3][1]);
        transpose4x4_bytes(rq[0][1], rq[1][1], rq[2][1], rq[3][1], cq[4][0], cq[5][0], cq[6][0], cq[7][0]);
        transpose4x4_bytes(rq[4][1], rq[5][1], rq[6][1], rq[7][1], cq[4][1], cq[5][1], cq[6][1], cq[7][1]);
      } else if (MODE == MODE_MX && inrange) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float s = cs[i];
          cq[i][0] = enc4_inrange<FMT>(b.at(0, i) * s, b.at(1, i) * s, b.at(2, i) * s, b.at(3, i) * s);
          cq[i][1] = enc4_inrange<FMT>(b.at(4, i) * s, b.at(5, i) * s, b.at(6, i) * s, b.at(7, i) * s);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float s = cs[i];
          cq[i][0] = enc4<FMT>(b.at(0, i) * s, b.at(1, i) * s, b.at(2, i) * s, b.at(3, i) * s);
          cq[i][1] = enc4<FMT>(b.at(4, i) * s, b.at(5, i) * s, b.at(6, i) * s, b.at(7, i) * s);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = tx * 8 + i;
        const int slot = ty ^ tx;
        *reinterpret_cast<uint2*>(lds_qt + col * QT_STRIDE + slot * 8) = make_uint2(cq[i][0], cq[i][1]);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int id = k * 256 + tid;
        const int col = id >> 3, r16 = id & 7;
        const int x = col >> 3;
        uint2 lo = *reinterpret_cast<const uint2*>(lds_qt + col * QT_STRIDE + ((2 * r16) ^ x) * 8);
        uint2 hi = *reinterpret_cast<const uint2*>(lds_qt + col * QT_STRIDE + ((2 * r16 + 1) ^ x) * 8);
        const int64_t gc = c0 + col, gr = r0 + r16 * 16;
        if (full) {
          *reinterpret_cast<uint4*>(a.qt + gc * a.rows + gr) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else if (gc < a.cols) {
          uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int bb = 0; bb < 16; ++bb)
            if (gr + bb < a.rows) a.qt[gc * a.rows + gr + bb] = (uint8_t)((w[bb >> 2] >> (8 * (bb & 3))) & 0xFF);
        }
      }
    }
    __syncthreads();  // the LDS tiles are reused by the next tile
  }

  if constexpr (MODE == MODE_TENSOR) {
    if (a.ws) {
      delayed_finish(a, amax_acc, FMAX, &lds_red[0][0]);
    } else if (a.amax_out) {
      block_max_to_global<256>(amax_acc, a.amax_out, &lds_red[0][0]);
    }
  }
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      n = p.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

template <typename In, int MODE>
void launch_tile(const TileArgs& a, int fmt, hipStream_t st) {
  // With a fused amax (or the delayed step's amax and history update) the
  // per-tensor cast runs a persistent grid of 2 workgroups per CU: the amax
  // ends in one device-scope atomic per workgroup on one address, which the
  // memory side performs one at a time (with 8 per CU a 64 MB tensor spent
  // more time on them than on its bytes).  Without
  // atomics every mode runs one tile per workgroup up to 128 per CU
  // (grid-stride beyond): [measured, same-box A/Bs against a persistent grid]
  // per-tensor cast X 32768 x 4096 +4 %, dY2 32768 x 14336 +3 %, W 4096 x
  // 4096 +3 % (against 2 per CU); MXFP8 dY 16384 x 14336 +12 %, 1 x 128 X
  // 16384 x 7168 / dY 16384 x 18432 +6 / +8 %, 128 x 128 W 18432 x 7168
  // +3-4 %, MXFP8 X and W (16384 / 14336 x 4096) +0-2 % (against 8 per CU).
  int64_t grid = a.ntiles;
  const bool atomics = MODE == MODE_TENSOR && (a.amax_out || a.ws);
  const int64_t cap = (int64_t)num_cus() * (atomics ? 2 : 128);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (fmt == kE4M3)
    hipLaunchKernelGGL((tile_kernel<In, MODE, kE4M3>), dim3((unsigned)grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((tile_kernel<In, MODE, kE5M2>), dim3((unsigned)grid), dim3(256), 0, st, a);
}

template <int MODE>
void launch_tile_dtype(const TileArgs& a, int dtype, int fmt, hipStream_t st) {
  if (dtype == 1)
    launch_tile<uint16_t, MODE>(a, fmt, st);
  else
    launch_tile<float, MODE>(a, fmt, st);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------
void launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t st) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 63) / 64), dim3(64), 0, st, p, v, n);
}

void launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* amax,
                 hipStream_t st) {
  uint32_t* out = reinterpret_cast<uint32_t*>(amax);
  launch_fill_u32(out, 0u, 1, st);
  if (rows == 0 || cols == 0) return;
  const int esz = dtype == 1 ? 2 : 4;
  // a dense matrix is one long row
  if (ld == cols) {
    cols = rows * cols;
    ld = cols;
    rows = 1;
  }
  const bool vec_ok = ((uintptr_t)x % 16 == 0) && ((ld * esz) % 16 == 0);
  const int64_t vecs = vec_ok ? cols / (16 / esz) : cols;
  // One workgroup per CU, 8 loads in flight per thread: every workgroup
  // ends in one device-scope atomic on one address, which the memory side
  // performs one at a time, so fewer and longer-lived workgroups stream
  // faster (4 per CU with 4 loads each lost 17-27 % to them).
  int64_t gx = (vecs + 256 * 8 - 1) / (256 * 8);
  const int64_t cap = (int64_t)num_cus();
  int64_t gy = rows;
  if (gx > cap) gx = cap;
  if (gx < 1) gx = 1;
  if (gy > 65535) gy = 65535;
  if (gx * gy > cap) gy = (cap + gx - 1) / gx;
  if (gy < 1) gy = 1;
  if (dtype == 1)
    hipLaunchKernelGGL(amax_kernel<uint16_t>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(x), rows, cols, ld, vec_ok, out);
  else
    hipLaunchKernelGGL(amax_kernel<float>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st,
                       reinterpret_cast<const float*>(x), rows, cols, ld, vec_ok, out);
}

void launch_compute_scale(const float* amax, int fmt, int margin, float* scale, float* scale_inv,
                          hipStream_t st) {
  hipLaunchKernelGGL(compute_scale_kernel, dim3(1), dim3(64), 0, st, amax, fp8_max(fmt), margin,
                     scale, scale_inv);
}

void launch_amax_update(float* history, int64_t L, int64_t step, const float* amax, int fmt,
                        int margin, float* scale, float* scale_inv, hipStream_t st) {
  hipLaunchKernelGGL(amax_update_kernel, dim3(1), dim3(256), 0, st, history, L, step % L, amax,
                     fp8_max(fmt), margin, scale, scale_inv);
}

static bool tile_vec_ok(const void* x, int esz, int64_t rows, int64_t cols, int64_t ld,
                        const uint8_t* q, const uint8_t* qt) {
  bool ok = ((uintptr_t)x % 16 == 0) && ((ld * esz) % 16 == 0);
  if (q) ok = ok && ((uintptr_t)q % 8 == 0) && (cols % 8 == 0);
  if (qt) ok = ok && ((uintptr_t)qt % 16 == 0) && (rows % 16 == 0);
  return ok;
}

void launch_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                           int fmt, const float* scale, uint8_t* q, uint8_t* qt, float* amax_out,
                           hipStream_t st) {
  if (amax_out) launch_fill_u32(reinterpret_cast<uint32_t*>(amax_out), 0u, 1, st);
  if (rows == 0 || cols == 0) return;
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.ld = ld;
  a.vec_ok = tile_vec_ok(x, dtype == 1 ? 2 : 4, rows, cols, ld, q, qt);
  a.scale = scale; a.q = q; a.qt = qt;
  a.amax_out = reinterpret_cast<uint32_t*>(amax_out);
  a.tiles_c = (cols + TILE - 1) / TILE;
  a.ntiles = ((rows + TILE - 1) / TILE) * a.tiles_c;
  launch_tile_dtype<MODE_TENSOR>(a, dtype, fmt, st);
}

void launch_cast_transpose_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                   int margin, float* history, int64_t L, int64_t step, float* scale,
                                   float* scale_inv, uint8_t* q, uint8_t* qt, float* amax_out, uint32_t* ws,
                                   hipStream_t st) {
  if (rows == 0 || cols == 0) {
    // nothing to quantize: the amax is 0 (ws[0] is 0 between calls)
    if (amax_out) launch_fill_u32(reinterpret_cast<uint32_t*>(amax_out), 0u, 1, st);
    launch_amax_update(history, L, step, reinterpret_cast<const float*>(ws), fmt, margin, scale, scale_inv, st);
    return;
  }
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.ld = ld;
  a.vec_ok = tile_vec_ok(x, dtype == 1 ? 2 : 4, rows, cols, ld, q, qt);
  a.scale = scale; a.q = q; a.qt = qt;
  a.amax_out = reinterpret_cast<uint32_t*>(amax_out);
  a.ws = ws;
  a.hist = history; a.hist_len = L; a.slot = step % L;
  a.scale_w = scale; a.scale_inv_w = scale_inv;
  a.margin = margin;
  a.tiles_c = (cols + TILE - 1) / TILE;
  a.ntiles = ((rows + TILE - 1) / TILE) * a.tiles_c;
  launch_tile_dtype<MODE_TENSOR>(a, dtype, fmt, st);
}

// ---------------------------------------------------------------------------
// allocation-free variant of the one-launch delayed step: the workspace is a
// file-scope device array, one copy per GPU, whose address is looked up once
// per device (the host-side name of the array is not a device address)
// ---------------------------------------------------------------------------
constexpr int kScratchWords = (DELAYED_GROUPS + 1) * WS_LINE;  // 4224 bytes
static_assert(kScratchWords * 4 == QSG_DELAYED_WORKSPACE_BYTES, "workspace size of include/qsg.h");
static __device__ __attribute__((aligned(256))) uint32_t scratch[kScratchWords];

int delayed_scratch(uint32_t** out, hipStream_t st) {
  static std::mutex mu;
  static uint32_t* ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -2;
    ptr[dev] = reinterpret_cast<uint32_t*>(p);
    // zero at load; cleared once more on first use, then every call leaves it zero
    launch_fill_u32(ptr[dev], 0u, kScratchWords, st);
  }
  *out = ptr[dev];
  return 0;
}

void launch_quantize_blocked(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int scaling, int fmt, int margin, bool mx_ceil, uint8_t* q, void* s,
                             uint8_t* qt, void* st_, hipStream_t st) {
  if (rows == 0 || cols == 0) return;
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.ld = ld;
  a.vec_ok = tile_vec_ok(x, dtype == 1 ? 2 : 4, rows, cols, ld, q, qt);
  a.q = q; a.qt = qt; a.s = q ? s : nullptr; a.st = qt ? st_ : nullptr;
  a.margin = margin; a.mx_ceil = mx_ceil;
  a.s_vec = a.s && ((uintptr_t)a.s % 4 == 0) && (cols % 128 == 0);
  a.st_vec = a.st && ((uintptr_t)a.st % 4 == 0) && (rows % 128 == 0);
  a.tiles_c = (cols + TILE - 1) / TILE;
  a.ntiles = ((rows + TILE - 1) / TILE) * a.tiles_c;
  if (scaling == 2)
    launch_tile_dtype<MODE_MX>(a, dtype, fmt, st);
  else if (scaling == 3)
    launch_tile_dtype<MODE_B1X128>(a, dtype, fmt, st);
  else
    launch_tile_dtype<MODE_B128X128>(a, dtype, fmt, st);
}

}  // namespace qsg
