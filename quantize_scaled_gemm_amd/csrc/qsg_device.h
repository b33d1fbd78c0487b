// Device helpers shared by the gfx950 kernels: FP8 encoding, bit tricks,
// wavefront reductions.
//
// FP8 formats: OCP 8-bit floating point (E4M3 max 448, E5M2 max 57344), as
// named by the "--fp8-format {e4m3,hybrid}" flag of the "Low-Precision
// Training Guide".  Encoding is saturating round-to-nearest-even: finite
// overflow and infinities clamp to the signed maximum, NaN gives sign|0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte streaming store (written once, not read again by this kernel).
__device__ __forceinline__ void st_stream8(void* p, uint32_t lo, uint32_t hi) {
  const u32x2 v = {lo, hi};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<kE4M3> {
  static constexpr float kMax = 448.0f;
  static constexpr int kEmaxElem = 8;  // 448 = 1.75 * 2^8
};
template <>
struct Fp8Traits<kE5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr int kEmaxElem = 15;  // 57344 = 1.75 * 2^15
};

__host__ __device__ inline float fp8_max(int fmt) { return fmt == kE4M3 ? 448.0f : 57344.0f; }

// Convert two binary32 values to FP8 and place the two codes in the low
// (HI=false) or high (HI=true) 16 bits of `old`.  The hardware conversion
// rounds to nearest even; the med3 clamp makes it saturating for finite
// values and infinities.  NaN inputs are patched to sign|0x7F afterwards so
// the result does not depend on how the clamp and the conversion treat NaN.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
  constexpr float m = Fp8Traits<FMT>::kMax;
  float ca = __builtin_amdgcn_fmed3f(a, -m, m);
  float cb = __builtin_amdgcn_fmed3f(b, -m, m);
  uint32_t r;
  if constexpr (FMT == kE4M3)
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, (int)old, HI);
  else
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, (int)old, HI);
  if (__builtin_expect(__builtin_isnan(a) | __builtin_isnan(b), 0)) {
    const int sh = HI ? 16 : 0;
    if (__builtin_isnan(a)) {
      uint32_t code = ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
      r = (r & ~(0xFFu << sh)) | (code << sh);
    }
    if (__builtin_isnan(b)) {
      uint32_t code = ((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu;
      r = (r & ~(0xFF00u << sh)) | (code << (sh + 8));
    }
  }
  return r;
}

// Four binary32 values -> four FP8 codes packed little-endian in a dword.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
  uint32_t lo = cvt_pk<FMT, false>(a, b, 0u);
  return cvt_pk<FMT, true>(c, d, lo);
}

// Four binary32 values known to be finite with |v| <= max (no clamp, no NaN
// patch needed): the hardware RNE conversion alone gives enc().
template <int FMT>
__device__ __forceinline__ uint32_t enc4_inrange(float a, float b, float c, float d) {
  uint32_t r;
  if constexpr (FMT == kE4M3) {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
  } else {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, (int)r, true);
  }
  return r;
}

// bf16 <-> fp32 (exact widening; RNE narrowing of finite values, NaN kept quiet).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two binary32 values rounded to bfloat16 (round to nearest even) and packed,
// `lo` in the low half: a single v_cvt_pk_bf16_f32 on gfx950.
typedef float qsg_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 qsg_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const qsg_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, qsg_bf16x2));
}

// |x| of a binary32 bit pattern; NaNs become the canonical 0x7FC00000 so
// that an integer max over |x| patterns is order-free and reports NaN as
// 0x7FC00000 (NaN > +inf > finite as unsigned integers).
__device__ __forceinline__ uint32_t abs_bits_canon(uint32_t u) {
  u &= 0x7FFFFFFFu;
  return u > 0x7F800000u ? 0x7FC00000u : u;
}

// Wavefront (64 lanes) unsigned max via DPP/permute-free shuffles.
// Cross-lane moves without the LDS: DPP within a row of 16 lanes (quad
// permutes, row rotates) and gfx950's v_permlane16/32_swap across rows.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

__device__ __forceinline__ uint32_t umax_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max(v, v of lane l ^ 16): a swap of rows 1 and 0 (and 3 and 2) between two
// copies of v leaves each lane holding its own value and its partner's
__device__ __forceinline__ uint32_t max_xor16(uint32_t v) {
  const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return umax_u32(s[0], s[1]);
}
// max(v, v of lane l ^ 32), likewise with the two halves of the wave
__device__ __forceinline__ uint32_t max_xor32(uint32_t v) {
  const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax_u32(s[0], s[1]);
}

// Max over lanes that differ only in the bits of MASK (xor pattern).  Bits 2
// and 3 go together: max over lanes i + 0, 4, 8, 12 of a row by two rotates
// is the max over i ^ {0, 4, 8, 12}.
template <int MASK>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(((MASK >> 2) & 3) == 0 || ((MASK >> 2) & 3) == 3, "lane bits 2 and 3 are reduced together");
  if constexpr (MASK & 1) v = umax_u32(v, dpp_u32<kDppXor1>(v));
  if constexpr (MASK & 2) v = umax_u32(v, dpp_u32<kDppXor2>(v));
  if constexpr (MASK & 4) {
    v = umax_u32(v, dpp_u32<kDppRor4>(v));
    v = umax_u32(v, dpp_u32<kDppRor8>(v));
  }
  if constexpr (MASK & 16) v = max_xor16(v);
  if constexpr (MASK & 32) v = max_xor32(v);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return group_max_u32<0x3F>(v); }

// Fold a workgroup's per-thread maxima (unsigned |x| bit patterns) into the
// device-wide maximum at *out.  The workgroup reduces through LDS first and
// only issues the device-scope atomic when its maximum exceeds the value it
// reads at *out: thousands of workgroups would otherwise serialise on one
// address.  A stale (smaller) read only costs an extra atomic, never a wrong
// result.  Every thread of the workgroup must call this.
template <int NTHREADS>
__device__ __forceinline__ void block_max_to_global(uint32_t m, uint32_t* out, uint32_t* lds_scratch) {
  m = wave_max_u32(m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds_scratch[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < NTHREADS / 64; ++i) m = m > lds_scratch[i] ? m : lds_scratch[i];
    if (m > 0x7F800000u) m = 0x7FC00000u;
    const uint32_t cur = __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m > cur) atomicMax(out, m);
  }
}

// Per-tensor scale (recipe "tensorwise" and the --fp8-margin knob of the
// "Low-Precision Training Guide"): scale = fp32(fmax / amax) * 2^-margin,
// with amax == 0 or non-finite giving 1 and an overflowing quotient giving
// FLT_MAX.  The division is the IEEE correctly rounded one.
__device__ __forceinline__ float scale_from_amax(float amax, float fmax, int margin) {
  uint32_t ab = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (ab == 0u || ab >= 0x7F800000u) return 1.0f;
  float s = __fdiv_rn(fmax, amax);
  if (__float_as_uint(s) == 0x7F800000u) s = __uint_as_float(0x7F7FFFFFu);
  return s * __builtin_ldexpf(1.0f, -margin);
}

// 2^-e as binary32 for e in [-127, 127] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_neg(int e) {
  return e == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - e) << 23);
}

// MXFP8 shared exponent of a block from its amax bit pattern (non-negative,
// NaN canonicalised): amax = 2^E (1 + f).  CEIL: E - emax + [f > 0.75];
// OCP floor: E - emax.  Then + margin, clamp to [-127, 127]; amax 0 -> 0.
__device__ __forceinline__ int mx_exponent(uint32_t abits, int emax_elem, bool ceil_rule, int margin) {
  if (abits == 0u) return 0;
  uint32_t ef = abits >> 23;
  uint32_t man = abits & 0x7FFFFFu;
  int E;
  uint32_t fbits;
  if (ef == 0u) {
    int p = 31 - __clz(man);  // leading one of the subnormal significand
    E = p - 149;
    fbits = (man << (23 - p)) & 0x7FFFFFu;
  } else {
    E = (int)ef - 127;
    fbits = man;
  }
  int e = E - emax_elem + ((ceil_rule && fbits > 0x600000u) ? 1 : 0) + margin;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e;
}

}  // namespace qsg
