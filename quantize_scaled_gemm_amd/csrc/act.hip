// FP8 store of an MLP activation's input ("Benefits of Using FP8 Precision
// with MegaDLMs and Required Hardware", configuration field
// activation_func_fp8_input_store: the input of the MLP activation is kept in
// FP8 for the backward pass).  The activation is GeLU in its erf form,
//   gelu(h)  = h * Phi(h) = 0.5 h erfc(-h / sqrt 2),
//   gelu'(h) = Phi(h) + h phi(h),  phi(h) = exp(-h^2 / 2) / sqrt(2 pi),
// written with erfc so that large negative inputs keep their relative
// accuracy (1 + erf(x) cancels there).
//
//   forward:  a = bf16(gelu(h)),  q = enc(fp32(h * scale)),  optional fused amax(h)
//   backward: h' = fp32(dec(q) * scale_inv),  dh = bf16(da * gelu'(h'))
//
// Both are single HBM-bound passes: 16-byte loads of 8 bf16 values per lane,
// 16-byte stores of the bf16 results and 8-byte stores of the FP8 codes
// (forward 2 + 2 + 1 B per element, backward 2 + 1 + 2 B), grid-stride over
// the 8-value chunks of a row (x) and the rows (y), at most 8 workgroups per
// CU; a dense matrix is treated as one long row.
#include <hip/hip_runtime.h>

#include "qsg_device.h"
#include "qsg_internal.h"

namespace qsg {

namespace {

constexpr float kInvSqrt2Pi = 0.39894228040143267794f;

// Upper normal tail Q(a) = 1 - Phi(a), a >= 0, written as exp(-a^2/2) R(a)
// with R(a) = erfcx(a / sqrt 2) / 2 approximated by t P(t), t = 1 / (1 + 0.3 a),
// P of degree 7 fitted by least squares on the relative error over [0, 14]
// (fit_normal_tail.py beside this file; relative error of R below 5e-7 in
// binary32).  The product keeps its relative accuracy deep in the tail, and
// the exponential is shared with the density term of the derivative.
__device__ __forceinline__ float tail_r(float a) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3f, a, 1.0f));
  float p = 0.03591236099600792f;
  p = fmaf(p, t, -0.15817970037460327f);
  p = fmaf(p, t, 0.2080099880695343f);
  p = fmaf(p, t, -0.05518290773034096f);
  p = fmaf(p, t, 0.12934212386608124f);
  p = fmaf(p, t, 0.09968014806509018f);
  p = fmaf(p, t, 0.120790995657444f);
  p = fmaf(p, t, 0.11962689459323883f);
  return p * t;
}

// Phi(h) and exp(-h^2/2)
__device__ __forceinline__ float normal_cdf(float h, float& e) {
  const float a = fabsf(h);
  e = __expf(-0.5f * a * a);
  const float q = e * tail_r(a);
  return h >= 0.0f ? 1.0f - q : q;
}

__device__ __forceinline__ float gelu_f(float h) {
  float e;
  return h * normal_cdf(h, e);
}

__device__ __forceinline__ float gelu_grad_f(float h) {
  float e;
  const float cdf = normal_cdf(h, e);
  return fmaf(h, kInvSqrt2Pi * e, cdf);
}

// FP8 code (E4M3 or E5M2, OCP layout) -> binary32, exact.
template <int FMT>
__device__ __forceinline__ float fp8_decode(uint32_t code) {
  const uint32_t s = (code & 0x80u) << 24;
  if constexpr (FMT == kE4M3) {
    const uint32_t e = (code >> 3) & 0xF, m = code & 0x7;
    if (e == 0xF && m == 0x7) return __uint_as_float(s | 0x7FC00000u);
    if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));  // m * 2^-9
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
  } else {
    const uint32_t e = (code >> 2) & 0x1F, m = code & 0x3;
    if (e == 0x1F) return __uint_as_float(s | (m ? 0x7FC00000u : 0x7F800000u));
    if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 1.52587890625e-05f));  // m * 2^-16
    return __uint_as_float(s | ((e + 112u) << 23) | (m << 21));
  }
}

struct ActArgs {
  const uint16_t* x;  // forward: h; backward: da (bf16 bits)
  int64_t rows, cols, ld;
  bool vec_ok;        // 16-byte loads of x, 16-byte stores of y, 8-byte of q
  const float* scale; // forward: scale; backward: scale_inv
  uint8_t* q;         // rows x cols FP8 codes (forward out, backward in)
  uint16_t* y;        // rows x cols bf16 (forward a, backward dh)
  uint32_t* amax_out; // forward only, may be null
};

template <int FMT>
__global__ __launch_bounds__(256) void act_fwd_kernel(ActArgs g) {
  const float s = *g.scale;
  const int64_t cv = g.vec_ok ? g.cols / 8 : 0;  // whole 8-value chunks per row
  const int64_t per_row = cv + (g.cols - cv * 8);  // chunks, then single tail elements
  uint32_t m = 0;
  for (int64_t r = blockIdx.y; r < g.rows; r += gridDim.y)
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < per_row; k += (int64_t)gridDim.x * 256) {
    if (k < cv) {
      const int64_t c = k * 8;
      const u32x4 u = ld_stream16(g.x + r * g.ld + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      float h[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = bf16lo(w[j]);
        h[2 * j + 1] = bf16hi(w[j]);
        const uint32_t lo = (w[j] << 16) & 0x7FFFFFFFu, hi = w[j] & 0x7FFF0000u;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
      }
      const uint32_t d0 = enc4<FMT>(h[0] * s, h[1] * s, h[2] * s, h[3] * s);
      const uint32_t d1 = enc4<FMT>(h[4] * s, h[5] * s, h[6] * s, h[7] * s);
      st_stream8(g.q + r * g.cols + c, d0, d1);
      u32x4 o;
      o.x = pack_bf16x2(gelu_f(h[0]), gelu_f(h[1]));
      o.y = pack_bf16x2(gelu_f(h[2]), gelu_f(h[3]));
      o.z = pack_bf16x2(gelu_f(h[4]), gelu_f(h[5]));
      o.w = pack_bf16x2(gelu_f(h[6]), gelu_f(h[7]));
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(g.y + r * g.cols + c));
    } else {
      const int64_t c = cv * 8 + (k - cv);
      const uint32_t b = g.x[r * g.ld + c];
      const float h = __uint_as_float(b << 16);
      const uint32_t ab = (b << 16) & 0x7FFFFFFFu;
      m = m > ab ? m : ab;
      g.q[r * g.cols + c] = (uint8_t)(enc4<FMT>(h * s, 0.0f, 0.0f, 0.0f) & 0xFF);
      g.y[r * g.cols + c] = (uint16_t)(pack_bf16x2(gelu_f(h), 0.0f) & 0xFFFF);
    }
  }
  if (g.amax_out) {
    __shared__ uint32_t red[4];
    block_max_to_global<256>(m, g.amax_out, red);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void act_bwd_kernel(ActArgs g) {
  const float si = *g.scale;
  const int64_t cv = g.vec_ok ? g.cols / 8 : 0;
  const int64_t per_row = cv + (g.cols - cv * 8);
  for (int64_t r = blockIdx.y; r < g.rows; r += gridDim.y)
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < per_row; k += (int64_t)gridDim.x * 256) {
    if (k < cv) {
      const int64_t c = k * 8;
      const u32x4 u = ld_stream16(g.x + r * g.ld + c);
      const uint2 qq = *reinterpret_cast<const uint2*>(g.q + r * g.cols + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      const uint32_t qw[2] = {qq.x, qq.y};
      float d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float da = (j & 1) ? bf16hi(w[j >> 1]) : bf16lo(w[j >> 1]);
        const float h = fp8_decode<FMT>((qw[j >> 2] >> (8 * (j & 3))) & 0xFF) * si;
        d[j] = da * gelu_grad_f(h);
      }
      u32x4 o;
      o.x = pack_bf16x2(d[0], d[1]);
      o.y = pack_bf16x2(d[2], d[3]);
      o.z = pack_bf16x2(d[4], d[5]);
      o.w = pack_bf16x2(d[6], d[7]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(g.y + r * g.cols + c));
    } else {
      const int64_t c = cv * 8 + (k - cv);
      const float da = __uint_as_float((uint32_t)g.x[r * g.ld + c] << 16);
      const float h = fp8_decode<FMT>(g.q[r * g.cols + c]) * si;
      g.y[r * g.cols + c] = (uint16_t)(pack_bf16x2(da * gelu_grad_f(h), 0.0f) & 0xFFFF);
    }
  }
}

int num_cus_act() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  return 256;
}

// A dense matrix is one long row; x and y have the same dense layout then.
ActArgs act_args(const void* x, int64_t rows, int64_t cols, int64_t ld, const float* scale, uint8_t* q, void* y) {
  ActArgs g{};
  if (ld == cols) {
    cols = rows * cols;
    ld = cols;
    rows = 1;
  }
  g.x = reinterpret_cast<const uint16_t*>(x);
  g.rows = rows; g.cols = cols; g.ld = ld;
  g.scale = scale; g.q = q;
  g.y = reinterpret_cast<uint16_t*>(y);
  g.vec_ok = ((uintptr_t)x % 16 == 0) && (ld % 8 == 0) && ((uintptr_t)y % 16 == 0) && ((uintptr_t)q % 8 == 0) &&
             (cols % 8 == 0);
  return g;
}

// (chunks of a row over x, rows over y), at most per_cu workgroups per CU in all
dim3 act_grid(const ActArgs& g, int per_cu) {
  const int64_t cv = g.vec_ok ? g.cols / 8 : 0;
  const int64_t per_row = cv + (g.cols - cv * 8);
  const int64_t cap = (int64_t)num_cus_act() * per_cu;
  int64_t gx = (per_row + 255) / 256;
  if (gx > cap) gx = cap;
  if (gx < 1) gx = 1;
  int64_t gy = cap / gx;
  if (gy > g.rows) gy = g.rows;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  return dim3((unsigned)gx, (unsigned)gy);
}

}  // namespace

void launch_act_fp8_store_fwd(const void* h, int64_t rows, int64_t cols, int64_t ld, int fmt, const float* scale,
                              void* a, uint8_t* q, float* amax_out, hipStream_t st) {
  if (amax_out) launch_fill_u32(reinterpret_cast<uint32_t*>(amax_out), 0u, 1, st);
  if (rows == 0 || cols == 0) return;
  ActArgs g = act_args(h, rows, cols, ld, scale, q, a);
  g.amax_out = reinterpret_cast<uint32_t*>(amax_out);
  // with the fused amax every workgroup ends in an atomic on one address,
  // which the memory side performs one at a time: fewer workgroups then
  const dim3 grid = act_grid(g, amax_out ? 2 : 8);
  if (fmt == kE4M3)
    hipLaunchKernelGGL(act_fwd_kernel<kE4M3>, grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(act_fwd_kernel<kE5M2>, grid, dim3(256), 0, st, g);
}

void launch_act_fp8_store_bwd(const void* da, int64_t rows, int64_t cols, int64_t ld, int fmt, const uint8_t* q,
                              const float* scale_inv, void* dh, hipStream_t st) {
  if (rows == 0 || cols == 0) return;
  const ActArgs g = act_args(da, rows, cols, ld, scale_inv, const_cast<uint8_t*>(q), dh);
  const dim3 grid = act_grid(g, 8);
  if (fmt == kE4M3)
    hipLaunchKernelGGL(act_bwd_kernel<kE4M3>, grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(act_bwd_kernel<kE5M2>, grid, dim3(256), 0, st, g);
}

}  // namespace qsg
