// FP8 dispatch of token rows (DeepEP page, section "DeepEP とは？", item 5:
// native FP8 data dispatch, which cuts the bytes the dispatch moves; section
// "DeepEP の性能": FP8 dispatch with BF16 combine).  The pages fix neither the
// format nor the scaling; this library uses OCP FP8 E4M3 (sign, 4 exponent
// bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite
// value 448) with one power-of-two scale per token row: 2^E, E the smallest
// integer with max_k |x[t,k]| <= 448 * 2^E (0 for an all-zero row), and codes
// x / 2^E rounded to the nearest E4M3 value, ties to the even mantissa.  A
// power-of-two scale keeps the division and the later widening exact, so the
// codes are a pure function of x.
//
// One wave per token row: the row's largest magnitude (bf16 magnitudes order
// as their 15-bit patterns), E from its exponent and mantissa bits, then the
// codes of 8 elements per lane per step (16-byte loads, 8-byte stores).
//
// The same pass also writes the row the receiving side gets back: each code
// widened to its E4M3 value times 2^E and rounded to bf16 (exact, since an
// E4M3 value has at most 4 significant bits, unless the product falls below
// bf16's subnormal range), which the experts' first Linear then reads like
// any bf16 row.
#include "moe_common.h"

namespace moe {
namespace {

// Smallest E with a <= 448 * 2^E for a finite a > 0 given as float32 bits:
// with a = m * 2^e, m in [0.5, 1), and 448 = 0.875 * 2^9, E = e - 9 when
// m <= 0.875, else e - 8.
__device__ __forceinline__ int scale_exponent(uint32_t bits) {
  const uint32_t ea = (bits >> 23) & 0xFF, ma = bits & 0x7FFFFF;
  if (ea == 0) {
    if (ma == 0) return 0;
    const int b = 31 - __clz(ma);                   // leading one of a subnormal
    const bool small = b < 2 || ma <= (7u << (b - 2));
    return (b - 148) - (small ? 9 : 8);
  }
  const int e = static_cast<int>(ea) - 126;
  return ma <= 0x600000u ? e - 9 : e - 8;
}

// E4M3 code of v (|v| <= 448), round to nearest even.  Below 2^-6 the grid
// step is 2^-9, so the code is v * 512 rounded to an integer (exact product,
// hardware round-half-even); above, the float32 mantissa is rounded to three
// bits (a carry moves into the exponent) and re-biased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t e = (b >> 23) - 120u;              // (exp - 127) + 7
  return sign | (e << 3) | ((b >> 20) & 7u);
}

// Eight E4M3 codes (bytes of cw, element order) widened to bf16 times the
// row's scale sc = 2^E: v_cvt_pk_f32_fp8 gives each code's value exactly in
// float32, the product by 2^E is exact unless it leaves float32's normal
// range, and the value (at most 4 significant bits) is exact in bf16.
__device__ __forceinline__ uint4 widen_fp8x8(uint2 cw, float sc) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw.x), false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw.x), true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw.y), false);
  const f32x2_t e = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(cw.y), true);
  uint4 o;
  o.x = pack_bf16x2(a.x * sc, a.y * sc);
  o.y = pack_bf16x2(b.x * sc, b.y * sc);
  o.z = pack_bf16x2(c.x * sc, c.y * sc);
  o.w = pack_bf16x2(e.x * sc, e.y * sc);
  return o;
}

__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const uint16_t *__restrict__ x,
                                                                int64_t T, int d,
                                                                uint8_t *__restrict__ q,
                                                                int32_t *__restrict__ exps,
                                                                uint16_t *__restrict__ xw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t *row = x + t * d;
  const int nv = d / 8;                              // 8-element groups (d % 64 == 0)
  uint32_t amax = 0;
  for (int i = lane; i < nv; i += 64) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + i * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, w[j] & 0x7FFFu);
      amax = max(amax, (w[j] >> 16) & 0x7FFFu);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = max(amax, static_cast<uint32_t>(__shfl_xor(amax, off)));
  const int E = scale_exponent(amax << 16);
  const float sc = __builtin_ldexpf(1.0f, E);
  if (lane == 0) exps[t] = E;
  uint8_t *qrow = q + t * d;
  for (int i = lane; i < nv; i += 64) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + i * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = e4m3_code(__builtin_ldexpf(__uint_as_float(w[j] << 16), -E));
      c[2 * j + 1] = e4m3_code(__builtin_ldexpf(__uint_as_float(w[j] & 0xFFFF0000u), -E));
    }
    uint2 out;
    out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<uint2 *>(qrow + i * 8) = out;
    if (xw) *reinterpret_cast<uint4 *>(xw + t * d + i * 8) = widen_fp8x8(out, sc);
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void *x, int64_t T, int d, uint8_t *q, int32_t *exps,
                               void *xw, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4));
  hipLaunchKernelGGL(quantize_rows_fp8_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t *>(x), T, d, q, exps,
                     static_cast<uint16_t *>(xw));
  return hipGetLastError();
}

}  // namespace moe
