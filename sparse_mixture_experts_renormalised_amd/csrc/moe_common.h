// Internal helpers shared by the MoE kernels (device side) and the host
// launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxRouted = 1024;   // top-K keeps up to 16 logits per lane
constexpr int kMaxShared = 64;

// bfloat16 is carried as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Two floats to packed bfloat16 (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950, the same bits as f32_to_bf16 on each.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_hw_t));
}

// 16-byte store of a layer output that the kernel does not read back, with
// the non-temporal policy so that it does not displace operand data in the
// caches.  (Measured: this helps full-line tile stores; partial-line 8-byte
// stores lose their write combining and get slower.)
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ void store_nt(uint16_t *p, V v) {
  static_assert(sizeof(V) == 16, "16-byte vectors");
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt_t, v), reinterpret_cast<u32x4_nt_t *>(p));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// SiLU with the hardware exp2 and reciprocal (about 1 ulp each in float32),
// for epilogues that round to bfloat16 right after.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace moe

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files, called from moe_api.cpp)
// ---------------------------------------------------------------------------
namespace moe {

struct GemmGroups {
  // Routed groups: rows offsets[g] .. offsets[g+1]-1 (device array).
  const int32_t *offsets;
  int n_routed;
  // A rows of routed groups: row r reads A[r], or A[a_index[r]] when a_index
  // is set (the dispatch gather fused into the load).
  const void *A;
  const int32_t *a_index;
  // Shared groups: rows 0..T_sh-1 of each, reading A_sh + g*a_sh_stride
  // (elements) + r*K.
  int n_shared;
  int64_t T_sh;
  const void *A_sh;
  int64_t a_sh_stride;
  // Weights [G][Nout][K], biases [G][Nout] or NULL.
  const void *W, *bias, *W_sh, *bias_sh;
  // Outputs: routed row r -> C + r*Nout; shared group g row t ->
  // C_sh + (g*T_sh + t)*Nout.
  void *C, *C_sh;
  int Nout, K;
  int64_t max_routed_rows;   // host upper bound on offsets[n_routed]
  int64_t max_group_rows;    // host upper bound on the rows of one routed group
  // Optional scratch (split_bytes bytes, 256-aligned) for splitting K when
  // a product's work does not divide evenly over the chip; NULL: never split.
  void *split_ws;
  size_t split_bytes;
};

// Scratch bytes with which launch_grouped_gemm splits this product (and
// every smaller one) as it sees fit; needs only Nout, n_routed, n_shared,
// T_sh and max_routed_rows.
size_t grouped_gemm_split_bytes(const GemmGroups &g);

enum Epilogue { kEpiBias = 0, kEpiBiasSilu = 1 };

hipError_t launch_router_logits(bool bf16, const void *x, const float *w, const float *bias,
                                float *logits, int64_t T, int d, int N, hipStream_t s);
hipError_t launch_topk_gates(const float *logits, const float *sel_bias, int64_t T, int N, int K,
                             int32_t *idx, float *gates, hipStream_t s);
size_t balance_workspace_bytes(int64_t T, int N);
hipError_t launch_balance_stats(const float *logits, const int32_t *idx, int64_t T, int N, int K,
                                float alpha, float *f, float *P, float *loss, void *ws,
                                hipStream_t s);
hipError_t launch_dispatch(const int32_t *idx, int64_t T, int K, int N, int64_t capacity,
                           int32_t *counts, int32_t *offsets, int32_t *row_token,
                           int32_t *slot_row, int32_t *n_dropped, void *ws, hipStream_t s);
size_t dispatch_workspace_bytes(int64_t T, int K, int N);
hipError_t launch_gather_rows(bool bf16, const void *x, const int32_t *row_token,
                              const int32_t *total_rows, int64_t max_rows, int d, void *out,
                              hipStream_t s);
hipError_t launch_grouped_gemm(bool bf16, const GemmGroups &g, Epilogue epi, hipStream_t s);
// E4M3 codes q [T][d] and per-row scale exponents exps [T] of x (bf16), and,
// when xw is not null, the codes widened back to bf16 rows xw [T][d].
hipError_t launch_quantize_fp8(const void *x, int64_t T, int d, uint8_t *q, int32_t *exps,
                               void *xw, hipStream_t s);
hipError_t launch_combine(bool bf16, const void *y_rows, const int32_t *slot_row,
                          const float *gates, const void *shared_out, int n_shared, int64_t T,
                          int K, int d, void *y, hipStream_t s);

}  // namespace moe
