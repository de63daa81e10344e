// Combine: y_t = sum_i S_i[t] + sum_{k kept} g[t,k] * Y[slot_row[t,k]]
// (DeepSeekMoE explainer page, section 共有エキスパート機構, output equation;
// "Sparse MoE Top-Kルーティング" page, section ルーティングの仕組み, gate-weighted
// sum).  Accumulates in float32 in a fixed order: shared experts in index
// order, then slots k ascending; a dropped slot (row -1) adds nothing.
//
// One workgroup per token; the K (row, gate) pairs are loaded once into LDS
// and every thread walks 16-byte column chunks, so each row is read with
// fully coalesced 16-byte loads.  Pure HBM traffic: K gathered rows plus the
// shared rows in, one row out.
#include "moe_common.h"

namespace moe {
namespace {

typedef uint32_t nt4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  const nt4_t v = __builtin_nontemporal_load(reinterpret_cast<const nt4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4 *p, uint4 q) {
  __builtin_nontemporal_store((nt4_t){q.x, q.y, q.z, q.w}, reinterpret_cast<nt4_t *>(p));
}

template <bool BF16>
struct Chunk;   // 16 bytes of activations

template <>
struct Chunk<true> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void add(float *acc, const uint4 q, float g) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += g * __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += g * __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void add1(float *acc, const uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float *acc) {
    uint4 q;
    q.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    q.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    q.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    q.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    return q;
  }
};

template <>
struct Chunk<false> {
  static constexpr int kElems = 4;
  static __device__ __forceinline__ void add(float *acc, const uint4 q, float g) {
    acc[0] += g * __uint_as_float(q.x);
    acc[1] += g * __uint_as_float(q.y);
    acc[2] += g * __uint_as_float(q.z);
    acc[3] += g * __uint_as_float(q.w);
  }
  static __device__ __forceinline__ void add1(float *acc, const uint4 q) {
    acc[0] += __uint_as_float(q.x);
    acc[1] += __uint_as_float(q.y);
    acc[2] += __uint_as_float(q.z);
    acc[3] += __uint_as_float(q.w);
  }
  static __device__ __forceinline__ uint4 pack(const float *acc) {
    return make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                      __float_as_uint(acc[3]));
  }
};

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4 *__restrict__ y_rows,
                                                      const int32_t *__restrict__ slot_row,
                                                      const float *__restrict__ gates,
                                                      const uint4 *__restrict__ shared_out,
                                                      int n_shared, int64_t T, int K, int nvec,
                                                      uint4 *__restrict__ y) {
  using C = Chunk<BF16>;
  __shared__ int32_t s_row[64];
  __shared__ float s_gate[64];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) {
    s_row[threadIdx.x] = slot_row[t * K + threadIdx.x];
    s_gate[threadIdx.x] = gates[t * K + threadIdx.x];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
    float acc[C::kElems];
#pragma unroll
    for (int j = 0; j < C::kElems; ++j) acc[j] = 0.0f;
    // every input row is read once and the output is not read again here:
    // non-temporal loads and stores keep them from displacing cached data
    for (int sh = 0; sh < n_shared; ++sh)
      C::add1(acc, load_nt(&shared_out[(static_cast<int64_t>(sh) * T + t) * nvec + i]));
    for (int k = 0; k < K; ++k) {
      const int32_t r = s_row[k];
      if (r >= 0) C::add(acc, load_nt(&y_rows[static_cast<int64_t>(r) * nvec + i]), s_gate[k]);
    }
    store_nt(&y[t * nvec + i], C::pack(acc));
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, const void *y_rows, const int32_t *slot_row,
                          const float *gates, const void *shared_out, int n_shared, int64_t T,
                          int K, int d, void *y, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int nvec = d * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(T)), block(256);
  if (shared_out == nullptr) n_shared = 0;
  if (bf16)
    hipLaunchKernelGGL((combine_kernel<true>), grid, block, 0, s,
                       static_cast<const uint4 *>(y_rows), slot_row, gates,
                       static_cast<const uint4 *>(shared_out), n_shared, T, K, nvec,
                       static_cast<uint4 *>(y));
  else
    hipLaunchKernelGGL((combine_kernel<false>), grid, block, 0, s,
                       static_cast<const uint4 *>(y_rows), slot_row, gates,
                       static_cast<const uint4 *>(shared_out), n_shared, T, K, nvec,
                       static_cast<uint4 *>(y));
  return hipGetLastError();
}

}  // namespace moe
