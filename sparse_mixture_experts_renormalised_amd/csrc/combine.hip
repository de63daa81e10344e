// Combine: y_t = sum_i S_i[t] + sum_{k kept} g[t,k] * Y[slot_row[t,k]]
// (DeepSeekMoE explainer page, section 共有エキスパート機構, output equation;
// "Sparse MoE Top-Kルーティング" page, section ルーティングの仕組み, gate-weighted
// sum).  Accumulates in float32 in a fixed order: shared experts in index
// order, then slots k ascending; a dropped slot (row -1) adds nothing.
//
// Workgroup (t, b) of B covers the 16-byte column chunks 256 b + 256 B j ..
// of token t's row (B = 1 for many tokens, more for few); the K (row, gate)
// pairs are loaded once into LDS, and each row is read with fully coalesced
// 16-byte loads.  Pure HBM
// traffic: K gathered rows plus the shared rows in, one row out.
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

template <bool BF16, int BATCH>
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
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < nvec; i += gridDim.y * blockDim.x) {
    float acc[C::kElems];
#pragma unroll
    for (int j = 0; j < C::kElems; ++j) acc[j] = 0.0f;
    // every input row is read once and the output is not read again here:
    // non-temporal loads and stores keep them from displacing cached data
    for (int sh = 0; sh < n_shared; ++sh)
      C::add1(acc, load_nt(&shared_out[(static_cast<int64_t>(sh) * T + t) * nvec + i]));
    if constexpr (BATCH == 1) {
      for (int k = 0; k < K; ++k) {
        const int32_t r = s_row[k];
        if (r >= 0) C::add(acc, load_nt(&y_rows[static_cast<int64_t>(r) * nvec + i]), s_gate[k]);
      }
    } else {
      // slots in batches of BATCH: a batch's loads are all issued before its
      // first add, and the adds keep slot order
      for (int k0 = 0; k0 < K; k0 += BATCH) {
        uint4 q[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const int32_t r = k0 + j < K ? s_row[k0 + j] : -1;
          if (r >= 0) q[j] = load_nt(&y_rows[static_cast<int64_t>(r) * nvec + i]);
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const int32_t r = k0 + j < K ? s_row[k0 + j] : -1;
          if (r >= 0) C::add(acc, q[j], s_gate[k0 + j]);
        }
      }
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
  // few tokens (decode): one 16-byte column chunk per thread, a token's row
  // spread over nvec / 256 workgroups; many tokens: one workgroup per token
  // walks its row (measured on MI355X)
  const unsigned split = T < 1024 ? static_cast<unsigned>((nvec + 255) / 256) : 1u;
  const dim3 grid(static_cast<unsigned>(T), split), block(256);
  if (shared_out == nullptr) n_shared = 0;
  const uint4 *yr = static_cast<const uint4 *>(y_rows);
  const uint4 *sh = static_cast<const uint4 *>(shared_out);
  uint4 *yo = static_cast<uint4 *>(y);
  // the split path also loads eight slot rows before adding them (decode);
  // with many tokens in flight the plain loop measures faster
  if (bf16) {
    if (split > 1)
      hipLaunchKernelGGL((combine_kernel<true, 8>), grid, block, 0, s, yr, slot_row, gates, sh, n_shared, T, K, nvec, yo);
    else
      hipLaunchKernelGGL((combine_kernel<true, 1>), grid, block, 0, s, yr, slot_row, gates, sh, n_shared, T, K, nvec, yo);
  } else {
    if (split > 1)
      hipLaunchKernelGGL((combine_kernel<false, 8>), grid, block, 0, s, yr, slot_row, gates, sh, n_shared, T, K, nvec, yo);
    else
      hipLaunchKernelGGL((combine_kernel<false, 1>), grid, block, 0, s, yr, slot_row, gates, sh, n_shared, T, K, nvec, yo);
  }
  return hipGetLastError();
}

}  // namespace moe
