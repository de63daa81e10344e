// Load statistics of one routing (DeepSeekMoE explainer page, section
// ルーティングとバランス損失, balance-loss equation):
//   f_j = (number of assignments (t, k) to expert j) / (T * K)
//   P_j = mean over tokens of the softmax over all N logits
//   L   = alpha * N * sum_j f_j * P_j
//
// Two passes, every sum in a fixed order so the results do not depend on
// timing:
//   1. one workgroup per 64 tokens, one wave per 16 of them: the wave holds a
//      token's N logits across its lanes, forms the softmax, and each lane
//      adds the probabilities of its experts token by token; the four waves'
//      sums are added in wave order into one partial row per workgroup;
//   2. one workgroup: an LDS histogram of the expert ids (integer counts, so
//      the order of the atomic adds does not matter), P_j as the sum of the
//      partial rows in row order, f_j, and the loss by a fixed tree.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokPerWave = 16;
constexpr int kTokPerBlock = 4 * kTokPerWave;

template <int J>   // J = ceil(N / 64) logits per lane
__global__ __launch_bounds__(256) void balance_partial_kernel(const float *__restrict__ logits,
                                                              int64_t T, int N,
                                                              float *__restrict__ partial) {
  __shared__ float s_part[4][J * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.0f;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + wave * kTokPerWave;
  for (int i = 0; i < kTokPerWave; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    const float *row = logits + t * N;
    float v[J];
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < N ? row[e] : -__builtin_inff();
      m = fmaxf(m, v[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      v[j] = (lane + 64 * j) < N ? expf(v[j] - m) : 0.0f;
      s += v[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] += v[j] * inv;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) s_part[wave][lane + 64 * j] = acc[j];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) {
    const float p = ((s_part[0][e] + s_part[1][e]) + s_part[2][e]) + s_part[3][e];
    partial[static_cast<int64_t>(blockIdx.x) * N + e] = p;
  }
}

__global__ __launch_bounds__(1024) void balance_final_kernel(const float *__restrict__ partial,
                                                             int64_t n_blocks,
                                                             const int32_t *__restrict__ idx,
                                                             int64_t T, int N, int K, float alpha,
                                                             float *__restrict__ f,
                                                             float *__restrict__ P,
                                                             float *__restrict__ loss) {
  __shared__ int s_count[kMaxRouted];
  __shared__ float s_term[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < N; e += 1024) s_count[e] = 0;
  __syncthreads();
  const int64_t n_assign = T * K;
  for (int64_t i = tid; i < n_assign; i += 1024) {
    const int e = idx[i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(N)) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();
  float term = 0.0f;
  if (tid < N) {
    float p = 0.0f;
    for (int64_t b = 0; b < n_blocks; ++b) p += partial[b * N + tid];
    p = p / static_cast<float>(T);
    const float fj = static_cast<float>(s_count[tid]) / static_cast<float>(n_assign);
    P[tid] = p;
    f[tid] = fj;
    term = fj * p;
  }
  s_term[tid] = term;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if (tid < w) s_term[tid] += s_term[tid + w];
    __syncthreads();
  }
  if (tid == 0) *loss = alpha * static_cast<float>(N) * s_term[0];
}

}  // namespace

size_t balance_workspace_bytes(int64_t T, int N) {
  const int64_t blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  return sizeof(float) * static_cast<size_t>(blocks) * N;
}

hipError_t launch_balance_stats(const float *logits, const int32_t *idx, int64_t T, int N, int K,
                                float alpha, float *f, float *P, float *loss, void *ws,
                                hipStream_t s) {
  const int64_t blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  float *partial = static_cast<float *>(ws);
  const int J = (N + 63) / 64;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (J <= 1)
    hipLaunchKernelGGL((balance_partial_kernel<1>), grid, block, 0, s, logits, T, N, partial);
  else if (J <= 2)
    hipLaunchKernelGGL((balance_partial_kernel<2>), grid, block, 0, s, logits, T, N, partial);
  else if (J <= 4)
    hipLaunchKernelGGL((balance_partial_kernel<4>), grid, block, 0, s, logits, T, N, partial);
  else if (J <= 8)
    hipLaunchKernelGGL((balance_partial_kernel<8>), grid, block, 0, s, logits, T, N, partial);
  else if (J <= 16)
    hipLaunchKernelGGL((balance_partial_kernel<16>), grid, block, 0, s, logits, T, N, partial);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(1024), 0, s, partial, blocks, idx, T, N,
                     K, alpha, f, P, loss);
  return hipGetLastError();
}

}  // namespace moe
