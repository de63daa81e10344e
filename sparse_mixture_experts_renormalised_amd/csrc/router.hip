// Router scores, top-K selection and renormalised gates.
//
// Router: one score per expert from a bias-free linear map of the token
// ("Sparse MoE Top-Kルーティング" page, section ルーティングの仕組み; the
// DeepSeekMoE explainer page, gate equation s = softmax(W_r x)), plus an
// optional per-expert bias that is part of the logit.
//
// Fixed float32 order: for every (t, e) one fused multiply-add chain over k
// ascending from +0, then the bias with one rounding.  Each lane owns whole
// logits, so no reduction tree is involved and the bits do not depend on the
// launch shape.  A wave covers 64 tokens (one per lane) and ME experts; the
// expert weights are wave-uniform and come in through scalar loads, so each
// fused multiply-add is one VALU instruction with an SGPR operand.
//
// Top-K: one wave per token, N logits spread over the lanes' registers, K
// rounds of a wave-wide arg-max on the key (logit desc, expert id asc).  Gates
// are the softmax over the K kept logits, which equals s_j / sum_TopK s_k of
// the DeepSeekMoE explainer's gate equation.
#include "moe_common.h"

namespace moe {
namespace {

template <int ME, bool BF16>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void *__restrict__ xv, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int N) {
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_eg = N / ME;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t tg = gw / n_eg;
  const int eg = static_cast<int>(gw - tg * n_eg);
  const int64_t t0 = tg * kWave;
  if (t0 >= T) return;
  const int64_t t = t0 + lane;
  const bool valid = t < T;
  const int64_t tc = valid ? t : T - 1;
  const float *__restrict__ wr = w + static_cast<int64_t>(eg) * ME * d;

  float acc[ME];
#pragma unroll
  for (int e = 0; e < ME; ++e) acc[e] = 0.0f;

  if constexpr (BF16) {
    const uint4 *xr = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xv) + tc * d);
    for (int k8 = 0; k8 < (d >> 3); ++k8) {
      const uint4 q = xr[k8];
      float xs[8];
      xs[0] = __uint_as_float(q.x << 16); xs[1] = __uint_as_float(q.x & 0xFFFF0000u);
      xs[2] = __uint_as_float(q.y << 16); xs[3] = __uint_as_float(q.y & 0xFFFF0000u);
      xs[4] = __uint_as_float(q.z << 16); xs[5] = __uint_as_float(q.z & 0xFFFF0000u);
      xs[6] = __uint_as_float(q.w << 16); xs[7] = __uint_as_float(q.w & 0xFFFF0000u);
      const float *wk = wr + (k8 << 3);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int e = 0; e < ME; ++e) acc[e] = __builtin_fmaf(xs[j], wk[e * d + j], acc[e]);
      }
    }
  } else {
    const float4 *xr = reinterpret_cast<const float4 *>(static_cast<const float *>(xv) + tc * d);
    for (int k8 = 0; k8 < (d >> 3); ++k8) {
      const float4 a = xr[2 * k8], b = xr[2 * k8 + 1];
      const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const float *wk = wr + (k8 << 3);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int e = 0; e < ME; ++e) acc[e] = __builtin_fmaf(xs[j], wk[e * d + j], acc[e]);
      }
    }
  }
  if (!valid) return;
  float *out = logits + t * N + static_cast<int64_t>(eg) * ME;
#pragma unroll
  for (int e = 0; e < ME; ++e) {
    float v = acc[e];
    if (bias) v = v + bias[eg * ME + e];
    out[e] = v;
  }
}

// Key order: a beats b iff a.v > b.v, or equal values and a.i < b.i.
__device__ __forceinline__ bool key_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int J>   // J = ceil(N / 64) logits per lane
__global__ __launch_bounds__(256) void topk_gates_kernel(const float *__restrict__ logits,
                                                         int64_t T, int N, int K,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + t * N;
  float v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < N ? row[e] : -__builtin_inff();
  }
  uint32_t taken = 0;
  float kept_v = 0.0f;   // lane k keeps slot k's logit
  int kept_i = 0;
  float best0 = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < N && !((taken >> j) & 1u) && key_better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (key_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (k == 0) best0 = bv;
    if (lane == k) { kept_v = bv; kept_i = bi; }
  }
  // softmax over the K kept logits, shifted by the largest (slot 0)
  const float p = lane < K ? expf(kept_v - best0) : 0.0f;
  float s = p;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane < K) {
    idx[t * K + lane] = kept_i;
    gates[t * K + lane] = p / s;
  }
}

}  // namespace

hipError_t launch_router_logits(bool bf16, const void *x, const float *w, const float *bias,
                                float *logits, int64_t T, int d, int N, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // experts per wave: keep at least ~2048 waves in flight when the shape allows
  const int64_t tgroups = (T + kWave - 1) / kWave;
  int me = 1;
  for (int cand : {16, 8, 4, 2}) {
    if (N % cand == 0 && tgroups * (N / cand) >= 2048) { me = cand; break; }
  }
  const int64_t waves = tgroups * (N / me);
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
#define MOE_ROUTER_CASE(ME)                                                                   \
  case ME:                                                                                    \
    if (bf16)                                                                                 \
      hipLaunchKernelGGL((router_logits_kernel<ME, true>), grid, block, 0, s, x, w, bias,    \
                         logits, T, d, N);                                                    \
    else                                                                                      \
      hipLaunchKernelGGL((router_logits_kernel<ME, false>), grid, block, 0, s, x, w, bias,   \
                         logits, T, d, N);                                                    \
    break;
  switch (me) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

hipError_t launch_topk_gates(const float *logits, int64_t T, int N, int K, int32_t *idx,
                             float *gates, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4)), block(256);
  const int J = (N + 63) / 64;
  if (J <= 1) {
    hipLaunchKernelGGL((topk_gates_kernel<1>), grid, block, 0, s, logits, T, N, K, idx, gates);
  } else if (J <= 2) {
    hipLaunchKernelGGL((topk_gates_kernel<2>), grid, block, 0, s, logits, T, N, K, idx, gates);
  } else if (J <= 4) {
    hipLaunchKernelGGL((topk_gates_kernel<4>), grid, block, 0, s, logits, T, N, K, idx, gates);
  } else if (J <= 8) {
    hipLaunchKernelGGL((topk_gates_kernel<8>), grid, block, 0, s, logits, T, N, K, idx, gates);
  } else if (J <= 16) {
    hipLaunchKernelGGL((topk_gates_kernel<16>), grid, block, 0, s, logits, T, N, K, idx, gates);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
