// Router scores, top-K selection and renormalised gates.
//
// Router: one score per expert from a bias-free linear map of the token
// ("Sparse MoE Top-Kルーティング" page, section ルーティングの仕組み; the
// DeepSeekMoE explainer page, gate equation s = softmax(W_r x)), plus an
// optional per-expert bias that is part of the logit.
//
// Fixed float32 order: for every (t, e) one fused multiply-add chain over k
// ascending from +0, then the bias with one rounding.  Each thread owns whole
// logits, so no reduction tree is involved and the bits do not depend on the
// launch shape.
//
// Top-K: one wave per token, N logits spread over the lanes' registers, K
// rounds of a wave-wide arg-max on the key (logit desc, expert id asc).  Gates
// are the softmax over the K kept logits, which equals s_j / sum_TopK s_k of
// the DeepSeekMoE explainer's gate equation.
#include "moe_common.h"

namespace moe {
namespace {

// Logits as a register-tiled product: a workgroup covers BT tokens x BE
// experts, each thread MT tokens x ME experts; K advances in chunks of KC
// staged through LDS (x converted to float32 exactly, layout [k][token] and
// [k][expert] so each thread reads its MT / ME values as one vector).  Every
// accumulator still sees its terms one at a time in ascending k.
template <int BT, int BE, int MT, int ME, int KC, bool BF16>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void *__restrict__ xv, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int N) {
  constexpr int NTT = BT / MT;                  // thread columns over tokens
  static_assert(NTT * (BE / ME) == 256, "256 threads per workgroup");
  constexpr int XV = BF16 ? 8 : 4;              // x elements per 16-byte load
  constexpr int X_LOADS = BT * KC / XV;         // 16-byte loads per x chunk
  constexpr int W_LOADS = BE * KC / 4;          // 16-byte loads per W chunk
  constexpr int XPT = (X_LOADS + 255) / 256;    // per thread
  constexpr int WPT = (W_LOADS + 255) / 256;
  __shared__ __attribute__((aligned(16))) float s_x[2][KC][BT];
  __shared__ __attribute__((aligned(16))) float s_w[2][KC][BE];

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e0 = blockIdx.y * BE;
  const int tm = tid % NTT, te = tid / NTT;

  uint4 rx[XPT];
  float4 rw[WPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int id = tid + i * 256;
      if (id < X_LOADS) {
        const int r = id / (KC / XV), c = id % (KC / XV);
        int64_t t = t0 + r;
        if (t >= T) t = T - 1;
        if constexpr (BF16)
          rx[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xv) + t * d + k0 + c * XV);
        else
          rx[i] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(xv) + t * d + k0 + c * XV);
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256;
      if (id < W_LOADS) {
        const int r = id / (KC / 4), c = id % (KC / 4);
        int e = e0 + r;
        if (e >= N) e = N - 1;
        rw[i] = *reinterpret_cast<const float4 *>(w + static_cast<int64_t>(e) * d + k0 + c * 4);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int id = tid + i * 256;
      if (id < X_LOADS) {
        const int r = id / (KC / XV), c = id % (KC / XV);
        if constexpr (BF16) {
          const uint32_t q[4] = {rx[i].x, rx[i].y, rx[i].z, rx[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s_x[buf][c * 8 + 2 * j][r] = __uint_as_float(q[j] << 16);
            s_x[buf][c * 8 + 2 * j + 1][r] = __uint_as_float(q[j] & 0xFFFF0000u);
          }
        } else {
          s_x[buf][c * 4 + 0][r] = __uint_as_float(rx[i].x);
          s_x[buf][c * 4 + 1][r] = __uint_as_float(rx[i].y);
          s_x[buf][c * 4 + 2][r] = __uint_as_float(rx[i].z);
          s_x[buf][c * 4 + 3][r] = __uint_as_float(rx[i].w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256;
      if (id < W_LOADS) {
        const int r = id / (KC / 4), c = id % (KC / 4);
        s_w[buf][c * 4 + 0][r] = rw[i].x;
        s_w[buf][c * 4 + 1][r] = rw[i].y;
        s_w[buf][c * 4 + 2][r] = rw[i].z;
        s_w[buf][c * 4 + 3][r] = rw[i].w;
      }
    }
  };

  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.0f;

  const int nchunks = d / KC;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunks) gload((ch + 1) * KC);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float xs[MT], ws[ME];
#pragma unroll
      for (int i = 0; i < MT; ++i) xs[i] = s_x[buf][k][tm * MT + i];
#pragma unroll
      for (int j = 0; j < ME; ++j) ws[j] = s_w[buf][k][te * ME + j];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < ME; ++j) acc[i][j] = __builtin_fmaf(xs[i], ws[j], acc[i][j]);
    }
    if (ch + 1 < nchunks) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t t = t0 + tm * MT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < ME; ++j) {
      const int e = e0 + te * ME + j;
      if (e >= N) continue;
      float v = acc[i][j];
      if (bias) v = v + bias[e];
      logits[t * N + e] = v;
    }
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
  // Block shapes measured on MI355X: wide routers over many tokens use 32x64
  // blocks with 2x4 logits per thread, mid-sized ones 32x32 with 2x2, and
  // short batches or narrow routers 64x8 with 2x1, so that they still spread
  // over the chip.
  const int64_t TN = T * static_cast<int64_t>(N);
  const int kc32 = d % 32 == 0;
#define MOE_ROUTER_LAUNCH(BT, BE, MT, ME, KC)                                                   \
  {                                                                                             \
    const dim3 grid(static_cast<unsigned>((T + BT - 1) / BT),                                   \
                    static_cast<unsigned>((N + BE - 1) / BE));                                  \
    if (bf16)                                                                                   \
      hipLaunchKernelGGL((router_logits_kernel<BT, BE, MT, ME, KC, true>), grid, dim3(256), 0, \
                         s, x, w, bias, logits, T, d, N);                                       \
    else                                                                                        \
      hipLaunchKernelGGL((router_logits_kernel<BT, BE, MT, ME, KC, false>), grid, dim3(256), 0,\
                         s, x, w, bias, logits, T, d, N);                                       \
  }
  if (N >= 64 && TN >= (int64_t(1) << 19)) {
    if (kc32) MOE_ROUTER_LAUNCH(32, 64, 2, 4, 32) else MOE_ROUTER_LAUNCH(32, 64, 2, 4, 16)
  } else if (N >= 32 && TN >= (int64_t(1) << 17)) {
    if (kc32) MOE_ROUTER_LAUNCH(32, 32, 2, 2, 32) else MOE_ROUTER_LAUNCH(32, 32, 2, 2, 16)
  } else {
    if (kc32) MOE_ROUTER_LAUNCH(64, 8, 2, 1, 32) else MOE_ROUTER_LAUNCH(64, 8, 2, 1, 16)
  }
#undef MOE_ROUTER_LAUNCH
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
