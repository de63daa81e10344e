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
// [k][expert] so each thread reads its MT / ME values as one vector).  Global
// loads run PF chunks ahead (PF = 2: two register sets).  Every accumulator
// still sees its terms one at a time in ascending k.
template <int BT, int BE, int MT, int ME, int KC, bool BF16, int PF = 1>
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

  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.0f;
  uint4 rx[2][XPT];
  float4 rw[2][WPT];
  auto gload_set = [&](uint4 (&rxs)[XPT], float4 (&rws)[WPT], int k0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int id = tid + i * 256;
      if (id < X_LOADS) {
        const int r = id / (KC / XV), c = id % (KC / XV);
        int64_t t = t0 + r;
        if (t >= T) t = T - 1;
        if constexpr (BF16)
          rxs[i] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xv) + t * d + k0 + c * XV);
        else
          rxs[i] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(xv) + t * d + k0 + c * XV);
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256;
      if (id < W_LOADS) {
        const int r = id / (KC / 4), c = id % (KC / 4);
        int e = e0 + r;
        if (e >= N) e = N - 1;
        rws[i] = *reinterpret_cast<const float4 *>(w + static_cast<int64_t>(e) * d + k0 + c * 4);
      }
    }
  };
  auto lstore_set = [&](int buf, const uint4 (&rxs)[XPT], const float4 (&rws)[WPT]) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int id = tid + i * 256;
      if (id < X_LOADS) {
        const int r = id / (KC / XV), c = id % (KC / XV);
        if constexpr (BF16) {
          const uint32_t q[4] = {rxs[i].x, rxs[i].y, rxs[i].z, rxs[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s_x[buf][c * 8 + 2 * j][r] = __uint_as_float(q[j] << 16);
            s_x[buf][c * 8 + 2 * j + 1][r] = __uint_as_float(q[j] & 0xFFFF0000u);
          }
        } else {
          s_x[buf][c * 4 + 0][r] = __uint_as_float(rxs[i].x);
          s_x[buf][c * 4 + 1][r] = __uint_as_float(rxs[i].y);
          s_x[buf][c * 4 + 2][r] = __uint_as_float(rxs[i].z);
          s_x[buf][c * 4 + 3][r] = __uint_as_float(rxs[i].w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256;
      if (id < W_LOADS) {
        const int r = id / (KC / 4), c = id % (KC / 4);
        s_w[buf][c * 4 + 0][r] = rws[i].x;
        s_w[buf][c * 4 + 1][r] = rws[i].y;
        s_w[buf][c * 4 + 2][r] = rws[i].z;
        s_w[buf][c * 4 + 3][r] = rws[i].w;
      }
    }
  };

  auto gload = [&](int k0) { gload_set(rx[0], rw[0], k0); };
  auto lstore = [&](int buf) { lstore_set(buf, rx[0], rw[0]); };
  auto compute = [&](int buf) {
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
  };

  const int nchunks = d / KC;
  if constexpr (PF == 1) {
    gload(0);
    lstore(0);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
      const int buf = ch & 1;
      if (ch + 1 < nchunks) gload((ch + 1) * KC);
      compute(buf);
      if (ch + 1 < nchunks) lstore(buf ^ 1);
      __syncthreads();
    }
  } else {
    // loads run two chunks ahead in two register sets: chunk c+2 is loaded
    // while chunk c is multiplied and stored to LDS at the end of chunk c+1
    gload_set(rx[0], rw[0], 0);
    if (nchunks > 1) gload_set(rx[1], rw[1], KC);
    lstore_set(0, rx[0], rw[0]);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ch += 2) {
      if (ch + 2 < nchunks) gload_set(rx[0], rw[0], (ch + 2) * KC);
      compute(0);
      if (ch + 1 < nchunks) lstore_set(1, rx[1], rw[1]);
      __syncthreads();
      if (ch + 1 >= nchunks) break;
      if (ch + 3 < nchunks) gload_set(rx[1], rw[1], (ch + 3) * KC);
      compute(1);
      if (ch + 2 < nchunks) lstore_set(0, rx[0], rw[0]);
      __syncthreads();
    }
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

// Short batches (and narrow routers) have few logits, each a long chain, so
// the LDS tiles above cannot keep enough memory traffic in flight.  Here a
// workgroup of 128 threads owns 16 tokens x 8 experts, one logit per thread,
// and streams 64-wide k-chunks of x (bf16, as stored) and W (float32) into a
// ring of S LDS stages with global-to-LDS copies issued S-1 chunks ahead.  A
// copy instruction moves 1 KB: 8 rows of x or 4 rows of W.  x rows are 128
// bytes of 8 pieces; piece c of row r sits at c ^ ((r >> 1) & 7), so the 16
// tokens read by a 16-lane group hit distinct banks; the W row of such a
// group is one broadcast address.
namespace ring {
constexpr int NT = 128, BT = 16, BE = 8, KC = 64;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// One wave-wide copy of 64 x 16 bytes into the LDS block at byte address m0.
__device__ __forceinline__ void dma16(const void *src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int LPS, int MAXN>
__device__ __forceinline__ void wait_chunks(int n) {
  if constexpr (MAXN >= 0) {
    if (n >= MAXN) {
      wait_and_barrier<MAXN * LPS>();
      return;
    }
    wait_chunks<LPS, MAXN - 1>(n);
  }
}
}  // namespace ring

template <int S>
__global__ __launch_bounds__(128) void router_logits_ring_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int N) {
  using namespace ring;
  constexpr int XB = BT * KC * 2;                // bytes of x per stage (2 KB)
  constexpr int WB = BE * KC * 4;                // bytes of W per stage (2 KB)
  constexpr int STAGE = XB + WB;
  constexpr int LPS = 2;                         // copies per wave per stage
  static_assert((S - 2) * LPS <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[S * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int tt = tid & 15, te = tid >> 4;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e0 = blockIdx.y * BE;
  const uint32_t ring0 = uniform(static_cast<int>(lds_addr(s_ring)));

  // wave w copies x rows 8w .. 8w+7 and W rows 4w .. 4w+3 of every chunk
  const int xr = 8 * wave + (lane >> 3);
  int64_t xt = t0 + xr;
  if (xt >= T) xt = T - 1;
  const uint16_t *x_src = x + xt * d + ((lane & 7) ^ ((xr >> 1) & 7)) * 8;
  const int wr = 4 * wave + (lane >> 4);
  const int we = min(e0 + wr, N - 1);
  const float *w_src = w + static_cast<int64_t>(we) * d + (lane & 15) * 4;
  auto issue = [&](int c, int st) {
    const uint32_t base = ring0 + static_cast<uint32_t>(st) * STAGE;
    dma16(x_src + c * KC, base + wave * 1024);
    dma16(w_src + c * KC, base + XB + wave * 1024);
  };

  const int nch = d / KC;
  float acc = 0.0f;
  // a chunk's operands are read from LDS into registers before its chain of
  // multiply-adds, so the LDS latency is paid once per chunk
  uint4 xa[KC / 8];
  float4 wa[KC / 4];
  auto read = [&](int c, uint4 (&xq)[KC / 8], float4 (&wv)[KC / 4]) {
    const uint8_t *st = s_ring + (c % S) * STAGE;
    const uint16_t *xs = reinterpret_cast<const uint16_t *>(st) + tt * KC;
    const float *ws = reinterpret_cast<const float *>(st + XB) + te * KC;
#pragma unroll
    for (int pc = 0; pc < KC / 8; ++pc) {
      xq[pc] = *reinterpret_cast<const uint4 *>(xs + ((pc ^ ((tt >> 1) & 7)) << 3));
      wv[2 * pc] = *reinterpret_cast<const float4 *>(ws + pc * 8);
      wv[2 * pc + 1] = *reinterpret_cast<const float4 *>(ws + pc * 8 + 4);
    }
  };
  auto chain = [&](const uint4 (&xq)[KC / 8], const float4 (&wv)[KC / 4]) {
#pragma unroll
    for (int pc = 0; pc < KC / 8; ++pc) {
      const uint4 q = xq[pc];
      const float4 u = wv[2 * pc], v = wv[2 * pc + 1];
      acc = __builtin_fmaf(__uint_as_float(q.x << 16), u.x, acc);
      acc = __builtin_fmaf(__uint_as_float(q.x & 0xFFFF0000u), u.y, acc);
      acc = __builtin_fmaf(__uint_as_float(q.y << 16), u.z, acc);
      acc = __builtin_fmaf(__uint_as_float(q.y & 0xFFFF0000u), u.w, acc);
      acc = __builtin_fmaf(__uint_as_float(q.z << 16), v.x, acc);
      acc = __builtin_fmaf(__uint_as_float(q.z & 0xFFFF0000u), v.y, acc);
      acc = __builtin_fmaf(__uint_as_float(q.w << 16), v.z, acc);
      acc = __builtin_fmaf(__uint_as_float(q.w & 0xFFFF0000u), v.w, acc);
    }
  };
  const int pro = min(S - 1, nch);
  for (int c = 0; c < pro; ++c) issue(c, c % S);
  for (int c = 0; c < nch; ++c) {
    // copies of chunks c+1 .. min(c+S-2, nch-1) may stay in flight
    const int later = min(S - 2, nch - 1 - c);
    if (later == S - 2) wait_and_barrier<(S - 2) * LPS>();
    else wait_chunks<LPS, S - 3>(later);
    if (c + S - 1 < nch) issue(c + S - 1, (c + S - 1) % S);
    read(c, xa, wa);
    chain(xa, wa);
  }
  const int64_t t = t0 + tt;
  const int e = e0 + te;
  if (t < T && e < N) {
    float v = acc;
    if (bias) v = v + bias[e];
    logits[t * N + e] = v;
  }
}

// Key order: a beats b iff a.v > b.v, or equal values and a.i < b.i.
__device__ __forceinline__ bool key_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int J>   // J = ceil(N / 64) logits per lane
__global__ __launch_bounds__(256) void topk_gates_kernel(const float *__restrict__ logits,
                                                         const float *__restrict__ sel_bias,
                                                         int64_t T, int N, int K,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + t * N;
  float v[J], key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < N ? row[e] : -__builtin_inff();
    // selection key: the logit, or (selection-only bias) fl32(logit + bias)
    key[j] = (sel_bias && e < N) ? v[j] + sel_bias[e] : v[j];
  }
  uint32_t taken = 0;
  float kept_v = -__builtin_inff();   // lane k keeps slot k's (unbiased) logit
  int kept_i = 0;
  for (int k = 0; k < K; ++k) {
    float bk = -__builtin_inff(), bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < N && !((taken >> j) & 1u) && key_better(key[j], e, bk, bi)) {
        bk = key[j];
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (key_better(ok, oi, bk, bi)) { bk = ok; bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) { kept_v = bv; kept_i = bi; }
  }
  // softmax over the K kept logits, shifted by their largest
  float m = kept_v;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float p = lane < K ? expf(kept_v - m) : 0.0f;
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
  // Shapes measured on MI355X: few logits in all (a decode batch, a narrow
  // router) go to the LDS-ring kernel, one logit per thread; otherwise wide
  // routers over many tokens use 64x32 blocks with 4x2 logits per thread,
  // mid-sized ones 32x32 with 2x2 (both loading two chunks ahead), and the
  // rest 64x8 with 2x1.
  const int64_t TN = T * static_cast<int64_t>(N);
  const int kc32 = d % 32 == 0;
#define MOE_ROUTER_LAUNCH(BT, BE, MT, ME, KC, PF)                                               \
  {                                                                                             \
    const dim3 grid(static_cast<unsigned>((T + BT - 1) / BT),                                   \
                    static_cast<unsigned>((N + BE - 1) / BE));                                  \
    if (bf16)                                                                                   \
      hipLaunchKernelGGL((router_logits_kernel<BT, BE, MT, ME, KC, true, PF>), grid, dim3(256),\
                         0, s, x, w, bias, logits, T, d, N);                                    \
    else                                                                                        \
      hipLaunchKernelGGL((router_logits_kernel<BT, BE, MT, ME, KC, false, PF>), grid,          \
                         dim3(256), 0, s, x, w, bias, logits, T, d, N);                         \
  }
  if (bf16 && d % 64 == 0 && TN < (int64_t(1) << 17)) {
    const dim3 grid(static_cast<unsigned>((T + ring::BT - 1) / ring::BT),
                    static_cast<unsigned>((N + ring::BE - 1) / ring::BE));
    hipLaunchKernelGGL((router_logits_ring_kernel<12>), grid, dim3(ring::NT), 0, s,
                       static_cast<const uint16_t *>(x), w, bias, logits, T, d, N);
    return hipGetLastError();
  }
  if (N >= 64 && TN >= (int64_t(1) << 19)) {
    if (kc32) MOE_ROUTER_LAUNCH(64, 32, 4, 2, 32, 2) else MOE_ROUTER_LAUNCH(64, 32, 4, 2, 16, 2)
  } else if (N >= 32 && TN >= (int64_t(1) << 17)) {
    if (kc32) MOE_ROUTER_LAUNCH(32, 32, 2, 2, 32, 2) else MOE_ROUTER_LAUNCH(32, 32, 2, 2, 16, 2)
  } else {
    if (kc32) MOE_ROUTER_LAUNCH(64, 8, 2, 1, 32, 1) else MOE_ROUTER_LAUNCH(64, 8, 2, 1, 16, 1)
  }
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

hipError_t launch_topk_gates(const float *logits, const float *sel_bias, int64_t T, int N, int K,
                             int32_t *idx, float *gates, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4)), block(256);
  const int J = (N + 63) / 64;
  if (J <= 1) {
    hipLaunchKernelGGL((topk_gates_kernel<1>), grid, block, 0, s, logits, sel_bias, T, N, K, idx, gates);
  } else if (J <= 2) {
    hipLaunchKernelGGL((topk_gates_kernel<2>), grid, block, 0, s, logits, sel_bias, T, N, K, idx, gates);
  } else if (J <= 4) {
    hipLaunchKernelGGL((topk_gates_kernel<4>), grid, block, 0, s, logits, sel_bias, T, N, K, idx, gates);
  } else if (J <= 8) {
    hipLaunchKernelGGL((topk_gates_kernel<8>), grid, block, 0, s, logits, sel_bias, T, N, K, idx, gates);
  } else if (J <= 16) {
    hipLaunchKernelGGL((topk_gates_kernel<16>), grid, block, 0, s, logits, sel_bias, T, N, K, idx, gates);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
