// Router scores, top-K selection and renormalised gates.
//
// Router: one score per expert from a bias-free linear map of the token
// ("Sparse MoE Top-Kルーティング" page, section ルーティングの仕組み; the
// DeepSeekMoE explainer page, gate equation s = softmax(W_r x)), plus an
// optional per-expert bias that is part of the logit.
//
// Fixed float32 order: for every (t, e) one fused multiply-add chain over k
// ascending from +0, then the bias with one rounding.  Every kernel below
// keeps each logit in one accumulator that sees its terms in that order (a
// thread's register, or one output of a float32 matrix-core chain), so no
// reduction tree is involved and the bits do not depend on the launch shape.
//
// Top-K: one wave per token, N logits spread over the lanes' registers, K
// rounds of a wave-wide arg-max on the key (logit desc, expert id asc), packed
// into one ordered 64-bit integer.  Gates
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
// their time is the chain itself: one dependent float32 multiply-add costs
// about 5 cycles on MI355X whatever else the wave issues in between, which is
// 16 us for a 7168-long chain.  Here one logit is one lane's chain: a wave
// owns 64 tokens (one per lane) and one expert, a workgroup E experts of the
// same 64 tokens.  The expert's W row is the same for every lane, so it comes
// through the scalar cache into SGPRs (s_load, read as a v_fmac operand) and
// never touches LDS or vector registers; only x goes through LDS.  x (bf16,
// as stored) streams in 64-wide k-chunks through a ring of S stages filled by
// global-to-LDS copies S-1 chunks ahead (a copy instruction moves 8 rows of
// 128 bytes; piece c of row r sits at c ^ ((r >> 1) & 7), so the 64 rows read
// by one instruction spread over the banks).  Each stage also takes one copy
// of the wave's W chunk into a landing slot that nothing reads: it brings the
// row into L2 ahead of the scalar loads, which would otherwise wait on HBM.
// A chunk is consumed in two halves of 32 k; the x fragment and the 32 W
// values of the next half are requested before the current half's chain, so
// the wait for them (LDS reads and scalar loads share one counter, and scalar
// loads return out of order, so only a full wait is exact) falls one half
// later.
namespace ring {
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// One wave-wide copy of 64 x 16 bytes into the LDS block at byte address m0.
__device__ __forceinline__ void dma16(const void *src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// Leaves at most N copies in flight, drains the LDS queue and joins the
// workgroup.  Written as the waitcnt builtin (encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 = 7 for "no wait", lgkmcnt 11:8 = 0) so that the
// compiler's own wait insertion knows every earlier LDS read has returned and
// does not hold later multiplies on reads issued after this point.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
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

// wait_and_barrier<n * LPS> for a run-time n in [0, MAXN]; n = 0 is the
// unconditional last case, so every path waits (the compiler then knows the
// LDS and scalar-load counter is clear after it).
template <int LPS, int MAXN>
__device__ __forceinline__ void wait_upto(int n) {
  if constexpr (MAXN <= 0) {
    wait_and_barrier<0>();
  } else {
    if (n >= MAXN) {
      wait_and_barrier<MAXN * LPS>();
      return;
    }
    wait_upto<LPS, MAXN - 1>(n);
  }
}

// LDS and scalar loads issued so far have returned.
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
}  // namespace ring

namespace swv {
constexpr int BT = 64, KC = 64, XS = BT * KC * 2;   // tokens per tile, k per chunk, x bytes per stage
}

template <int E, int S>
__global__ __launch_bounds__(64 * E) void router_logits_sw_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int N) {
  using namespace swv;
  static_assert(E == 1 || E == 2 || E == 4, "experts per workgroup");
  constexpr int XC = 8 / E;                  // x copies per wave per stage
  constexpr int STAGE = XS + E * 1024;       // x tile + one landing slot per wave
  constexpr int LPS = XC + 1;                // copies per wave per stage
  static_assert(S >= 4 && (S - 2) * LPS <= 63, "vmcnt range");
  static_assert(S * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[S * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e_out = static_cast<int>(blockIdx.y) * E + wave;
  const int e = uniform(min(e_out, N - 1));  // past N: a duplicate chain, not stored
  const uint32_t ring0 = uniform(static_cast<int>(ring::lds_addr(s_ring)));

  // copy j of this wave moves x rows 8 (wave XC + j) .. +7 of every chunk
  const uint16_t *x_src[XC];
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int r = 8 * (wave * XC + j) + (lane >> 3);
    int64_t xt = t0 + r;
    if (xt >= T) xt = T - 1;
    x_src[j] = x + xt * d + ((lane & 7) ^ ((r >> 1) & 7)) * 8;
  }
  const float *w_row = w + static_cast<int64_t>(e) * d;
  const float *w_touch = w_row + (lane & 15) * 4;   // the chunk's 256 bytes (each 4 times)
  // the constant address space lets uniform loads of W become scalar loads
  using cfloat = __attribute__((address_space(4))) const float;
  cfloat *w_sc = (cfloat *)w_row;
  auto issue = [&](int c, int st) {
    const uint32_t base = ring0 + static_cast<uint32_t>(st) * STAGE;
#pragma unroll
    for (int j = 0; j < XC; ++j) ring::dma16(x_src[j] + c * KC, base + (wave * XC + j) * 1024);
    ring::dma16(w_touch + c * KC, base + XS + wave * 1024);
  };

  const int nch = d / KC;
  const uint8_t *xrow = s_ring + lane * (KC * 2);
  const int sw = (lane >> 1) & 7;
  // operands of one half chunk: 32 bf16 of the lane's token, 32 W values
  uint4 xa[4], xb[4];
  float wa[32], wb[32];
  auto fetch = [&](int c, int h, uint4 (&xq)[4], float (&wv)[32]) {
    const uint8_t *st = xrow + (c % S) * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xq[i] = *reinterpret_cast<const uint4 *>(st + (((4 * h + i) ^ sw) << 4));
    cfloat *wp = w_sc + c * KC + h * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) wv[i] = wp[i];
  };
  float acc = 0.0f;
  auto chain = [&](const uint4 (&xq)[4], const float (&wv)[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = xq[i];
      acc = __builtin_fmaf(__uint_as_float(q.x << 16), wv[8 * i + 0], acc);
      acc = __builtin_fmaf(__uint_as_float(q.x & 0xFFFF0000u), wv[8 * i + 1], acc);
      acc = __builtin_fmaf(__uint_as_float(q.y << 16), wv[8 * i + 2], acc);
      acc = __builtin_fmaf(__uint_as_float(q.y & 0xFFFF0000u), wv[8 * i + 3], acc);
      acc = __builtin_fmaf(__uint_as_float(q.z << 16), wv[8 * i + 4], acc);
      acc = __builtin_fmaf(__uint_as_float(q.z & 0xFFFF0000u), wv[8 * i + 5], acc);
      acc = __builtin_fmaf(__uint_as_float(q.w << 16), wv[8 * i + 6], acc);
      acc = __builtin_fmaf(__uint_as_float(q.w & 0xFFFF0000u), wv[8 * i + 7], acc);
    }
    // keeps the chain ahead of the waits and copies that follow it
    asm volatile("" : "+v"(acc));
  };

  const int pro = min(S - 1, nch);
  for (int c = 0; c < pro; ++c) issue(c, c);
  ring::wait_upto<LPS, S - 2>(min(S - 2, nch - 1));   // chunk 0 has landed
  fetch(0, 0, xa, wa);
  for (int c = 0; c < nch; ++c) {
    // first half of chunk c while its second half is requested
    ring::wait_lgkm();
    __builtin_amdgcn_sched_barrier(0);
    fetch(c, 1, xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    chain(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    // second half while the next chunk's first half is requested; chunk c+1
    // must have landed first, and its arrival frees the stage of chunk c-1
    // for chunk c+S-1.  After the last chunk the request repeats it, which
    // keeps the register roles fixed (a conditional request would add copies
    // and waits).
    ring::wait_lgkm();
    if (c + 1 < nch) {
      ring::wait_upto<LPS, S - 3>(min(S - 3, nch - c - 2));
      if (c + S - 1 < nch) issue(c + S - 1, (c + S - 1) % S);
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch(min(c + 1, nch - 1), 0, xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    chain(xb, wb);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int64_t t = t0 + lane;
  if (t < T && e_out < N) {
    float v = acc;
    if (bias) v = v + bias[e_out];
    logits[t * N + e_out] = v;
  }
}

// Logits on the float32 matrix cores.  v_mfma_f32_16x16x4_f32 adds to each of
// its 16 x 16 outputs the four products of one k-quad one at a time in
// ascending k, each with one rounding: on MI355X its results equal, bit for
// bit, four fused multiply-adds in that order (checked against a host fmaf
// chain on normal, subnormal and signed-zero operands).  A chain of these
// instructions over ascending k-quads is therefore the fixed order itself.
//
// Lane l of the instruction supplies A[l % 16][k0 + l / 16] (a token's x) and
// B[k0 + l / 16][l % 16] (an expert's W row) and receives outputs
// (4 * (l / 16) + r, l % 16), r = 0..3.  A workgroup of AT x AE waves covers
// BT = 16 AT TT tokens x BE = 16 AE TE experts; each wave owns TT x TE tiles.
// x (bf16, as stored) and W (float32) stream through an LDS ring of S stages
// of 64 k each, filled by 1 KB global-to-LDS copies issued S-1 stages ahead:
// a copy moves 8 token rows of 128 bytes or 4 expert rows of 256 bytes.  The
// 16-byte piece p of row r sits at p ^ (r & 7), so the 16 rows that one
// instruction's lanes read spread over the banks.
namespace rmf {
constexpr int KC = 64;
constexpr int XROW = KC * 2;     // bytes of a token's stage row
constexpr int WROW = KC * 4;     // bytes of an expert's stage row
}  // namespace rmf

// Scheduling pattern for one stage: each multiply followed by PER of the next
// stage's LDS reads, so that the reads are in flight while the dependent
// multiplies of a tile hold the wave's issue.
template <int I, int NM, int NR, int PER>
__device__ __forceinline__ void interleave_reads() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
    constexpr int r = NR - I * PER < PER ? NR - I * PER : PER;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);   // LDS reads
    interleave_reads<I + 1, NM, NR, PER>();
  }
}

template <int AT, int AE, int TT, int TE, int S>
__global__ __launch_bounds__(64 * AT * AE) void router_logits_mfma_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int N) {
  using namespace rmf;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int NWAVE = AT * AE;
  constexpr int BT = 16 * AT * TT, BE = 16 * AE * TE;
  constexpr int XB = BT * XROW, WB = BE * WROW, STAGE = XB + WB;
  constexpr int NX = XB / 1024, NW = WB / 1024;
  constexpr int CPW = (NX + NW) / NWAVE;      // copies per wave per stage
  static_assert(CPW * NWAVE == NX + NW, "copies split evenly over the waves");
  static_assert((S - 2) * CPW <= 63, "vmcnt range");
  static_assert(S >= 4, "one stage read ahead of the multiply, two in flight");
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[S * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e0 = blockIdx.y * BE;
  const uint32_t ring0 = uniform(static_cast<int>(ring::lds_addr(s_ring)));

  // this wave's copies: source row pointers (lane's piece, swizzled), byte
  // step per stage and LDS destination within a stage
  const uint8_t *src[CPW];
  int step[CPW], dst[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int c = wave * CPW + q;
    if (c < NX) {
      const int r = 8 * c + (lane >> 3);
      const int64_t t = min(t0 + r, T - 1);
      src[q] = reinterpret_cast<const uint8_t *>(x + t * d + (((lane & 7) ^ (r & 7)) << 3));
      step[q] = XROW;
      dst[q] = c * 1024;
    } else {
      const int r = 4 * (c - NX) + (lane >> 4);
      const int e = min(e0 + r, N - 1);
      src[q] = reinterpret_cast<const uint8_t *>(w + static_cast<int64_t>(e) * d + (((lane & 15) ^ (r & 7)) << 2));
      step[q] = WROW;
      dst[q] = XB + (c - NX) * 1024;
    }
  }
  auto issue = [&](int ch, int slot) {
    const uint32_t base = ring0 + static_cast<uint32_t>(slot * STAGE);
#pragma unroll
    for (int q = 0; q < CPW; ++q)
      ring::dma16(src[q] + static_cast<int64_t>(ch) * step[q], base + dst[q]);
  };

  // fragment addresses: lane reads row i of each tile at k = 4j + g of the stage
  const int i = lane & 15, g = lane >> 4, i7 = i & 7;
  const int wt = wave % AT, we = wave / AT;
  const int xrow = wt * TT * 16 + i, wrow = we * TE * 16 + i;
  int xo[8], wo[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    xo[q] = xrow * XROW + ((q ^ i7) << 4) + 2 * g;
    wo[q] = XB + wrow * WROW + ((q ^ i7) << 4) + 4 * g;
  }

  f32x4 acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // a stage's fragments are read into registers one stage ahead, while the
  // matrix cores work through the previous stage; x stays as its 16 raw bits
  // until the multiply, so nothing waits on the reads in flight
  constexpr int NJ = KC / 4;
  uint32_t fa0[NJ][TT], fa1[NJ][TT];
  float fb0[NJ][TE], fb1[NJ][TE];
  auto read_frags = [&](int c, uint32_t (&fa)[NJ][TT], float (&fb)[NJ][TE]) {
    const uint8_t *sb = s_ring + (c % S) * STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        fa[j][a] = *reinterpret_cast<const uint16_t *>(sb + xo[j >> 1] + (j & 1) * 8 + a * 16 * XROW);
      }
#pragma unroll
      for (int b = 0; b < TE; ++b)
        fb[j][b] = *reinterpret_cast<const float *>(sb + wo[j & 7] + ((j & 8) << 4) + b * 16 * WROW);
    }
  };
  auto mfmas = [&](const uint32_t (&fa)[NJ][TT], const float (&fb)[NJ][TE]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        const float xa = __uint_as_float(fa[j][a] << 16);   // bf16 -> float32, exact
#pragma unroll
        for (int b = 0; b < TE; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, fb[j][b], acc[a][b], 0, 0, 0);
      }
  };

  const int nch = d / KC;
  const int pro = min(S - 1, nch);
  for (int c = 0; c < pro; ++c) issue(c, c);
  // stage 0 landed; stages 1 .. pro-1 may stay in flight
  if (pro - 1 == S - 2) ring::wait_and_barrier<(S - 2) * CPW>();
  else ring::wait_chunks<CPW, S - 3>(pro - 1);
  read_frags(0, fa0, fb0);
  // step c: wait for stage c+1, refill the slot of stage c-1 (its fragments
  // were consumed in step c-1), read stage c+1, multiply stage c
  auto advance = [&](int c, const uint32_t (&fa)[NJ][TT], const float (&fb)[NJ][TE],
                     uint32_t (&na)[NJ][TT], float (&nb)[NJ][TE]) {
    if (c + 1 < nch) {
      const int later = min(S - 3, nch - 2 - c);   // stages c+2 .. may stay in flight
      if (later == S - 3) ring::wait_and_barrier<(S - 3) * CPW>();
      else ring::wait_chunks<CPW, S - 4>(later);
      if (c + S - 1 < nch) issue(c + S - 1, (c + S - 1) % S);
    } else {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every path enters drained
    }
    // unconditional, so the next buffer is always freshly loaded (no merge of
    // old and new values, which would make the compiler copy -- and wait on --
    // the reads in flight); after the last stage it re-reads a landed slot
    // and the values go unused
    __builtin_amdgcn_sched_barrier(0);
    read_frags(c + 1, na, nb);
    mfmas(fa, fb);
    // reads per stage: 16 per token tile (16-bit) and 8 per expert tile (the
    // compiler pairs the float32 reads of k-quads j and j + 8)
    constexpr int NM = NJ * TT * TE, NR = NJ * TT + NJ / 2 * TE;
    interleave_reads<0, NM, NR, (NR + NM - 1) / NM>();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int c = 0; c < nch; c += 2) {
    advance(c, fa0, fb0, fa1, fb1);
    if (c + 1 >= nch) break;
    advance(c + 1, fa1, fb1, fa0, fb0);
  }
#pragma unroll
  for (int b = 0; b < TE; ++b) {
    const int e = e0 + wrow + b * 16;
    if (e >= N) continue;
    const float be = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wt * TT * 16 + a * 16 + 4 * g + r;
        if (t >= T) continue;
        float v = acc[a][b][r];
        if (bias) v = v + be;
        logits[t * N + e] = v;
      }
  }
}

// Key order: a beats b iff a.v > b.v, or equal values and a.i < b.i.  As one
// 64-bit integer whose unsigned order is that order: the float's bits mapped
// to an order-preserving unsigned value (-0 taken as +0, so that equal values
// tie as they compare), above the complement of the expert id, so that the
// lower id wins a tie.  0 is below every key (an entry already taken or past
// N); -inf maps above it.
__device__ __forceinline__ uint64_t pack_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~e);
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
  float v[J];
  uint64_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < N ? row[e] : 0.0f;
    // selection key: the logit, or (selection-only bias) fl32(logit + bias)
    key[j] = e < N ? pack_key(sel_bias ? v[j] + sel_bias[e] : v[j], e) : 0ull;
  }
  float kept_v = -__builtin_inff();   // lane k keeps slot k's (unbiased) logit
  int kept_i = 0;
  for (int k = 0; k < K; ++k) {
    // the lane's best remaining key and its logit, then the wave's best
    uint64_t best = 0ull;
    float bv = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (key[j] > best) {
        best = key[j];
        bv = v[j];
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    const int bi = static_cast<int>(~static_cast<uint32_t>(best));
    bv = __shfl(bv, bi & 63);          // the owning lane's best is the winner
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (bi == lane + 64 * j) key[j] = 0ull;   // taken
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
  // Shapes measured on MI355X.  bf16 tokens with d a multiple of 64: few
  // 16 x 16 output tiles in all (a decode batch, a narrow router) go to the
  // one-logit-per-lane kernel with W in scalar registers, the rest to the
  // matrix cores.
  // float32 tokens and other d use the register-tiled kernel: 64x32 blocks
  // with 4x2 logits per thread for wide routers over many tokens, 32x32 with
  // 2x2 for mid-sized ones (both loading two chunks ahead), 64x8 with 2x1
  // otherwise.
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
  if (bf16 && d % 64 == 0) {
    const int64_t tiles = ((T + 15) / 16) * ((N + 15) / 16);
    if (tiles <= 512) {
      // few 16 x 16 output tiles: a matrix-core chain per tile would be bound
      // by the latency of its dependent multiplies, so one logit per lane
      const unsigned tb = static_cast<unsigned>((T + swv::BT - 1) / swv::BT);
      const uint16_t *xb = static_cast<const uint16_t *>(x);
      if (N == 1)
        hipLaunchKernelGGL((router_logits_sw_kernel<1, 8>), dim3(tb, 1), dim3(64), 0, s, xb, w,
                           bias, logits, T, d, N);
      else if (N == 2)
        hipLaunchKernelGGL((router_logits_sw_kernel<2, 8>), dim3(tb, 1), dim3(128), 0, s, xb, w,
                           bias, logits, T, d, N);
      else
        hipLaunchKernelGGL((router_logits_sw_kernel<4, 8>),
                           dim3(tb, static_cast<unsigned>((N + 3) / 4)), dim3(256), 0, s, xb, w,
                           bias, logits, T, d, N);
      return hipGetLastError();
    }
#define MOE_ROUTER_MFMA(AT, AE, TT, TE, S)                                                      \
  {                                                                                             \
    constexpr int BT = 16 * AT * TT, BE = 16 * AE * TE;                                         \
    const dim3 grid(static_cast<unsigned>((T + BT - 1) / BT),                                   \
                    static_cast<unsigned>((N + BE - 1) / BE));                                  \
    hipLaunchKernelGGL((router_logits_mfma_kernel<AT, AE, TT, TE, S>), grid, dim3(64 * AT * AE),\
                       0, s, static_cast<const uint16_t *>(x), w, bias, logits, T, d, N);       \
  }
    // measured on MI355X: 64 x 64 per workgroup of 8 waves (two per SIMD, one
    // token tile x two expert tiles each) for many tiles, 32 x 32 of 4 waves
    // in between, 64 tokens x 16 experts for narrow routers
    if (N <= 16) MOE_ROUTER_MFMA(4, 1, 1, 1, 8)
    else if (tiles <= 2048) MOE_ROUTER_MFMA(2, 2, 1, 1, 8)
    else MOE_ROUTER_MFMA(4, 2, 1, 2, 4)
#undef MOE_ROUTER_MFMA
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
