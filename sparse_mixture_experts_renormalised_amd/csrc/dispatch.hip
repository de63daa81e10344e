// Dispatch as an on-device permutation of (token, slot) assignments.
//
// On one GPU the exchange that sends each token to its experts and back
// ("エキスパート並列（Expert Parallelism）" page, section 推論フロー) becomes a
// stable permutation into per-expert row slices.  An expert keeps its first C
// tokens in token order and drops the rest ("Sparse MoE Top-Kルーティング" page,
// section 解決策2: エキスパートキャパシティファクター).
//
// Three passes, no floating point and no order-dependent atomics:
//   1. per 64-token chunk (one wave), a 64-bit lane mask per expert marks the
//      chunk's tokens that chose it (LDS atomic OR is order-independent);
//      the masks and their popcounts (chunk histogram) go to the workspace;
//   2. one workgroup scans the histogram over chunks per expert (base rank of
//      every chunk), clips the totals at C, scans the clipped counts into
//      offsets and sums the drops;
//   3. per chunk, the rank of (t, k) in its expert is the chunk base plus the
//      popcount of the mask bits below lane t; kept iff rank < C.
// A token never picks one expert twice, so each mask bit is set at most once.
// Small problems run the three passes in one workgroup (dispatch_fused_kernel).
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kChunk = 64;          // tokens per chunk (one per lane)
constexpr int kChunksPerBlock = 4;  // one wave per chunk

__global__ __launch_bounds__(256) void dispatch_masks_kernel(const int32_t *__restrict__ idx,
                                                             int64_t T, int K, int N,
                                                             uint64_t *__restrict__ masks,
                                                             int32_t *__restrict__ hist) {
  extern __shared__ uint64_t s_mask[];   // [kChunksPerBlock][N]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n_chunks = (T + kChunk - 1) / kChunk;
  for (int i = threadIdx.x; i < kChunksPerBlock * N; i += blockDim.x) s_mask[i] = 0;
  __syncthreads();
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + wave;
  uint64_t *my = s_mask + wave * N;
  if (c < n_chunks) {
    const int64_t t = c * kChunk + lane;
    if (t < T) {
      for (int k = 0; k < K; ++k) {
        const int e = idx[t * K + k];
        atomicOr(reinterpret_cast<unsigned long long *>(&my[e]), 1ull << lane);
      }
    }
  }
  __syncthreads();
  if (c < n_chunks) {
    for (int e = lane; e < N; e += kWave) {
      const uint64_t m = my[e];
      masks[c * N + e] = m;
      hist[c * N + e] = __popcll(m);
    }
  }
}

// Single workgroup of 1024 threads.  Expert x's chunk counts are summed by a
// segment of P adjacent lanes of one wave (P = 1024 / N rounded down to a
// power of two, at most 64): lane j of the segment takes the contiguous
// chunks j L .. (j+1) L - 1, L = ceil(n_chunks / P), and adds them with eight
// loads in flight; the segment scans its P partial sums with shuffles, and
// each lane then writes the base ranks of its own chunks.  The loop waits for
// one memory latency per eight chunks of a lane instead of per eight chunks of
// the expert.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t *__restrict__ hist, int64_t n_chunks, int N, int64_t capacity,
    int32_t *__restrict__ base, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ n_dropped) {
  __shared__ int32_t s_cnt[kMaxRouted];
  __shared__ int32_t s_drop[kMaxRouted];
  __shared__ int32_t s_wave[16];
  int P = kWave;
  while (P > 1 && P * N > static_cast<int>(blockDim.x)) P >>= 1;
  {
    const int j = threadIdx.x & (P - 1);
    const int x = threadIdx.x / P;   // expert of this lane's segment (idle if >= N)
    const int64_t L = (n_chunks + P - 1) / P;
    const int64_t c_beg = min(n_chunks, j * L), c_end = min(n_chunks, c_beg + L);
    int32_t part = 0;
    if (x < N) {
      for (int64_t c0 = c_beg; c0 < c_end; c0 += 8) {
        int32_t hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = c0 + i < c_end ? hist[(c0 + i) * N + x] : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) part += hv[i];
      }
    }
    // inclusive scan of the partial sums within the segment (segments are
    // aligned, so lane - off stays inside it whenever j >= off)
    int32_t incl = part;
    for (int off = 1; off < P; off <<= 1) {
      const int32_t o = __shfl_up(incl, off);
      if (j >= off) incl += o;
    }
    const int32_t total = __shfl(incl, (threadIdx.x & (kWave - 1) & ~(P - 1)) + P - 1);
    if (x < N) {
      int32_t run = incl - part;   // base rank of chunk c_beg
      for (int64_t c0 = c_beg; c0 < c_end; c0 += 8) {
        int32_t hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = c0 + i < c_end ? hist[(c0 + i) * N + x] : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (c0 + i < c_end) base[(c0 + i) * N + x] = run;
          run += hv[i];
        }
      }
      if (j == 0) {
        const int32_t kept =
            (capacity >= 0 && total > capacity) ? static_cast<int32_t>(capacity) : total;
        counts[x] = kept;
        s_cnt[x] = kept;
        s_drop[x] = total - kept;
      }
    }
  }
  __syncthreads();
  // exclusive scan of s_cnt over N <= 1024 entries: one entry per thread
  const int e = threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t v = e < N ? s_cnt[e] : 0;
  int32_t dr = e < N ? s_drop[e] : 0;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dr += __shfl_xor(dr, off);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int32_t wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += s_wave[w];
  if (e < N) offsets[e] = wave_base + incl - v;
  if (e == N - 1) offsets[N] = wave_base + incl;
  __syncthreads();
  if (lane == 0) s_wave[wave] = dr;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t tot = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += s_wave[w];
    *n_dropped = tot;
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t *__restrict__ idx, int64_t T, int K, int N, int64_t capacity,
    const uint64_t *__restrict__ masks, const int32_t *__restrict__ base,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ row_token,
    int32_t *__restrict__ slot_row) {
  const int lane = threadIdx.x & 63;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kChunksPerBlock + (threadIdx.x >> 6);
  const int64_t t = c * kChunk + lane;
  if (t >= T) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // eight slots at a time: their expert ids, then the loads that depend on
  // them, then the stores, so a token waits for two memory latencies per eight
  // slots rather than two per slot
  for (int k0 = 0; k0 < K; k0 += 8) {
    int ev[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ev[i] = k0 + i < K ? idx[t * K + k0 + i] : 0;
    int32_t bv[8], ov[8];
    uint64_t mv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (k0 + i < K) {
        bv[i] = base[c * N + ev[i]];
        mv[i] = masks[c * N + ev[i]];
        ov[i] = offsets[ev[i]];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (k0 + i >= K) break;
      const int64_t rank = bv[i] + __popcll(mv[i] & below);
      int32_t r = -1;
      if (capacity < 0 || rank < capacity) {
        r = ov[i] + static_cast<int32_t>(rank);
        row_token[r] = static_cast<int32_t>(t);
      }
      slot_row[t * K + k0 + i] = r;
    }
  }
}

// The three passes above in one workgroup of 1024 threads, for problems whose
// chunk masks and chunk base ranks fit in LDS (n_chunks * N small): the
// launches and their gaps would otherwise dominate a decode batch.  Same
// arithmetic, so the same outputs: wave w builds the masks of chunks
// w, w+16, ..; thread e scans expert e over the chunks; the scan of the
// clipped counts and the drop total are those of dispatch_scan_kernel; the
// ranks are those of dispatch_scatter_kernel.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;

__global__ __launch_bounds__(kFusedThreads) void dispatch_fused_kernel(
    const int32_t *__restrict__ idx, int64_t T, int K, int N, int64_t capacity,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ row_token,
    int32_t *__restrict__ slot_row, int32_t *__restrict__ n_dropped) {
  extern __shared__ uint64_t s_dyn[];
  __shared__ int32_t s_cnt[kMaxRouted];
  __shared__ int32_t s_drop[kMaxRouted];
  __shared__ int32_t s_off[kMaxRouted];
  __shared__ int32_t s_wave[kFusedWaves];
  const int n_chunks = static_cast<int>((T + kChunk - 1) / kChunk);
  uint64_t *s_mask = s_dyn;                                              // [n_chunks][N]
  int32_t *s_base = reinterpret_cast<int32_t *>(s_dyn + static_cast<size_t>(n_chunks) * N);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < n_chunks * N; i += kFusedThreads) s_mask[i] = 0;
  __syncthreads();
  // pass 1: per chunk, the lane mask of the tokens that chose each expert
  for (int c = wave; c < n_chunks; c += kFusedWaves) {
    const int64_t t = static_cast<int64_t>(c) * kChunk + lane;
    if (t < T)
      for (int k = 0; k < K; ++k)
        atomicOr(reinterpret_cast<unsigned long long *>(&s_mask[c * N + idx[t * K + k]]),
                 1ull << lane);
  }
  __syncthreads();
  // pass 2: base rank of every chunk per expert, clipped totals, drops
  for (int e = tid; e < N; e += kFusedThreads) {
    int32_t run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      s_base[c * N + e] = run;
      run += __popcll(s_mask[c * N + e]);
    }
    const int32_t kept = (capacity >= 0 && run > capacity) ? static_cast<int32_t>(capacity) : run;
    counts[e] = kept;
    s_cnt[e] = kept;
    s_drop[e] = run - kept;
  }
  __syncthreads();
  // exclusive scan of the clipped counts (N <= 1024: one entry per thread)
  {
    const int e = tid;
    const int32_t v = e < N ? s_cnt[e] : 0;
    int32_t dr = e < N ? s_drop[e] : 0;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dr += __shfl_xor(dr, off);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int32_t wave_base = 0;
    for (int w = 0; w < wave; ++w) wave_base += s_wave[w];
    if (e < N) {
      offsets[e] = wave_base + incl - v;
      s_off[e] = wave_base + incl - v;
    }
    if (e == N - 1) offsets[N] = wave_base + incl;
    __syncthreads();
    if (lane == 0) s_wave[wave] = dr;
    __syncthreads();
    if (tid == 0) {
      int32_t tot = 0;
      for (int w = 0; w < kFusedWaves; ++w) tot += s_wave[w];
      *n_dropped = tot;
    }
  }
  // pass 3: rank of (t, k) = chunk base + mask bits below the lane
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = wave; c < n_chunks; c += kFusedWaves) {
    const int64_t t = static_cast<int64_t>(c) * kChunk + lane;
    if (t >= T) continue;
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      const int64_t rank = s_base[c * N + e] + __popcll(s_mask[c * N + e] & below);
      int32_t r = -1;
      if (capacity < 0 || rank < capacity) {
        r = s_off[e] + static_cast<int32_t>(rank);
        row_token[r] = static_cast<int32_t>(t);
      }
      slot_row[t * K + k] = r;
    }
  }
}

// Limits of the fused dispatch: dynamic LDS for the masks and base ranks of
// every chunk, and assignments (measured on MI355X: at 8,192 one workgroup
// beats the three launches, at 32,768 it takes twice as long).
constexpr size_t kFusedMaxLds = 48 * 1024;
constexpr int64_t kFusedMaxAssign = 8192;

// out[r] = x[row_token[r]] for r < *total_rows; one workgroup per row.
template <typename VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const VEC *__restrict__ x,
                                                          const int32_t *__restrict__ row_token,
                                                          const int32_t *__restrict__ total_rows,
                                                          int nvec, VEC *__restrict__ out) {
  const int64_t r = blockIdx.x;
  if (r >= *total_rows) return;
  const int64_t t = row_token[r];
  const VEC *src = x + t * nvec;
  VEC *dst = out + r * nvec;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) dst[i] = src[i];
}

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t dispatch_workspace_bytes(int64_t T, int K, int N) {
  (void)K;
  const int64_t n_chunks = (T + kChunk - 1) / kChunk;
  const size_t cells = static_cast<size_t>(n_chunks) * static_cast<size_t>(N);
  return align256(cells * sizeof(uint64_t)) + 2 * align256(cells * sizeof(int32_t));
}

hipError_t launch_dispatch(const int32_t *idx, int64_t T, int K, int N, int64_t capacity,
                           int32_t *counts, int32_t *offsets, int32_t *row_token,
                           int32_t *slot_row, int32_t *n_dropped, void *ws, hipStream_t s) {
  const int64_t n_chunks = (T + kChunk - 1) / kChunk;
  const size_t cells = static_cast<size_t>(n_chunks) * static_cast<size_t>(N);
  char *p = static_cast<char *>(ws);
  uint64_t *masks = reinterpret_cast<uint64_t *>(p);
  p += align256(cells * sizeof(uint64_t));
  int32_t *hist = reinterpret_cast<int32_t *>(p);
  p += align256(cells * sizeof(int32_t));
  int32_t *base = reinterpret_cast<int32_t *>(p);

  const size_t fused_lds = cells * (sizeof(uint64_t) + sizeof(int32_t));
  if (fused_lds <= kFusedMaxLds && T * K <= kFusedMaxAssign) {
    hipLaunchKernelGGL(dispatch_fused_kernel, dim3(1), dim3(kFusedThreads), fused_lds, s, idx, T,
                       K, N, capacity, counts, offsets, row_token, slot_row, n_dropped);
    return hipGetLastError();
  }
  const unsigned blocks = static_cast<unsigned>((n_chunks + kChunksPerBlock - 1) / kChunksPerBlock);
  if (n_chunks > 0) {
    hipLaunchKernelGGL(dispatch_masks_kernel, dim3(blocks), dim3(256),
                       kChunksPerBlock * N * sizeof(uint64_t), s, idx, T, K, N, masks, hist);
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, hist, n_chunks, N, capacity,
                     base, counts, offsets, n_dropped);
  if (n_chunks > 0) {
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(blocks), dim3(256), 0, s, idx, T, K, N,
                       capacity, masks, base, offsets, row_token, slot_row);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(bool bf16, const void *x, const int32_t *row_token,
                              const int32_t *total_rows, int64_t max_rows, int d, void *out,
                              hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const int row_bytes = d * (bf16 ? 2 : 4);
  const int nvec = row_bytes / 16;
  hipLaunchKernelGGL((gather_rows_kernel<uint4>), dim3(static_cast<unsigned>(max_rows)), dim3(256),
                     0, s, static_cast<const uint4 *>(x), row_token, total_rows, nvec,
                     static_cast<uint4 *>(out));
  return hipGetLastError();
}

}  // namespace moe
