// Grouped expert GEMM: every group (expert) multiplies its own contiguous
// slice of rows by its own weight matrix, with the bias and, for the first
// Linear, the SiLU fused into the epilogue (DeepSeekMoE explainer page,
// section アルゴリズム: expert = Linear(d, d_ff) - SiLU - Linear(d_ff, d)).
//
//   out[r, n] = epi( sum_k A[r, k] * W_g[n, k] + bias_g[n] ),  r in group g
//
// Both operands keep the reduction dimension contiguous (activations row-major
// [rows][K], weights in nn.Linear layout [Nout][K]), so both tiles are loaded
// the same way.
//
// Groups: routed groups take their row ranges from the device-resident
// offsets written by the dispatch (no host round trip); shared-expert groups
// cover all T_sh rows.  Every workgroup rebuilds the prefix sum of m-tiles
// per group in LDS from those offsets, so the launch is sized from a host
// upper bound and the work list lives entirely on the device.
//
// Scheduling: persistent workgroups; the work list is split into eight equal
// contiguous parts, one per XCD (workgroups are dealt to the eight XCDs
// round-robin by id), so the workgroups running together on one XCD share
// weight and activation tiles in that XCD's L2.
//
// Kernels, chosen by operand type and group size (rows per expert):
//   * 256x256 tiles (groups above 128 rows): MFMA v_mfma_f32_32x32x16_bf16
//     with fp32 accumulators, operands copied global -> two swizzled LDS
//     buffers two K-steps ahead with the copies spread among the MFMAs
//     (addressed from wave-uniform SGPR bases when offsets fit in 32 bits),
//     tail tiles of 1..128 rows at half height, or quarter height up to 64
//     rows in the first Linear (run beside the full tiles of their columns
//     while their weight blocks are cached), and a K (or M) split of the last
//     partial round of tiles;
//   * a stream kernel (groups of up to 128 rows, bound by the weight stream):
//     weights and activations copied straight into a ring of LDS stages
//     several chunks ahead, non-temporal for weights read once, units of one
//     or two heights, a K split when a product has too few units to fill
//     the chip (decode), and otherwise a K split of the last round's units;
//   * fp32 operands: a plain LDS-tiled VALU kernel (4x4 register tile).
// The weight tile is the MFMA's first operand, so each lane ends up holding
// four consecutive output features of one row and the epilogues store packed
// bf16 pairs.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxGroups = kMaxRouted + kMaxShared;
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // 16 bytes, register-friendly

struct GemmArgs {
  const int32_t *offsets;
  const void *A;
  const int32_t *a_index;
  const void *A_sh;
  const void *W;
  const void *bias;
  const void *W_sh;
  const void *bias_sh;
  void *C;
  void *C_sh;
  int64_t T_sh;
  int64_t a_sh_stride;
  int n_routed;
  int n_shared;
  int Nout;
  int K;
  // Only groups whose row count lies in [cls_lo, cls_hi] get tiles, so two
  // kernels can split one grouped product by group size.
  int64_t cls_lo;
  int64_t cls_hi;
};

__device__ __forceinline__ int64_t group_rows(const GemmArgs &a, int g) {
  const int64_t rows = g < a.n_routed ? (a.offsets[g + 1] - a.offsets[g]) : a.T_sh;
  return (rows >= a.cls_lo && rows <= a.cls_hi) ? rows : 0;
}

// Block-wide exclusive scan of one int per thread (NT threads, NT % 64 == 0).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *s_tmp, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = s_tmp[w];
    base += (w < wave) ? s : 0;
    tot += s;
  }
  *total = tot;
  return base + incl - v;
}

// m-tile prefix over groups, built in LDS by every workgroup.
template <int NT, int BM>
__device__ int build_tile_prefix(const GemmArgs &a, int *s_pref, int *s_tmp) {
  const int n_groups = a.n_routed + a.n_shared;
  const int per = (n_groups + NT - 1) / NT;
  const int g0 = threadIdx.x * per;
  const int g1 = min(g0 + per, n_groups);
  int local = 0;
  for (int g = g0; g < g1; ++g) local += static_cast<int>((group_rows(a, g) + BM - 1) / BM);
  int total;
  int run = block_excl_scan<NT>(local, s_tmp, &total);
  for (int g = g0; g < g1; ++g) {
    s_pref[g] = run;
    run += static_cast<int>((group_rows(a, g) + BM - 1) / BM);
  }
  if (threadIdx.x == 0) s_pref[n_groups] = total;
  __syncthreads();
  return total;
}

// Prefix over groups of count(g) tiles, built in LDS by every workgroup.
template <int NT, typename F>
__device__ int build_prefix(int n_groups, F count, int *s_pref, int *s_tmp) {
  const int per = (n_groups + NT - 1) / NT;
  const int g0 = threadIdx.x * per;
  const int g1 = min(g0 + per, n_groups);
  int local = 0;
  for (int g = g0; g < g1; ++g) local += count(g);
  int total;
  int run = block_excl_scan<NT>(local, s_tmp, &total);
  for (int g = g0; g < g1; ++g) {
    s_pref[g] = run;
    run += count(g);
  }
  if (threadIdx.x == 0) s_pref[n_groups] = total;
  __syncthreads();
  return total;
}

// Group of m-tile mt: largest g with s_pref[g] <= mt (never an empty group).
__device__ __forceinline__ int find_group(const int *s_pref, int n_groups, int mt) {
  int lo = 0, hi = n_groups;   // invariant: s_pref[lo] <= mt < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T>
struct TileView {
  const T *W;              // group's weights [Nout][K]
  const T *bias;           // group's bias [Nout] or null
  int64_t rows;            // rows of the group
  int64_t row0;            // first row of this tile within the group
  int64_t out_base;        // output row index of the group's row 0
  T *C;                    // output base
  int g;
};

template <typename T>
__device__ __forceinline__ TileView<T> tile_view(const GemmArgs &a, int g, int lm, int BM) {
  TileView<T> v;
  v.g = g;
  v.row0 = static_cast<int64_t>(lm) * BM;
  if (g < a.n_routed) {
    const int64_t o0 = a.offsets[g];
    v.rows = a.offsets[g + 1] - o0;
    v.out_base = o0;
    v.W = static_cast<const T *>(a.W) + static_cast<int64_t>(g) * a.Nout * a.K;
    v.bias = a.bias ? static_cast<const T *>(a.bias) + static_cast<int64_t>(g) * a.Nout : nullptr;
    v.C = static_cast<T *>(a.C);
  } else {
    const int gs = g - a.n_routed;
    v.rows = a.T_sh;
    v.out_base = static_cast<int64_t>(gs) * a.T_sh;
    v.W = static_cast<const T *>(a.W_sh) + static_cast<int64_t>(gs) * a.Nout * a.K;
    v.bias = a.bias_sh ? static_cast<const T *>(a.bias_sh) + static_cast<int64_t>(gs) * a.Nout
                       : nullptr;
    v.C = static_cast<T *>(a.C_sh);
  }
  return v;
}

// Source row pointer of local row r (clamped into the group).
template <typename T>
__device__ __forceinline__ const T *a_row_ptr(const GemmArgs &a, const TileView<T> &v,
                                              int64_t r) {
  if (r >= v.rows) r = v.rows - 1;
  if (v.g < a.n_routed) {
    const int64_t gr = v.out_base + r;
    const int64_t src = a.a_index ? static_cast<int64_t>(a.a_index[gr]) : gr;
    return static_cast<const T *>(a.A) + src * a.K;
  }
  const int gs = v.g - a.n_routed;
  return static_cast<const T *>(a.A_sh) + static_cast<int64_t>(gs) * a.a_sh_stride + r * a.K;
}

// Decode a linear tile index into (m-tile, n-tile), banded by GM m-tiles.
template <int GM>
__device__ __forceinline__ void decode_tile(int L, int total_m, int n_nt, int *mt, int *nt) {
  const int band = L / (GM * n_nt);
  const int first = band * GM;
  const int gm = min(GM, total_m - first);
  const int r = L - band * GM * n_nt;
  *mt = first + r % gm;
  *nt = r / gm;
}

// ---------------------------------------------------------------------------
// Global-to-LDS copies shared by the MFMA kernels.
// ---------------------------------------------------------------------------
namespace dma {
// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// One wave-wide LDS DMA (64 lanes x 16 B into the 1 KB block at LDS byte
// address m0), written as inline assembly so the compiler does not drain
// every load in flight before later LDS reads; the explicit waits cover it.
// The s_nop separates the compiler's write of M0 from the copy that reads it.
__device__ __forceinline__ void dma16(const uint16_t *src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
// The same copy with the non-temporal policy, for data read exactly once (a
// weight block used by a single row block): streaming it past the caches
// raises the sustained read rate from about 6.1 to 7.2 TB/s on MI355X.
__device__ __forceinline__ void dma16_nt(const uint16_t *src, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(m0) : "memory");
}

// The same copy addressed as a wave-uniform 64-bit base in SGPRs plus a 32-bit
// per-lane byte offset (the instruction's SGPR-base form): advancing along K
// then costs one scalar add per base instead of a 64-bit vector add per copy.
__device__ __forceinline__ void dma16s(uint32_t voff, const uint16_t *sbase, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Wait until at most N of this wave's copies are in flight and its LDS reads
// are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace dma

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: 256x256 tiles, four 128x128 wave tiles, two LDS buffers
// of one 64-wide K-step each, filled by global-to-LDS copies two K-steps
// ahead.  Each step's fragments (all four 16-wide slices) are read from LDS
// into registers once; the copies of step kb+2 are spread one per three
// MFMAs over the first three slices of step kb, and the fragment reads of
// step kb+1 over its last slice.
// ---------------------------------------------------------------------------
namespace rs {
constexpr int BM = 256, BN = 256, BK = 64, NT = 256, WTM = 128, WTN = 128;
constexpr int TM = WTM / 32, TN = WTN / 32, NS = BK / 16;
constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;   // 16-byte chunks per thread
constexpr int TILE = (BM + BN) * BK;                    // bf16 elements in LDS

struct Frags {
  bf16x8_t a[NS][TM];
  bf16x8_t b[NS][TN];
};

// chunk kc of tile row r at chunk position kc ^ ((r / 2) % 8) of its 128-byte
// row: with 64 four-byte banks serving 16 lanes of 16 bytes at a time, the
// 16 rows read together (same logical chunk) then cover all banks once.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void read_frags(const uint16_t *tile, Frags &f, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) {
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int row = wm * WTM + mi * 32 + (lane & 31);
      f.a[ks][mi] = *reinterpret_cast<const bf16x8_t *>(tile + row * BK + (swz(row, c) << 3));
    }
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      const int row = wn * WTN + ni * 32 + (lane & 31);
      f.b[ks][ni] =
          *reinterpret_cast<const bf16x8_t *>(tile + BM * BK + row * BK + (swz(row, c) << 3));
    }
  }
}

__device__ __forceinline__ void mfma_all(const Frags &f, f32x16_t (&acc)[TN][TM]) {
#pragma unroll
  for (int ks = 0; ks < NS; ++ks)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][ni], f.a[ks][mi], acc[ni][mi],
                                                              0, 0, 0);
}

// MFMAs number M0 .. M1-1 of a step, in mfma_all's (slice, ni, mi) order.
template <int M0, int M1>
__device__ __forceinline__ void mfma_range(const Frags &f, f32x16_t (&acc)[TN][TM]) {
#pragma unroll
  for (int m = M0; m < M1; ++m) {
    const int ks = m / (TN * TM), ni = (m / TM) % TN, mi = m % TM;
    acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][ni], f.a[ks][mi], acc[ni][mi],
                                                          0, 0, 0);
  }
}

// Instruction order of a step's last slice: two fragment reads of the next
// step before each of its sixteen MFMAs.
__device__ __forceinline__ void schedule_last_slice() {
#pragma unroll
  for (int i = 0; i < NS * (TM + TN) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
  }
}
// Workgroup barrier that also waits for this wave's LDS operations.  As an
// asm statement it orders memory operations but lets MFMAs move across it,
// so a whole K-step stays one scheduling region.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace rs

// Half- and quarter-height tiles: the last m-tile of a group often holds 128
// rows or fewer (an expert of 1,052 rows leaves 28 in its fifth 256-row
// tile).  Such a tile is computed as H x 256 (H = 128 or 64) by all four
// waves (2 x 2 waves of H/2 x 128) instead of leaving waves to multiply
// padding rows: same operand path and swizzle, H/256 of the A rows and MFMAs.
template <int H>
struct Rh {
static constexpr int BM = H, BN = 256, BK = 64, NT = 256, WTM = H / 2, WTN = 128;
static constexpr int TM = WTM / 32, TN = WTN / 32, NS = BK / 16;
static constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
static __device__ __forceinline__ int swz(int r, int c) { return rs::swz(r, c); }

struct Frags {
  bf16x8_t a[NS][TM];
  bf16x8_t b[NS][TN];
};

template <bool NTB>
static __device__ __forceinline__ void gload(u32x4_t (&ra)[A_CH], u32x4_t (&rb)[B_CH],
                                      const uint16_t *const (&a_src)[A_CH],
                                      const uint16_t *const (&b_src)[B_CH], int kb) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4_t *>(a_src[i] + kb * BK);
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(b_src[i] + kb * BK);
    if constexpr (NTB) rb[i] = __builtin_nontemporal_load(p);
    else rb[i] = *p;
  }
}

static __device__ __forceinline__ void lstore(uint16_t *tile, const u32x4_t (&ra)[A_CH],
                                       const u32x4_t (&rb)[B_CH], int tid) {
  const int kc = tid & 7;
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int row = (tid >> 3) + i * (NT / 8);
    *reinterpret_cast<u32x4_t *>(tile + row * BK + (swz(row, kc) << 3)) = ra[i];
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int row = (tid >> 3) + i * (NT / 8);
    *reinterpret_cast<u32x4_t *>(tile + BM * BK + row * BK + (swz(row, kc) << 3)) = rb[i];
  }
}

static __device__ __forceinline__ void read_frags(const uint16_t *tile, Frags &f, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) {
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int row = wm * WTM + mi * 32 + (lane & 31);
      f.a[ks][mi] = *reinterpret_cast<const bf16x8_t *>(tile + row * BK + (swz(row, c) << 3));
    }
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      const int row = wn * WTN + ni * 32 + (lane & 31);
      f.b[ks][ni] =
          *reinterpret_cast<const bf16x8_t *>(tile + BM * BK + row * BK + (swz(row, c) << 3));
    }
  }
}

static __device__ __forceinline__ void mfma_all(const Frags &f, f32x16_t (&acc)[TN][TM]) {
#pragma unroll
  for (int ks = 0; ks < NS; ++ks)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][ni], f.a[ks][mi], acc[ni][mi],
                                                              0, 0, 0);
}

// One step: each global load / LDS write shares a slot with one or two MFMAs
// (two when there are enough: H = 128 has 32 MFMAs for 12 loads), then the
// fragment reads go before the remaining MFMAs, a few per MFMA.
static __device__ __forceinline__ void schedule_step() {
  constexpr int LOADS = A_CH + B_CH, MF = NS * TN * TM, READS = NS * (TM + TN);
  constexpr int PER = MF >= 2 * LOADS ? 2 : 1;
  constexpr int REST = MF - PER * LOADS;
  constexpr int RPM = REST > 0 ? (READS + REST - 1) / REST : READS;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    if constexpr (PER == 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
  }
#pragma unroll
  for (int i = 0; i < REST; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
  }
}

// Accumulators of one H x 256 tile over K-steps k0 .. k0+nk-1, and its
// epilogue (bias, SiLU, bf16 store through the LDS staging rows).  NTB: the
// weight loads take the non-temporal policy (blocks read once).
template <bool NTB = false>
static __device__ __forceinline__ void tile(const GemmArgs &a, const TileView<uint16_t> &v, int n0,
                                            int k0, int nk, uint16_t *s_tile, int tid, int lane,
                                            int wm, int wn, f32x16_t (&acc)[TN][TM]);
template <int EPI>
static __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TN][TM], const GemmArgs &a,
                                                const TileView<uint16_t> &v, int n0,
                                                uint16_t *s_tile, int lane, int wm, int wn,
                                                int tid);
};
// the 128-row tiles, the height of the split and M-split paths
namespace rh {
using T = Rh<128>;
constexpr int BM = T::BM, TM = T::TM, TN = T::TN, WTM = T::WTM;
}  // namespace rh

// Store of ROWS staged output rows of 256 bf16 from LDS (row r at r * 256, its
// 16-byte chunks swizzled by r & 31) by the 256 threads of a workgroup: thread
// t owns chunk t % 32 of rows t / 32 + 8j.  All of a thread's LDS reads are
// issued before its first store, so their latency is paid once and not per
// row; the global addresses step by a fixed row stride.  row_of(j) is the
// tile row (from v.row0) that staged row t / 32 + 8j holds, minus t / 32.
template <int ROWS, typename RowOf>
__device__ __forceinline__ void store_staged_rows(const uint16_t *s_tile, const GemmArgs &a,
                                                  const TileView<uint16_t> &v, int n0,
                                                  int etid, RowOf row_of) {
  constexpr int BN = 256, CH = BN / 8, RPI = 256 / CH, NIT = ROWS / RPI;
  static_assert(ROWS % RPI == 0, "whole sweeps");
  const int c = etid % CH, r0 = etid / CH;
  u32x4_t val[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) {
    const int r = r0 + RPI * j;
    val[j] = *reinterpret_cast<const u32x4_t *>(s_tile + r * BN + ((c ^ (r & 31)) << 3));
  }
  const int n = n0 + c * 8;
  if (n >= a.Nout) return;
  uint16_t *base = v.C + (v.out_base + v.row0 + r0) * a.Nout + n;
  const int64_t lim = v.rows - v.row0 - r0;   // rows of the view from this thread's first
#pragma unroll
  for (int j = 0; j < NIT; ++j) {
    const int lr = row_of(j);
    if (lr < lim) store_nt(base + static_cast<int64_t>(lr) * a.Nout, val[j]);
  }
}

// Epilogue of a 256x256 tile through LDS in two passes of 128 rows (the tile
// buffer holds 128 x 256 bf16): in pass p every wave stores its row blocks
// mi = 2p, 2p+1, so all four waves work in both passes.  Without the SiLU,
// pass 0's staged rows are read back into registers and their global stores
// are issued one per column block of pass 1, under pass 1's arithmetic
// (measured: with the SiLU the held rows spill and cost more than the overlap
// gains, so there each pass stores its own rows).  The barriers only
// order LDS accesses; they wait for no global load or store.
template <int EPI, bool BIAS>
__device__ __forceinline__ void rs_epilogue(const f32x16_t (&acc)[rs::TN][rs::TM],
                                            const GemmArgs &a, const TileView<uint16_t> &v,
                                            int n0, uint16_t *s_tile, int lane, int wm, int wn,
                                            int tid) {
  using namespace rs;
  int el = lane, ewm = wm, ewn = wn, etid = tid;
  asm volatile("" : "+v"(el), "+v"(etid), "+s"(ewm), "+s"(ewn));
  static_assert(TILE >= 128 * BN, "128 C-tile rows must fit");
  static_assert(TN * 4 == 16, "one held row per column block of pass 1");
  constexpr bool HOLD = EPI != kEpiBiasSilu;
  // pass 0's rows, as store_staged_rows lays them out: thread t holds chunk
  // t % 32 of staged rows t / 32 + 8j, tile rows (j / 8) * 128 + t / 32 + 8 (j % 8)
  u32x4_t held[16];
  uint16_t *hbase = nullptr;
  int64_t hlim = 0;
  bool hcol = false;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (HOLD && pass == 1) {
          const int j = ni * 4 + q;
          const int lr = (j >> 3) * 128 + 8 * (j & 7);
          if (hcol && lr < hlim) store_nt(hbase + static_cast<int64_t>(lr) * a.Nout, held[j]);
        }
        const int nl = ewn * WTN + ni * 32 + q * 8 + (el >> 5) * 4;
        const int n = n0 + nl;
        float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (BIAS && n < a.Nout) {
          const uint2 bq = *reinterpret_cast<const uint2 *>(v.bias + n);
          bv[0] = __uint_as_float(bq.x << 16);
          bv[1] = __uint_as_float(bq.x & 0xFFFF0000u);
          bv[2] = __uint_as_float(bq.y << 16);
          bv[3] = __uint_as_float(bq.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int mi = pass * 2 + mm;
          const int ml = ewm * 64 + mm * 32 + (el & 31);   // row within the pass
          float o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            o[j] = acc[ni][mi][q * 4 + j];
            if (BIAS) o[j] += bv[j];
            if (EPI == kEpiBiasSilu) o[j] = silu_fast(o[j]);
          }
          uint2 packed;
          packed.x = pack_bf16x2(o[0], o[1]);
          packed.y = pack_bf16x2(o[2], o[3]);
          const int p = (nl >> 3) ^ (ml & 31);
          *reinterpret_cast<uint2 *>(s_tile + ml * BN + p * 8 + ((nl >> 2) & 1) * 4) = packed;
        }
      }
    }
    rs::lds_barrier();
    // LDS row ml of the pass is tile row (ml/64)*128 + pass*64 + ml%64; the
    // thread's rows t/32 + 8j (t/32 < 8) cross from the first 64 at j = 8
    if (!HOLD) {
      store_staged_rows<128>(s_tile, a, v, n0, etid,
                             [&](int j) { return (j >> 3) * 128 + pass * 64 + 8 * (j & 7); });
    } else if (pass == 0) {
      const int c = etid % 32, r0 = etid / 32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = r0 + 8 * j;
        held[j] = *reinterpret_cast<const u32x4_t *>(s_tile + r * BN + ((c ^ (r & 31)) << 3));
      }
      const int n = n0 + c * 8;
      hcol = n < a.Nout;
      hbase = v.C + (v.out_base + v.row0 + r0) * a.Nout + n;
      hlim = v.rows - v.row0 - r0;
    } else {
      store_staged_rows<128>(s_tile, a, v, n0, etid,
                             [&](int j) { return (j >> 3) * 128 + 64 + 8 * (j & 7); });
    }
    rs::lds_barrier();
  }
}

template <int EPI>
__device__ __forceinline__ void rs_epilogue(const f32x16_t (&acc)[rs::TN][rs::TM],
                                            const GemmArgs &a, const TileView<uint16_t> &v,
                                            int n0, uint16_t *s_tile, int lane, int wm, int wn,
                                            int tid) {
  if (v.bias)
    rs_epilogue<EPI, true>(acc, a, v, n0, s_tile, lane, wm, wn, tid);
  else
    rs_epilogue<EPI, false>(acc, a, v, n0, s_tile, lane, wm, wn, tid);
}

// Splitting the last, partly filled round of tiles along K.  Per XCD the
// tiles form full rounds (one tile per workgroup of that XCD) and a remainder
// of rem tiles; when rem is at most half the XCD's workgroups, each
// remainder tile is cut into P contiguous K ranges computed by P workgroups
// at once.  Each piece stores its float32 accumulators (native register
// layout) in the scratch slot of its workgroup, and rs_fixup_kernel adds the
// pieces of a tile in piece order and runs the usual epilogue.
struct RsSplit {
  float *partial;      // [max_blocks][256 * 256] floats, or null: never split
  int max_blocks;      // grids wider than this do not split
};

struct RsPlan {
  int full, rem, P, kper;
};

// cnt work items of one XCD over its nslots workgroups: full rounds, then a
// remainder of rem items, cut into P K-pieces when rem fills at most half.
__device__ __forceinline__ RsPlan rs_plan(int cnt, int nslots, int nk, bool can_split) {
  RsPlan p;
  p.full = (cnt / nslots) * nslots;
  p.rem = cnt - p.full;
  int P = 1;
  if (can_split && p.rem > 0 && 2 * p.rem <= nslots) P = min(nslots / p.rem, nk / 32);
  if (P < 2) P = 1;
  p.kper = (nk + P - 1) / P;
  p.P = (nk + p.kper - 1) / p.kper;   // no empty pieces
  return p;
}

// The 256-row m-tiles in two lists: tiles of 129..256 rows, and the last
// tiles of groups that end with 1..128 rows (computed at half height).  Each
// XCD takes an equal contiguous share of the full list and every kXcds-th
// tail (in column order).  A tail reads the same weight block as the full
// tiles of its column, so it should run while that block is still cached:
// when the XCD's last, partly filled round has at least as many workgroups
// as the XCD has tails and is not split along K, tail q goes to workgroup q
// in round q*R/H (R rounds, H tails), which spreads the tails over the rounds
// in column order and gives each workgroup at most one; otherwise the tails
// run after the full tiles (a K-split last round is cheapest made of tails).
__device__ __forceinline__ bool rs_half_tail(int64_t rows) {
  const int64_t r = rows % rs::BM;
  return r != 0 && r <= rh::BM;
}

struct RsTiles {
  int total_mf, total_mh, n_nt;   // m-tiles per list, n-tiles
  int begin_f, cnt_f, cnt_h;      // this XCD's full tiles, and its count of tails
  int xcd, nslots, R;             // R = rounds of the XCD's cnt_f + cnt_h items
  bool inter;                     // tails interleaved (else after the full tiles);
                                  // cleared by the caller when the plan splits K
};

__device__ __forceinline__ RsTiles rs_tiles(const GemmArgs &a, int *s_pref_f, int *s_pref_h,
                                            int *s_tmp, int xcd, int nslots) {
  RsTiles t;
  const int n_groups = a.n_routed + a.n_shared;
  t.total_mf = build_prefix<rs::NT>(n_groups, [&](int g) {
    const int64_t rows = group_rows(a, g);
    return static_cast<int>((rows + rs::BM - 1) / rs::BM) - (rs_half_tail(rows) ? 1 : 0);
  }, s_pref_f, s_tmp);
  t.total_mh = build_prefix<rs::NT>(n_groups, [&](int g) {
    return rs_half_tail(group_rows(a, g)) ? 1 : 0;
  }, s_pref_h, s_tmp);
  t.n_nt = (a.Nout + rs::BN - 1) / rs::BN;
  const int tot_f = t.total_mf * t.n_nt, tot_h = t.total_mh * t.n_nt;
  const int part_f = (tot_f + kXcds - 1) / kXcds;
  t.begin_f = xcd * part_f;
  t.cnt_f = max(0, min(tot_f, t.begin_f + part_f) - t.begin_f);
  t.cnt_h = tot_h > xcd ? (tot_h - xcd + kXcds - 1) / kXcds : 0;
  t.xcd = xcd;
  t.nslots = nslots;
  const int L = t.cnt_f + t.cnt_h;
  t.R = L > 0 ? (L + nslots - 1) / nslots : 0;
  const int last = L - (t.R - 1) * nslots;   // items of the last round
  t.inter = t.cnt_h > 0 && t.cnt_h <= last;
  return t;
}

// Whether item i of this XCD's list is a tail (and which: q-th of the XCD).
__device__ __forceinline__ bool rs_is_tail(const RsTiles &t, int i, int *q) {
  if (!t.inter) {
    *q = i - t.cnt_f;
    return i >= t.cnt_f;
  }
  const int w = i % t.nslots;
  *q = w;
  return w < t.cnt_h && i / t.nslots == (w * t.R) / t.cnt_h;
}

// Tails of this XCD before item i (its full tiles before i are i minus that).
__device__ __forceinline__ int rs_tails_before(const RsTiles &t, int i) {
  if (!t.inter) return max(0, i - t.cnt_f);
  int n = 0;
  for (int q = 0; q < t.cnt_h; ++q) n += ((q * t.R) / t.cnt_h) * t.nslots + q < i;
  return n;
}

// Item i of this XCD's list: group, m-tile within the group, n-tile, and
// whether it is a tail (computed at half height).
template <int GM>
__device__ __forceinline__ bool rs_tile_at(const GemmArgs &a, const RsTiles &t,
                                           const int *s_pref_f, const int *s_pref_h, int i,
                                           int *g, int *lm, int *nt) {
  const int n_groups = a.n_routed + a.n_shared;
  int mt, q;
  if (!rs_is_tail(t, i, &q)) {
    decode_tile<GM>(t.begin_f + i - rs_tails_before(t, i), t.total_mf, t.n_nt, &mt, nt);
    *g = find_group(s_pref_f, n_groups, mt);
    *lm = mt - s_pref_f[*g];
    return false;
  }
  decode_tile<GM>(t.xcd + kXcds * q, t.total_mh, t.n_nt, &mt, nt);
  *g = find_group(s_pref_h, n_groups, mt);
  *lm = static_cast<int>((group_rows(a, *g) + rs::BM - 1) / rs::BM) - 1;
  return true;
}

// The k-th tail (want_tail) or full tile of this XCD's items from..end-1.
__device__ __forceinline__ int rs_kth_item(const RsTiles &t, int from, int end, int k,
                                           bool want_tail) {
  for (int i = from; i < end; ++i) {
    int q;
    if (rs_is_tail(t, i, &q) == want_tail && k-- == 0) return i;
  }
  return end - 1;   // not reached: the caller counted the items
}

// Source addresses of this thread's 16-byte chunks of a 256x256 tile, from
// K-step k0 on.  Copy i of wave w fills rows 8*(4i+w) .. +7 of the 512-row
// tile (A rows, then B rows) at LDS bytes (4i+w)*1024 .. +1023: lane l writes
// row 8*(4i+w) + l/8 at 16-byte position l%8, so it fetches the chunk that
// the swizzle puts there, c = (l%8) ^ ((row/2)%8).  With OFF32 the sources
// are 32-bit byte offsets from two wave-uniform bases (A and the group's W),
// which the host allows when every offset fits; otherwise 64-bit pointers.
template <bool OFF32>
struct RsSrc;
template <>
struct RsSrc<false> {
  const uint16_t *a[rs::A_CH];
  const uint16_t *b[rs::B_CH];
};
template <>
struct RsSrc<true> {
  uint32_t a[rs::A_CH];
  uint32_t b[rs::B_CH];
  const uint16_t *abase, *bbase;   // at K-step k0
};

__device__ __forceinline__ const uint16_t *uniform_ptr(const uint16_t *p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const uint16_t *>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <bool OFF32>
__device__ __forceinline__ void rs_src(const GemmArgs &a, const TileView<uint16_t> &v, int n0,
                                       int k0, int tid, RsSrc<OFF32> &src) {
  using namespace rs;
  const int c = (tid & 7) ^ ((tid >> 4) & 7);   // row = tid/8 + 32i, so (row/2)%8 = (tid/16)%8
  if constexpr (OFF32) {
    const uint16_t *ab = v.g < a.n_routed
                             ? static_cast<const uint16_t *>(a.A)
                             : static_cast<const uint16_t *>(a.A_sh) +
                                   static_cast<int64_t>(v.g - a.n_routed) * a.a_sh_stride;
    src.abase = uniform_ptr(ab + static_cast<int64_t>(k0) * BK);
    src.bbase = uniform_ptr(v.W + static_cast<int64_t>(k0) * BK);
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      src.a[i] = static_cast<uint32_t>(
          (a_row_ptr(a, v, v.row0 + (tid >> 3) + i * (NT / 8)) - ab) * 2 + c * 16);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int n = n0 + (tid >> 3) + i * (NT / 8);
      if (n >= a.Nout) n = a.Nout - 1;
      src.b[i] = static_cast<uint32_t>(static_cast<int64_t>(n) * a.K * 2 + c * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      src.a[i] = a_row_ptr(a, v, v.row0 + (tid >> 3) + i * (NT / 8)) + c * 8 + k0 * BK;
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int n = n0 + (tid >> 3) + i * (NT / 8);
      if (n >= a.Nout) n = a.Nout - 1;
      src.b[i] = v.W + static_cast<int64_t>(n) * a.K + c * 8 + k0 * BK;
    }
  }
}

// Copy I of K-step kb into the tile buffer at LDS byte address base.
template <bool OFF32>
__device__ __forceinline__ void rs_copy(const RsSrc<OFF32> &src, int i, int kb, uint32_t base,
                                        int wave) {
  using namespace rs;
  if constexpr (OFF32) {
    if (i < A_CH)
      dma::dma16s(src.a[i], src.abase + kb * BK, base + (4 * i + wave) * 1024);
    else
      dma::dma16s(src.b[i - A_CH], src.bbase + kb * BK, base + (4 * i + wave) * 1024);
  } else {
    if (i < A_CH)
      dma::dma16(src.a[i] + kb * BK, base + (4 * i + wave) * 1024);
    else
      dma::dma16(src.b[i - A_CH] + kb * BK, base + (4 * i + wave) * 1024);
  }
}

// Copies I.. of step kb, one before each group of three MFMAs of the first
// three slices (48 MFMAs for 16 copies); each group is its own scheduling
// region so the copies stay spread out.
template <int I, bool OFF32>
__device__ __forceinline__ void rs_copies_mfmas(const RsSrc<OFF32> &src, int kb, uint32_t base,
                                                int wave, const rs::Frags &f,
                                                f32x16_t (&acc)[rs::TN][rs::TM]) {
  if constexpr (I < rs::A_CH + rs::B_CH) {
    rs_copy(src, I, kb, base, wave);
    rs::mfma_range<3 * I, 3 * I + 3>(f, acc);
    __builtin_amdgcn_sched_barrier(0);
    rs_copies_mfmas<I + 1, OFF32>(src, kb, base, wave, f, acc);
  }
}

// Accumulators of one 256x256 tile over the nk K-steps that src points at.
// s_tile holds two tile buffers; step kb lives in buffer kb % 2.  Returns
// once the last step's MFMAs are issued; the caller passes an LDS barrier
// before reusing the buffers.
template <bool OFF32>
__device__ __forceinline__ void rs_body(const RsSrc<OFF32> &src, int nk, uint16_t *s_tile, int tid,
                                        int lane, int wm, int wn,
                                        f32x16_t (&acc)[rs::TN][rs::TM]) {
  using namespace rs;
  constexpr int NCP = A_CH + B_CH;   // copies per wave per step
  const int wave = uniform(tid >> 6);
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const uint32_t b0 = uniform(static_cast<int>(dma::lds_addr(s_tile)));
  const uint32_t b1 = b0 + TILE * 2;
  Frags f;
#pragma unroll
  for (int i = 0; i < NCP; ++i) rs_copy(src, i, 0, b0, wave);
  if (nk > 1) {
#pragma unroll
    for (int i = 0; i < NCP; ++i) rs_copy(src, i, 1, b1, wave);
    dma::wait_and_barrier<NCP>();           // step 0 landed for every wave
  } else {
    dma::wait_and_barrier<0>();
  }
  read_frags(s_tile, f, wm, wn, lane);
  __builtin_amdgcn_sched_barrier(0);
  // steady state (no branches, so each step is one scheduling region)
  int kb = 0;
  for (; kb + 2 < nk; ++kb) {
    const int cur = kb & 1;
    lds_barrier();                          // every wave has its fragments of step kb
    __builtin_amdgcn_sched_barrier(0);
    rs_copies_mfmas<0, OFF32>(src, kb + 2, cur ? b1 : b0, wave, f, acc);   // step kb+2 into buffer cur
    dma::wait_and_barrier<NCP>();           // step kb+1 landed for every wave
    mfma_range<48, 64>(f, acc);             // last slice of step kb
    read_frags(s_tile + (cur ? 0 : TILE), f, wm, wn, lane);          // step kb+1
    schedule_last_slice();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kb + 1 < nk) {                        // step nk-2: nothing left to copy
    const int cur = kb & 1;
    mfma_all(f, acc);
    dma::wait_and_barrier<0>();
    read_frags(s_tile + (cur ? 0 : TILE), f, wm, wn, lane);
  }
  mfma_all(f, acc);                         // last step
}

// Accumulators of one 256x256 tile over K-steps k0 .. k0+nk-1.
template <bool OFF32>
__device__ __forceinline__ void rs_tile(const GemmArgs &a, const TileView<uint16_t> &v, int n0,
                                        int k0, int nk, uint16_t *s_tile, int tid, int lane,
                                        int wm, int wn, f32x16_t (&acc)[rs::TN][rs::TM]) {
  RsSrc<OFF32> src;
  rs_src<OFF32>(a, v, n0, k0, tid, src);
  rs_body(src, nk, s_tile, tid, lane, wm, wn, acc);
  rs::lds_barrier();
}

template <int H>
template <bool NTB>
__device__ __forceinline__ void Rh<H>::tile(const GemmArgs &a, const TileView<uint16_t> &v, int n0,
                                            int k0, int nk, uint16_t *s_tile, int tid, int lane,
                                            int wm, int wn, f32x16_t (&acc)[TN][TM]) {
  const int kc = tid & 7;
  const uint16_t *a_src[A_CH];
  const uint16_t *b_src[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i)
    a_src[i] = a_row_ptr(a, v, v.row0 + (tid >> 3) + i * (NT / 8)) + kc * 8 + k0 * BK;
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    int n = n0 + (tid >> 3) + i * (NT / 8);
    if (n >= a.Nout) n = a.Nout - 1;
    b_src[i] = v.W + static_cast<int64_t>(n) * a.K + kc * 8 + k0 * BK;
  }
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4_t ra[A_CH], rb[B_CH];
  Frags f;
  gload<NTB>(ra, rb, a_src, b_src, 0);
  lstore(s_tile, ra, rb, tid);
  if (nk > 1) gload<NTB>(ra, rb, a_src, b_src, 1);
  __syncthreads();
  read_frags(s_tile, f, wm, wn, lane);
  __builtin_amdgcn_sched_barrier(0);
  int kb = 0;
  for (; kb + 2 < nk; ++kb) {
    rs::lds_barrier();
    lstore(s_tile, ra, rb, tid);
    gload<NTB>(ra, rb, a_src, b_src, kb + 2);
    mfma_all(f, acc);
    rs::lds_barrier();
    read_frags(s_tile, f, wm, wn, lane);
    schedule_step();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kb + 1 < nk) {
    rs::lds_barrier();
    lstore(s_tile, ra, rb, tid);
    mfma_all(f, acc);
    rs::lds_barrier();
    read_frags(s_tile, f, wm, wn, lane);
  }
  mfma_all(f, acc);
  __syncthreads();
}

template <int H>
template <int EPI>
__device__ __forceinline__ void Rh<H>::epilogue(const f32x16_t (&acc)[TN][TM], const GemmArgs &a,
                                                const TileView<uint16_t> &v, int n0,
                                                uint16_t *s_tile, int lane, int wm, int wn,
                                                int tid) {
  int el = lane, ewm = wm, ewn = wn, etid = tid;
  asm volatile("" : "+v"(el), "+v"(etid), "+s"(ewm), "+s"(ewn));
  constexpr int CH = BN / 8;
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = ewn * WTN + ni * 32 + q * 8 + (el >> 5) * 4;
      const int n = n0 + nl;
      float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (v.bias && n < a.Nout) {
        const uint2 bq = *reinterpret_cast<const uint2 *>(v.bias + n);
        bv[0] = __uint_as_float(bq.x << 16);
        bv[1] = __uint_as_float(bq.x & 0xFFFF0000u);
        bv[2] = __uint_as_float(bq.y << 16);
        bv[3] = __uint_as_float(bq.y & 0xFFFF0000u);
      }
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) {
        const int ml = ewm * WTM + mi * 32 + (el & 31);
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[j] = acc[ni][mi][q * 4 + j] + bv[j];
          if (EPI == kEpiBiasSilu) o[j] = silu_fast(o[j]);
        }
        uint2 packed;
        packed.x = pack_bf16x2(o[0], o[1]);
        packed.y = pack_bf16x2(o[2], o[3]);
        const int p = (nl >> 3) ^ (ml & 31);
        *reinterpret_cast<uint2 *>(s_tile + ml * BN + p * 8 + ((nl >> 2) & 1) * 4) = packed;
      }
    }
  }
  __syncthreads();
  store_staged_rows<BM>(s_tile, a, v, n0, etid, [](int j) { return 8 * j; });
  __syncthreads();
}

// PIECE = false: whole tiles of the full rounds (of every round when there is
// no split).  PIECE = true: the K pieces of the remainder tiles, one per
// workgroup, stored as float32 partial tiles (launched right after, with the
// same grid, so both derive the same plan).
template <int EPI, int GM, bool PIECE, bool OFF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_rs_kernel(GemmArgs a, RsSplit sp) {
  using namespace rs;
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[2 * TILE];
  __shared__ int s_pref_f[kMaxGroups + 1];
  __shared__ int s_pref_h[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int nk = a.K / BK;
  RsTiles t = rs_tiles(a, s_pref_f, s_pref_h, s_tmp, xcd, nslots);
  const RsPlan pl = rs_plan(t.cnt_f + t.cnt_h, nslots, nk,
                            sp.partial != nullptr && static_cast<int>(gridDim.x) <= sp.max_blocks);
  t.inter = t.inter && pl.P <= 1;
  f32x16_t acc[TN][TM];
  if constexpr (PIECE) {
    if (pl.P <= 1 || slot >= pl.rem * pl.P) return;
    int g, lm, nt;
    const bool tail = rs_tile_at<GM>(a, t, s_pref_f, s_pref_h, pl.full + slot / pl.P, &g, &lm, &nt);
    const TileView<uint16_t> v = tile_view<uint16_t>(a, g, lm, BM);
    const int k0 = (slot % pl.P) * pl.kper;
    const int kn = min(nk, k0 + pl.kper) - k0;
    float4 *dst = reinterpret_cast<float4 *>(sp.partial + static_cast<int64_t>(blockIdx.x) * (BM * BN));
    if (tail) {   // a half-height tail: its own register layout
      f32x16_t acch[rh::TN][rh::TM];
      // these pieces run after the full rounds and read their K range of the
      // weight block once, so past the caches (measured: the split round of
      // the Mixtral-shaped second Linear 1.2% shorter)
      rh::T::tile<true>(a, v, nt * BN, k0, kn, s_tile, tid, lane, wm, wn, acch);
#pragma unroll
      for (int i = 0; i < rh::TN; ++i)
#pragma unroll
        for (int j = 0; j < rh::TM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[((i * rh::TM + j) * 4 + q) * NT + tid] =
                make_float4(acch[i][j][4 * q], acch[i][j][4 * q + 1], acch[i][j][4 * q + 2],
                            acch[i][j][4 * q + 3]);
    } else {
      rs_tile<OFF32>(a, v, nt * BN, k0, kn, s_tile, tid, lane, wm, wn, acc);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[((i * TM + j) * 4 + q) * NT + tid] =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
    }
  } else {
    // A last, partly filled round that is not split along K (too few K-steps)
    // is split along M instead when it fits: each full-cost tile of that
    // round becomes two half-height tiles on two workgroups.
    const int cnt = t.cnt_f + t.cnt_h;
    const int rem_f = (cnt - pl.full) - (t.cnt_h - rs_tails_before(t, pl.full));
    const bool msplit = pl.P <= 1 && pl.rem > 0 && 2 * rem_f + (pl.rem - rem_f) <= nslots;
    const int end = pl.P > 1 || msplit ? pl.full : cnt;
    int g, lm, nt;
    for (int i = slot; i < end; i += nslots) {
      if (rs_tile_at<GM>(a, t, s_pref_f, s_pref_h, i, &g, &lm, &nt)) {   // a tail
        const TileView<uint16_t> v = tile_view<uint16_t>(a, g, lm, BM);
        // at quarter height in the first Linear (measured: in the second one
        // the extra path costs the K loop registers and time)
        bool quarter = false;
        if constexpr (EPI == kEpiBiasSilu) {
          quarter = v.rows - v.row0 <= Rh<64>::BM;
          if (quarter) {
            f32x16_t accq[Rh<64>::TN][Rh<64>::TM];
            Rh<64>::tile(a, v, nt * BN, 0, nk, s_tile, tid, lane, wm, wn, accq);
            Rh<64>::epilogue<EPI>(accq, a, v, nt * BN, s_tile, lane, wm, wn, tid);
          }
        }
        if (!quarter) {
          f32x16_t acch[rh::TN][rh::TM];
          rh::T::tile(a, v, nt * BN, 0, nk, s_tile, tid, lane, wm, wn, acch);
          rh::T::epilogue<EPI>(acch, a, v, nt * BN, s_tile, lane, wm, wn, tid);
        }
      } else {
        const TileView<uint16_t> v = tile_view<uint16_t>(a, g, lm, BM);
        rs_tile<OFF32>(a, v, nt * BN, 0, nk, s_tile, tid, lane, wm, wn, acc);
        rs_epilogue<EPI>(acc, a, v, nt * BN, s_tile, lane, wm, wn, tid);
      }
    }
    if (msplit && slot < 2 * rem_f + (pl.rem - rem_f)) {
      int item, upper = 0;
      if (slot < 2 * rem_f) {
        item = rs_kth_item(t, pl.full, cnt, slot / 2, false);
        upper = slot & 1;
      } else {
        item = rs_kth_item(t, pl.full, cnt, slot - 2 * rem_f, true);
      }
      rs_tile_at<GM>(a, t, s_pref_f, s_pref_h, item, &g, &lm, &nt);
      // rows 128*(2*lm + upper) .. +127 of the group: the upper or lower half
      // of a full-cost tile, or a tail tile (upper = 0)
      const TileView<uint16_t> v = tile_view<uint16_t>(a, g, 2 * lm + upper, rh::BM);
      f32x16_t acch[rh::TN][rh::TM];
      rh::T::tile(a, v, nt * BN, 0, nk, s_tile, tid, lane, wm, wn, acch);
      rh::T::epilogue<EPI>(acch, a, v, nt * BN, s_tile, lane, wm, wn, tid);
    }
  }
}

// Sum of the K pieces of the split remainder tiles (in piece order), then
// bias, SiLU and the bf16 store.  Workgroup b takes a quarter (16 of the 64
// float4 register chunks) of remainder tile (b / 8) / 4 of XCD b % 8 of a
// grouped_gemm_bf16_rs_kernel launch with gemm_grid workgroups; thread tid
// handles the values that thread tid of the GEMM held.
template <int EPI, int GM>
__global__ __launch_bounds__(256) void rs_fixup_kernel(GemmArgs a, RsSplit sp, int gemm_grid) {
  using namespace rs;
  __shared__ int s_pref_f[kMaxGroups + 1];
  __shared__ int s_pref_h[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int xcd = blockIdx.x % kXcds;
  const int t = (blockIdx.x / kXcds) >> 2;
  const int quarter = (blockIdx.x / kXcds) & 3;
  RsTiles tl = rs_tiles(a, s_pref_f, s_pref_h, s_tmp, xcd, gemm_grid / kXcds);
  const RsPlan pl = rs_plan(tl.cnt_f + tl.cnt_h, gemm_grid / kXcds, a.K / BK,
                            sp.partial != nullptr && gemm_grid <= sp.max_blocks);
  tl.inter = tl.inter && pl.P <= 1;   // as in the GEMM launch
  if (pl.P <= 1 || t >= pl.rem) return;
  int g, lm, nt;
  const bool half = rs_tile_at<GM>(a, tl, s_pref_f, s_pref_h, pl.full + t, &g, &lm, &nt);
  const TileView<uint16_t> v = tile_view<uint16_t>(a, g, lm, BM);
  const int n0 = nt * BN;
  const int64_t blk0 = static_cast<int64_t>(t * pl.P) * kXcds + xcd;   // piece 0's workgroup
  // a half-height tail holds 32 register chunks per thread (rh layout), a
  // full tile 64; this workgroup takes a quarter of them
  const int per = half ? 8 : 16;
  // all chunks of one piece are loaded together, pieces are added in order
  float4 acc[16];
  for (int pc = 0; pc < pl.P; ++pc) {
    const float4 *src = reinterpret_cast<const float4 *>(
        sp.partial + (blk0 + static_cast<int64_t>(pc) * kXcds) * (BM * BN));
    float4 p[16];
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
      if (cc < per) p[cc] = src[(quarter * per + cc) * NT + tid];
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) {
      if (cc >= per) continue;
      if (pc == 0) {
        acc[cc] = p[cc];
      } else {
        acc[cc].x += p[cc].x;
        acc[cc].y += p[cc].y;
        acc[cc].z += p[cc].z;
        acc[cc].w += p[cc].w;
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    if (cc >= per) continue;
    const int c = quarter * per + cc;         // (ni * tm + mi) * 4 + q
    int ni, mi, q;
    int64_t row;
    if (half) {
      ni = c >> 3, mi = (c >> 2) & 1, q = c & 3;
      row = v.row0 + wm * rh::WTM + mi * 32 + (lane & 31);
    } else {
      ni = c >> 4, mi = (c >> 2) & 3, q = c & 3;
      row = v.row0 + wm * WTM + mi * 32 + (lane & 31);
    }
    const int n = n0 + wn * WTN + ni * 32 + q * 8 + (lane >> 5) * 4;
    if (row >= v.rows || n >= a.Nout) continue;
    float o[4] = {acc[cc].x, acc[cc].y, acc[cc].z, acc[cc].w};
    if (v.bias) {
      const uint2 bq = *reinterpret_cast<const uint2 *>(v.bias + n);
      o[0] += __uint_as_float(bq.x << 16);
      o[1] += __uint_as_float(bq.x & 0xFFFF0000u);
      o[2] += __uint_as_float(bq.y << 16);
      o[3] += __uint_as_float(bq.y & 0xFFFF0000u);
    }
    if (EPI == kEpiBiasSilu)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = silu_fast(o[e]);
    uint2 packed;
    packed.x = pack_bf16x2(o[0], o[1]);
    packed.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(v.C + (v.out_base + row) * a.Nout + n) = packed;
  }
}

// ---------------------------------------------------------------------------
// bf16 stream kernel for groups with few rows (decode batches, the many small
// experts of a skewed prefill), bound by the weight stream: a deep ring of
// LDS stages keeps about 100 KB of weights in flight per CU.
//
// Work unit: (group, block of 32*NTB rows, block of 128*MB output features,
// k-split part); a wave owns 32*MB features of the unit.  Each 64-wide
// k-chunk of weights and activations goes from HBM straight into one LDS
// stage (global_load_lds: one wave instruction moves 8 rows x 128 bytes, so
// every request uses whole cache lines), rows of 128 bytes with the 16-byte
// pieces swizzled (piece c of row r sits at c ^ ((r >> 1) & 7)) so that the
// MFMA fragment reads of 32 rows hit distinct banks.  A chunk is loaded S-1
// chunks ahead; each step waits for its own wave's copies of the chunk, meets
// the other waves at a barrier (which also frees the oldest stage), refills
// that stage and runs the chunk's MFMAs.
//
// Few units (a decode batch touches few experts) would leave CUs idle, so
// the kernel splits K into up to ks_cap parts when there are fewer than four
// units per workgroup; every workgroup derives the same split from the
// device-side counts.  Split parts write float32 partial sums per output row.
// Otherwise, when an XCD's last round of units would leave at least half its
// workgroups idle, those units alone are split along K into pieces that fill
// the round (stream_plan).  stream_finish_kernel adds the parts or pieces in
// order and applies the epilogue.
// ---------------------------------------------------------------------------
struct StreamSplit {
  float *partial;      // [ks_cap][part_rows + n_shared * T_sh][Nout] or null
  int *ks_used;        // device scalar: the split the kernel chose
  int64_t part_rows;   // routed rows in the partial buffer (host bound)
  int ks_cap;          // 1: never split
  float *rem;          // [grid][rows x features of a unit]: K pieces of last-round units, or null
};

// The last round of a stream launch: each XCD's units run in rounds of its
// nslots workgroups; when the last round would leave at least half of them
// idle, its units are split along K into P pieces (at least four chunks each)
// that fill the idle workgroups, write float32 tiles to the rem buffer, and
// are added in piece order by stream_finish_kernel.
constexpr int kStreamRemBlocks = 256;                          // workgroups with a piece tile
constexpr int64_t kStreamRemTile = 128 * 256;                  // floats per piece tile (largest unit)
constexpr int64_t kStreamRemBytes = kStreamRemBlocks * kStreamRemTile * 4;

struct StreamPlan {
  int begin;   // first unit of the XCD
  int full;    // units in full rounds
  int rem;     // units of the last round
  int P;       // pieces per last-round unit (1: not split)
  int per;     // K chunks per piece
};

__device__ __forceinline__ StreamPlan stream_plan(int total, int xcd, int nslots, int nkc,
                                                  bool can_split) {
  StreamPlan p;
  const int part = (total + kXcds - 1) / kXcds;
  p.begin = xcd * part;
  const int cnt = max(0, min(total, p.begin + part) - p.begin);
  p.full = (cnt / nslots) * nslots;
  p.rem = cnt - p.full;
  p.P = 1;
  p.per = nkc;
  if (can_split && p.rem > 0 && 2 * p.rem <= nslots) {
    const int P = min(min(nslots / p.rem, 8), nkc / 4);
    if (P >= 2) {
      p.per = (nkc + P - 1) / P;
      p.P = (nkc + p.per - 1) / p.per;   // no empty pieces
    }
  }
  return p;
}

namespace st {
constexpr int NT = 256, NW = 4, KCH = 64;
using dma::lds_addr;
using dma::dma16;
using dma::dma16_nt;
using dma::wait_and_barrier;

// wait_and_barrier<n * LPS> for a run-time n in [0, MAXN].
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

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Split chosen from the unit count: at least four units per workgroup.
__device__ __forceinline__ int stream_split(int base_units, int nkc, int ks_cap, int grid,
                                            int *kc_per) {
  int ks = 1;
  if (ks_cap > 1 && base_units > 0) {
    ks = (4 * grid + base_units - 1) / base_units;
    ks = min(ks, ks_cap);
    ks = min(ks, max(1, nkc / 4));   // keep at least four chunks per part
    ks = max(ks, 1);
  }
  const int per = (nkc + ks - 1) / ks;
  *kc_per = per;
  return (nkc + per - 1) / per;      // no empty parts
}
}  // namespace st

// Store of a stream unit: lane holds row r32 of each 32-row block and
// features 8q + 4h .. +3 of each 32-feature block.  Without a K split the
// bias, SiLU and bf16 rounding are applied here; with one, the float32 part
// goes to the partial buffer.
template <int MB, int NTB, int EPI>
__device__ __forceinline__ void stream_store(const f32x16_t (&acc)[MB][NTB], const GemmArgs &a,
                                             const TileView<uint16_t> &v, int g, int nw0, int kp,
                                             int ks, const StreamSplit &sp, int r32, int h,
                                             float *piece, int wf0) {
#pragma unroll
  for (int j = 0; j < NTB; ++j) {
    const int64_t lr = v.row0 + 32 * j + r32;
    if (lr >= v.rows) continue;
    if (piece) {
      // a K piece of a last-round unit: float32 tile [unit row][unit feature]
      constexpr int NB = 4 * 32 * MB;
      float *dst = piece + static_cast<int64_t>(32 * j + r32) * NB + wf0;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16_t &c = acc[i][j];
          *reinterpret_cast<float4 *>(dst + 32 * i + 8 * q + 4 * h) =
              make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
        }
    } else if (ks > 1) {
      const int64_t prow = g < a.n_routed
                               ? v.out_base + lr
                               : sp.part_rows + static_cast<int64_t>(g - a.n_routed) * a.T_sh + lr;
      const int64_t nrows = sp.part_rows + static_cast<int64_t>(a.n_shared) * a.T_sh;
      float *dst = sp.partial + (static_cast<int64_t>(kp) * nrows + prow) * a.Nout;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nw0 + 32 * i + 8 * q + 4 * h;
          if (n < a.Nout) {
            const f32x16_t &c = acc[i][j];
            *reinterpret_cast<float4 *>(dst + n) =
                make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
          }
        }
    } else {
      uint16_t *dst = v.C + (v.out_base + lr) * a.Nout;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nw0 + 32 * i + 8 * q + 4 * h;
          if (n < a.Nout) {
            float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (v.bias) {
              const uint2 bq = *reinterpret_cast<const uint2 *>(v.bias + n);
              bv[0] = __uint_as_float(bq.x << 16);
              bv[1] = __uint_as_float(bq.x & 0xFFFF0000u);
              bv[2] = __uint_as_float(bq.y << 16);
              bv[3] = __uint_as_float(bq.y & 0xFFFF0000u);
            }
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = acc[i][j][4 * q + e] + bv[e];
              if (EPI == kEpiBiasSilu) o[e] = silu_fast(o[e]);
            }
            uint2 packed;
            packed.x = pack_bf16x2(o[0], o[1]);
            packed.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2 *>(dst + n) = packed;
          }
        }
    }
  }
}

// One unit of the stream kernel: rows rb*32*NTB .. of group g (mg row blocks),
// features nb*128*MB .., K part kp of kc_per chunks.  Ring stages are STRIDE
// bf16 elements apart; `stage` is the ring position of the next chunk,
// carried from unit to unit of one workgroup.
template <int MB, int NTB, int S, int STRIDE, int EPI>
__device__ __forceinline__ void stream_unit(const GemmArgs &a, const StreamSplit &sp, int g,
                                            int mg, int nb, int rb, int kp, int ks, int kc_per,
                                            uint16_t *s_ring, uint32_t ring0, int &stage,
                                            int lane, int wave, float *piece) {
  using namespace st;
  constexpr int MR = 32 * NTB;                   // rows per unit
  constexpr int NB = 4 * 32 * MB;                // features per unit
  constexpr int W_INS = NB / 8 / NW;             // weight copies per wave per chunk
  constexpr int X_INS = MR / 8 / NW;             // activation copies per wave per chunk
  constexpr int LPS = W_INS + X_INS;
  static_assert((NB + MR) * KCH <= STRIDE, "stage fits its ring slot");
  static_assert((S - 2) * LPS <= 63, "vmcnt range");
  const int r32 = lane & 31, h = lane >> 5;
  const int nkc = a.K / KCH;
  // lane's place in a copy: row lane/8 of an 8-row block, LDS piece lane%8
  const int crow = lane >> 3, cpos = lane & 7;
  const TileView<uint16_t> v = tile_view<uint16_t>(a, g, rb, MR);
  const int n0 = nb * NB;
  const int kc0 = kp * kc_per;
  const int nch = min(nkc, kc0 + kc_per) - kc0;

  // sources of this wave's copies (chunk 0 of the part)
  const uint16_t *w_src[W_INS];
  const uint16_t *x_src[X_INS];
#pragma unroll
  for (int i = 0; i < W_INS; ++i) {
    const int r = (i * NW + wave) * 8 + crow;
    const int n = min(n0 + r, a.Nout - 1);
    w_src[i] = v.W + static_cast<int64_t>(n) * a.K + kc0 * KCH + swz(r, cpos) * 8;
  }
#pragma unroll
  for (int i = 0; i < X_INS; ++i) {
    const int r = (i * NW + wave) * 8 + crow;
    x_src[i] = a_row_ptr(a, v, v.row0 + r) + kc0 * KCH + swz(r, cpos) * 8;
  }
  // weights of a group with one row block are read once: stream them
  const bool w_once = mg == 1;
  auto issue = [&](int c, int st_idx) {
    const uint32_t base = ring0 + static_cast<uint32_t>(st_idx) * (STRIDE * 2);
    if (w_once) {
#pragma unroll
      for (int i = 0; i < W_INS; ++i) dma16_nt(w_src[i] + c * KCH, base + (i * NW + wave) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < W_INS; ++i) dma16(w_src[i] + c * KCH, base + (i * NW + wave) * 1024);
    }
#pragma unroll
    for (int i = 0; i < X_INS; ++i)
      dma16(x_src[i] + c * KCH, base + NB * KCH * 2 + (i * NW + wave) * 1024);
  };

  f32x16_t acc[MB][NTB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NTB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int pro = min(S - 1, nch);
  for (int c = 0; c < pro; ++c) issue(c, (stage + c) % S);
  for (int c = 0; c < nch; ++c) {
    // copies of chunks c+1 .. min(c+S-2, nch-1) may stay in flight
    const int later = min(S - 2, nch - 1 - c);
    if (later == S - 2) wait_and_barrier<(S - 2) * LPS>();
    else wait_chunks<LPS, S - 3>(later);
    const int cur = (stage + c) % S;
    if (c + S - 1 < nch) issue(c + S - 1, (stage + c + S - 1) % S);
    const uint16_t *sw = s_ring + cur * STRIDE;
    const uint16_t *sx = sw + NB * KCH;
#pragma unroll
    for (int kst = 0; kst < 4; ++kst) {
      const int p = 2 * kst + h;
      bf16x8_t fw[MB], fx[NTB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = wave * 32 * MB + 32 * i + r32;
        fw[i] = *reinterpret_cast<const bf16x8_t *>(sw + r * KCH + swz(r, p) * 8);
      }
#pragma unroll
      for (int j = 0; j < NTB; ++j) {
        const int r = 32 * j + r32;
        fx[j] = *reinterpret_cast<const bf16x8_t *>(sx + r * KCH + swz(r, p) * 8);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NTB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fx[j], acc[i][j], 0, 0, 0);
    }
  }
  stage = (stage + nch) % S;
  stream_store<MB, NTB, EPI>(acc, a, v, g, n0 + wave * 32 * MB, kp, ks, sp, r32, h, piece,
                             wave * 32 * MB);
}

// NTB2 > NTB gives the kernel a second unit height: groups of more than
// 32*NTB rows take units of 32*NTB2 rows, so a group of up to 32*NTB2 rows
// reads each weight block once.  Both shapes share the ring (slots sized
// for the larger stage) and its position.
template <int MB, int NTB, int NTB2, int S, int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_stream_kernel(GemmArgs a, StreamSplit sp) {
  using namespace st;
  constexpr int MR1 = 32 * NTB, MR2 = 32 * (NTB2 > NTB ? NTB2 : NTB);
  constexpr int NB = 4 * 32 * MB;
  constexpr int STRIDE = (NB + MR2) * KCH;
  __shared__ __attribute__((aligned(16))) uint16_t s_ring[S * STRIDE];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n_groups = a.n_routed + a.n_shared;
  const int total_m = build_prefix<NT>(n_groups, [&](int g) {
    const int64_t rows = group_rows(a, g);
    const int mr = rows <= MR1 ? MR1 : MR2;
    return static_cast<int>((rows + mr - 1) / mr);
  }, s_pref, s_tmp);
  const int n_nb = (a.Nout + NB - 1) / NB;
  const int nkc = a.K / KCH;
  int kc_per;
  const int ks = stream_split(total_m * n_nb, nkc, sp.ks_cap, gridDim.x, &kc_per);
  if (blockIdx.x == 0 && threadIdx.x == 0 && sp.ks_used) *sp.ks_used = ks;
  const int total = total_m * n_nb * ks;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const uint32_t ring0 = uniform(static_cast<int>(lds_addr(s_ring)));
  int stage = 0;
  auto run = [&](int u, int kp, int ks_u, int per, float *piece) {
    const int g = find_group(s_pref, n_groups, u / n_nb);
    const int mg = s_pref[g + 1] - s_pref[g];
    const int uu = u - s_pref[g] * n_nb;
    const int nb = uu / mg, rb = uu % mg;
    if (NTB2 <= NTB || group_rows(a, g) <= MR1)
      stream_unit<MB, NTB, S, STRIDE, EPI>(a, sp, g, mg, nb, rb, kp, ks_u, per, s_ring, ring0,
                                           stage, lane, wave, piece);
    else
      stream_unit<MB, (NTB2 > NTB ? NTB2 : NTB), S, STRIDE, EPI>(a, sp, g, mg, nb, rb, kp, ks_u,
                                                                 per, s_ring, ring0, stage, lane,
                                                                 wave, piece);
  };
  // unit order: part fastest, then row block, then feature block, so the
  // workgroups running together share a weight block in L2
  const StreamPlan pl = stream_plan(total, xcd, nslots, nkc, ks == 1 && sp.rem != nullptr &&
                                                                 gridDim.x <= kStreamRemBlocks);
  // the XCD's count of split units, for stream_finish_kernel (header ints
  // 16 .. 23 of the split scratch; written on every launch)
  if (slot == 0 && threadIdx.x == 0 && sp.rem) sp.ks_used[16 + xcd] = pl.P > 1 ? pl.rem : 0;
  const int whole_end = pl.begin + pl.full + (pl.P > 1 ? 0 : pl.rem);
  for (int L = pl.begin + slot; L < whole_end; L += nslots) run(L / ks, L % ks, ks, kc_per, nullptr);
  if (pl.P > 1 && slot < pl.rem * pl.P)
    run(pl.begin + pl.full + slot / pl.P, slot % pl.P, pl.P, pl.per,
        sp.rem + static_cast<int64_t>(blockIdx.x) * kStreamRemTile);
}

// Sum of the K-split partials of output row prow, features n .. n+3, in part
// order; bias, epilogue, bf16 store.  Rows of routed groups past
// offsets[n_routed] do not exist and are skipped.
template <int EPI>
__device__ __forceinline__ void reduce_parts(const GemmArgs &a, const StreamSplit &sp, int ks,
                                             int64_t prow, int n) {
  const int64_t nrows = sp.part_rows + static_cast<int64_t>(a.n_shared) * a.T_sh;
  const uint16_t *bias;
  uint16_t *dst;
  if (prow < sp.part_rows) {
    if (prow >= a.offsets[a.n_routed]) return;
    int lo = 0, hi = a.n_routed;   // offsets[lo] <= prow < offsets[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= prow) lo = mid; else hi = mid;
    }
    if (group_rows(a, lo) == 0) return;   // another kernel's group
    bias = a.bias ? static_cast<const uint16_t *>(a.bias) + static_cast<int64_t>(lo) * a.Nout : nullptr;
    dst = static_cast<uint16_t *>(a.C) + prow * a.Nout;
  } else {
    const int gs = static_cast<int>((prow - sp.part_rows) / a.T_sh);
    if (group_rows(a, a.n_routed + gs) == 0) return;
    bias = a.bias_sh ? static_cast<const uint16_t *>(a.bias_sh) + static_cast<int64_t>(gs) * a.Nout
                     : nullptr;
    dst = static_cast<uint16_t *>(a.C_sh) + (prow - sp.part_rows) * a.Nout;
  }
  float4 s = *reinterpret_cast<const float4 *>(sp.partial + prow * a.Nout + n);
  for (int p = 1; p < ks; ++p) {
    const float4 t = *reinterpret_cast<const float4 *>(sp.partial + (p * nrows + prow) * a.Nout + n);
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  float o[4] = {s.x, s.y, s.z, s.w};
  if (bias) {
    const uint2 bq = *reinterpret_cast<const uint2 *>(bias + n);
    o[0] += __uint_as_float(bq.x << 16);
    o[1] += __uint_as_float(bq.x & 0xFFFF0000u);
    o[2] += __uint_as_float(bq.y << 16);
    o[3] += __uint_as_float(bq.y & 0xFFFF0000u);
  }
  if (EPI == kEpiBiasSilu)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = silu_fast(o[e]);
  uint2 packed;
  packed.x = pack_bf16x2(o[0], o[1]);
  packed.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2 *>(dst + n) = packed;
}

// After a stream launch of grid workgroups: with a uniform K split, the sum
// of every row's parts; otherwise workgroups (xcd, j, 0 .. fpu-1) of this
// launch add the pieces of the j-th last-round unit of that XCD, if the
// launch split it (stream_plan on the same device counts decides exactly as
// the stream kernel did).  fpu = workgroups per unit, one per 512 four-float
// elements of the unit, so a launch that split nothing is a small grid that
// exits at once.
constexpr int kFinishMaxPerUnit = 16;
constexpr int kFinishMaxUniform = 512;   // workgroups of the uniform K-split sum
template <int MB, int NTB, int NTB2, int EPI>
__global__ __launch_bounds__(256) void stream_finish_kernel(GemmArgs a, StreamSplit sp, int grid,
                                                            int fpu) {
  using namespace st;
  const int ks = *sp.ks_used;
  if (ks > 1) {
    const int64_t nrows = sp.part_rows + static_cast<int64_t>(a.n_shared) * a.T_sh;
    const int nq = a.Nout / 4;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nrows * nq;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
      reduce_parts<EPI>(a, sp, ks, i / nq, static_cast<int>(i % nq) * 4);
    return;
  }
  if (!sp.rem || grid > kStreamRemBlocks) return;
  const int nslots = grid / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int j = (blockIdx.x / kXcds) % (nslots / 2 > 0 ? nslots / 2 : 1);
  const int q = (blockIdx.x / kXcds) / (nslots / 2 > 0 ? nslots / 2 : 1);
  if (q >= fpu) return;                    // a workgroup of the uniform-sum grid only
  if (j >= sp.ks_used[16 + xcd]) return;   // not a split unit of this launch
  constexpr int MR1 = 32 * NTB, MR2 = 32 * (NTB2 > NTB ? NTB2 : NTB);
  constexpr int NB = 4 * 32 * MB;
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];
  const int n_groups = a.n_routed + a.n_shared;
  const int total_m = build_prefix<NT>(n_groups, [&](int g) {
    const int64_t rows = group_rows(a, g);
    const int mr = rows <= MR1 ? MR1 : MR2;
    return static_cast<int>((rows + mr - 1) / mr);
  }, s_pref, s_tmp);
  const int n_nb = (a.Nout + NB - 1) / NB;
  const StreamPlan pl = stream_plan(total_m * n_nb, xcd, nslots, a.K / KCH, true);
  if (pl.P <= 1 || j >= pl.rem) return;
  const int u = pl.begin + pl.full + j;
  const int g = find_group(s_pref, n_groups, u / n_nb);
  const int mg = s_pref[g + 1] - s_pref[g];
  const int uu = u - s_pref[g] * n_nb;
  const int nb = uu / mg, rb = uu % mg;
  const int MR = group_rows(a, g) <= MR1 ? MR1 : MR2;
  const TileView<uint16_t> v = tile_view<uint16_t>(a, g, rb, MR);
  const int n0 = nb * NB;
  const float *pieces = sp.rem + static_cast<int64_t>(j * pl.P * kXcds + xcd) * kStreamRemTile;
  for (int e = q * blockDim.x + threadIdx.x; e < MR * (NB / 4); e += fpu * blockDim.x) {
    const int r = e / (NB / 4), f = (e % (NB / 4)) * 4;
    const int64_t lr = v.row0 + r;
    const int n = n0 + f;
    if (lr >= v.rows || n >= a.Nout) continue;
    // piece kp of unit j sits at workgroup slot j*P + kp of this XCD; all of
    // an element's pieces are loaded before they are added in piece order
    float4 t[8];
#pragma unroll
    for (int kp = 0; kp < 8; ++kp)
      if (kp < pl.P)
        t[kp] = *reinterpret_cast<const float4 *>(
            pieces + static_cast<int64_t>(kp) * kXcds * kStreamRemTile + static_cast<int64_t>(r) * NB + f);
    float4 s = t[0];
#pragma unroll
    for (int kp = 1; kp < 8; ++kp)
      if (kp < pl.P) {
        s.x += t[kp].x;
        s.y += t[kp].y;
        s.z += t[kp].z;
        s.w += t[kp].w;
      }
    float o[4] = {s.x, s.y, s.z, s.w};
    if (v.bias) {
      const uint2 bq = *reinterpret_cast<const uint2 *>(v.bias + n);
      o[0] += __uint_as_float(bq.x << 16);
      o[1] += __uint_as_float(bq.x & 0xFFFF0000u);
      o[2] += __uint_as_float(bq.y << 16);
      o[3] += __uint_as_float(bq.y & 0xFFFF0000u);
    }
    if (EPI == kEpiBiasSilu)
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = silu_fast(o[q]);
    uint2 packed;
    packed.x = pack_bf16x2(o[0], o[1]);
    packed.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(v.C + (v.out_base + lr) * a.Nout + n) = packed;
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: 64x64 tiles, 256 threads
// ---------------------------------------------------------------------------
template <typename TA, int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_valu_kernel(GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16, NT = 256, GM = 8;
  __shared__ float s_a[BK][BM + 4];
  __shared__ float s_b[BK][BN + 4];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];
  const int tid = threadIdx.x;
  const int n_groups = a.n_routed + a.n_shared;
  const int total_m = build_tile_prefix<NT, BM>(a, s_pref, s_tmp);
  const int n_nt = (a.Nout + BN - 1) / BN;
  const int total = total_m * n_nt;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslots = gridDim.x / kXcds;
  const int part = (total + kXcds - 1) / kXcds;
  const int begin = xcd * part, end = min(total, begin + part);
  const int tm = tid & 15, tn = tid >> 4;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;   // loader: 64 rows x 4 chunks of 4

  for (int L = begin + slot; L < end; L += nslots) {
    int mt, nt;
    decode_tile<GM>(L, total_m, n_nt, &mt, &nt);
    const int g = find_group(s_pref, n_groups, mt);
    const TileView<TA> v = tile_view<TA>(a, g, mt - s_pref[g], BM);
    const int n0 = nt * BN;
    const TA *arow = a_row_ptr<TA>(a, v, v.row0 + lrow);
    int nb = n0 + lrow;
    if (nb >= a.Nout) nb = a.Nout - 1;
    const TA *brow = v.W + static_cast<int64_t>(nb) * a.K;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < a.K; k0 += BK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s_a[lk + j][lrow] = Act<TA>::to_f32(arow[k0 + lk + j]);
        s_b[lk + j][lrow] = Act<TA>::to_f32(brow[k0 + lk + j]);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < BK; ++k) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { av[i] = s_a[k][tm * 4 + i]; bv[i] = s_b[k][tn * 4 + i]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }
    TA *C = v.C;
    const TA *bias = v.bias;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rr = v.row0 + tm * 4 + i;
      if (rr >= v.rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tn * 4 + j;
        if (n >= a.Nout) continue;
        float o = acc[i][j];
        if (bias) o += Act<TA>::to_f32(bias[n]);
        if (EPI == kEpiBiasSilu) o = silu(o);
        C[(v.out_base + rr) * a.Nout + n] = Act<TA>::from_f32(o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct DevInfo {
  int cus = 0;
};

DevInfo &dev_info() {
  static DevInfo info[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  DevInfo &d = info[dev & 63];
  if (d.cus == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    d.cus = v;
  }
  return d;
}

GemmArgs make_args(const GemmGroups &g) {
  GemmArgs a;
  a.offsets = g.offsets;
  a.A = g.A;
  a.a_index = g.a_index;
  a.A_sh = g.A_sh;
  a.W = g.W;
  a.bias = g.bias;
  a.W_sh = g.W_sh;
  a.bias_sh = g.bias_sh;
  a.C = g.C;
  a.C_sh = g.C_sh;
  a.T_sh = g.T_sh;
  a.a_sh_stride = g.a_sh_stride;
  a.n_routed = g.n_routed;
  a.n_shared = g.n_shared;
  a.Nout = g.Nout;
  a.K = g.K;
  a.cls_lo = 0;
  a.cls_hi = INT64_MAX;
  return a;
}

int64_t tiles_upper_bound(const GemmGroups &g, int BM, int BN) {
  const int64_t m = g.max_routed_rows / BM + g.n_routed +
                    static_cast<int64_t>(g.n_shared) * ((g.T_sh + BM - 1) / BM);
  return m * ((g.Nout + BN - 1) / BN);
}

// Persistent grid: enough workgroups to fill the chip (per_cu resident per
// CU), never more than tiles exist, always a multiple of the XCD count.
unsigned persistent_grid(int64_t tiles_ub, int per_cu) {
  const int64_t full = static_cast<int64_t>(dev_info().cus) * per_cu;
  int64_t g = tiles_ub < full ? tiles_ub : full;
  g = ((g + kXcds - 1) / kXcds) * kXcds;
  if (g < kXcds) g = kXcds;
  return static_cast<unsigned>(g);
}

constexpr int kSplitCap = 8;
constexpr int64_t kSplitMaxRows = 4096;   // partial rows (reduce grid.y, scratch size)

int64_t split_rows(const GemmGroups &g) {
  return g.max_routed_rows + static_cast<int64_t>(g.n_shared) * g.T_sh;
}

template <int MB, int NTB, int S, int NTB2 = 0>
hipError_t launch_bf16_stream(const GemmArgs &a, const GemmGroups &g, Epilogue epi, int per_cu,
                              hipStream_t s) {
  // scratch: [0, 256) the split the kernel chose; then the last-round piece
  // tiles; then, for small products, the uniform K-split partial sums
  StreamSplit sp{};
  sp.ks_cap = 1;
  const int64_t prows = split_rows(g);
  const int64_t head = 256 + kStreamRemBytes;
  if (g.split_ws && static_cast<int64_t>(g.split_bytes) >= head) {
    char *ws = static_cast<char *>(g.split_ws);
    sp.ks_used = reinterpret_cast<int *>(ws);
    sp.rem = reinterpret_cast<float *>(ws + 256);
    if (prows <= kSplitMaxRows) {
      const int64_t per = prows * g.Nout * static_cast<int64_t>(sizeof(float));
      const int64_t cap = (static_cast<int64_t>(g.split_bytes) - head) / per;
      if (cap > 1) {
        sp.partial = reinterpret_cast<float *>(ws + head);
        sp.part_rows = g.max_routed_rows;
        sp.ks_cap = static_cast<int>(cap < kSplitCap ? cap : kSplitCap);
      }
    }
  }
  const unsigned grid =
      persistent_grid(tiles_upper_bound(g, 32 * NTB, 128 * MB) * sp.ks_cap, per_cu);
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((grouped_gemm_bf16_stream_kernel<MB, NTB, NTB2, S, kEpiBiasSilu>),
                       dim3(grid), dim3(256), 0, s, a, sp);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_stream_kernel<MB, NTB, NTB2, S, kEpiBias>), dim3(grid),
                       dim3(256), 0, s, a, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sp.ks_used) return e;
  // fpu workgroups per possible last-round unit (at most half of each XCD's
  // workgroups), one per 512 four-float elements of the largest unit; at
  // least enough for the uniform K-split sum's grid-stride loop
  constexpr int kUnitElems = 32 * (NTB2 > NTB ? NTB2 : NTB) * (4 * 32 * MB) / 4;
  constexpr int fpu = kUnitElems / 512 < 1 ? 1
                      : (kUnitElems / 512 > kFinishMaxPerUnit ? kFinishMaxPerUnit : kUnitElems / 512);
  int64_t fgrid = static_cast<int64_t>(kXcds) * ((grid / kXcds) / 2 > 0 ? (grid / kXcds) / 2 : 1) * fpu;
  if (sp.ks_cap > 1) {
    const int64_t need = (prows * (g.Nout / 4) + 255) / 256;
    const int64_t cap_blocks = need < kFinishMaxUniform ? need : kFinishMaxUniform;
    if (cap_blocks > fgrid) fgrid = cap_blocks;
  }
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((stream_finish_kernel<MB, NTB, NTB2, kEpiBiasSilu>), dim3(static_cast<unsigned>(fgrid)),
                       dim3(256), 0, s, a, sp, static_cast<int>(grid), fpu);
  else
    hipLaunchKernelGGL((stream_finish_kernel<MB, NTB, NTB2, kEpiBias>), dim3(static_cast<unsigned>(fgrid)),
                       dim3(256), 0, s, a, sp, static_cast<int>(grid), fpu);
  return hipGetLastError();
}

constexpr int64_t kRsPieceBytes = 256 * 256 * sizeof(float);
constexpr int kRsMaxBlocks = 256;

// The 256x256 kernel's copies address their sources as 32-bit byte offsets
// from wave-uniform bases when every offset fits: A rows lie below
// max(max_routed_rows, T_sh) (gathered rows index the T_sh tokens), W rows
// below Nout.  Larger operands take the 64-bit form.
bool rs_off32(const GemmGroups &g) {
  if (g.a_index && g.T_sh <= 0) return false;
  const int64_t rows = g.max_routed_rows > g.T_sh ? g.max_routed_rows : g.T_sh;
  const int64_t lim = (int64_t(1) << 32) - 4096;
  return rows * g.K * 2 < lim && static_cast<int64_t>(g.Nout) * g.K * 2 < lim;
}

template <int GM>
hipError_t launch_bf16_rs(const GemmArgs &a, const GemmGroups &g, Epilogue epi, hipStream_t s) {
  const unsigned grid = persistent_grid(tiles_upper_bound(g, 256, 256), 1);
  RsSplit sp{};
  if (g.split_ws && g.K / 64 >= 64) {
    sp.max_blocks = static_cast<int>(static_cast<int64_t>(g.split_bytes) / kRsPieceBytes);
    if (sp.max_blocks >= static_cast<int>(grid)) sp.partial = static_cast<float *>(g.split_ws);
  }
  const bool off32 = rs_off32(g);
#define MOE_RS_LAUNCH(EPI, PIECE)                                                                \
  {                                                                                              \
    if (off32)                                                                                   \
      hipLaunchKernelGGL((grouped_gemm_bf16_rs_kernel<EPI, GM, PIECE, true>), dim3(grid),        \
                         dim3(256), 0, s, a, sp);                                                \
    else                                                                                         \
      hipLaunchKernelGGL((grouped_gemm_bf16_rs_kernel<EPI, GM, PIECE, false>), dim3(grid),       \
                         dim3(256), 0, s, a, sp);                                                \
  }
  if (epi == kEpiBiasSilu) MOE_RS_LAUNCH(kEpiBiasSilu, false)
  else MOE_RS_LAUNCH(kEpiBias, false)
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sp.partial) return e;
  MOE_RS_LAUNCH(kEpiBias, true)
#undef MOE_RS_LAUNCH
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // at most half of each XCD's workgroups hold remainder tiles; four
  // fixup workgroups per tile
  const dim3 fgrid(static_cast<unsigned>(kXcds * 4 * (grid / kXcds / 2 > 0 ? grid / kXcds / 2 : 1)));
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((rs_fixup_kernel<kEpiBiasSilu, GM>), fgrid, dim3(256), 0, s, a, sp, static_cast<int>(grid));
  else
    hipLaunchKernelGGL((rs_fixup_kernel<kEpiBias, GM>), fgrid, dim3(256), 0, s, a, sp, static_cast<int>(grid));
  return hipGetLastError();
}

}  // namespace

size_t grouped_gemm_split_bytes(const GemmGroups &g) {
  // the stream kernel: its split word, the last-round piece tiles and, for
  // small products, K-split partial sums; the 256x256 kernel: one float32
  // 256x256 tile per workgroup of its split last round
  const int64_t prows = split_rows(g);
  size_t stream = 256 + static_cast<size_t>(kStreamRemBytes);
  if (prows <= kSplitMaxRows)
    stream += sizeof(float) * static_cast<size_t>(kSplitCap) * prows * g.Nout;
  const size_t rs = static_cast<size_t>(kRsMaxBlocks) * kRsPieceBytes;
  return stream > rs ? stream : rs;
}

hipError_t launch_grouped_gemm(bool bf16, const GemmGroups &g, Epilogue epi, hipStream_t s) {
  GemmArgs a = make_args(g);
  if (g.n_routed + g.n_shared <= 0 || g.Nout <= 0) return hipSuccess;
  if (bf16 && g.K % 64 == 0 && g.Nout % 4 == 0) {
    // Groups of up to kStreamRows rows are bound by their weight stream and
    // go to the stream kernel (units of 64 rows up to 64 rows, else 128, so
    // each weight block is read once); larger groups reuse each weight tile
    // across up to 256 rows in the 256x256 kernel, which measures faster
    // from about 130 rows on.  Each kernel takes its own size class.
    // Batches of at most 32 rows per group (decode) use the deep-ring
    // 32-row shape.
    constexpr int64_t kStreamRows = 128;
    const int64_t groups = g.n_routed > 0 ? g.n_routed : 1;
    const int64_t mean_rows = g.max_routed_rows / groups;
    const int64_t max_rows = g.n_routed > 0 ? g.max_group_rows : 0;
    const bool any_big = max_rows > kStreamRows || (g.n_shared > 0 && g.T_sh > kStreamRows);
    const bool any_small = (g.n_routed > 0 && mean_rows < 384) || (g.n_shared > 0 && g.T_sh <= kStreamRows);
    if (!any_big) {
      if (max_rows <= 32) return launch_bf16_stream<1, 1, 6>(a, g, epi, 1, s);
      return launch_bf16_stream<2, 2, 3, 4>(a, g, epi, 1, s);
    }
    if (!any_small) return launch_bf16_rs<4>(a, g, epi, s);
    GemmArgs ab = a, as = a;
    ab.cls_lo = kStreamRows + 1;
    as.cls_hi = kStreamRows;
    hipError_t e = launch_bf16_rs<4>(ab, g, epi, s);
    if (e != hipSuccess) return e;
    return launch_bf16_stream<2, 2, 3, 4>(as, g, epi, 1, s);
  }
  // bf16 widths are multiples of 64 (checked at the interface), so only
  // float32 operands reach the VALU kernel
  if (bf16) return hipErrorInvalidValue;
  const unsigned grid = persistent_grid(tiles_upper_bound(g, 64, 64), 4);
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((grouped_gemm_valu_kernel<float, kEpiBiasSilu>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_valu_kernel<float, kEpiBias>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
