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
// Scheduling: persistent workgroups; the tile range is split into eight equal
// contiguous parts, one per XCD (workgroups are dealt to the eight XCDs
// round-robin by id), and within a part tiles are visited in bands of GM
// m-tiles so that the workgroups running together on one XCD share weight
// tiles and activation tiles in that XCD's L2.
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulate.  Tiles go from
// HBM straight into LDS (global_load_lds, 16 bytes per lane, no staging
// registers), double buffered, with an XOR swizzle of the 16-byte chunks so
// the fragment reads of 32 rows hit distinct banks.  The weight tile is the MFMA's first operand,
// so each lane ends up holding four consecutive output features of one row
// and the epilogue writes 8-byte packed bf16 stores.
//
// fp32 path: a plain LDS-tiled VALU kernel (4x4 register tile per thread).
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
};

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
  for (int g = g0; g < g1; ++g) {
    const int64_t rows = g < a.n_routed ? (a.offsets[g + 1] - a.offsets[g]) : a.T_sh;
    local += static_cast<int>((rows + BM - 1) / BM);
  }
  int total;
  int run = block_excl_scan<NT>(local, s_tmp, &total);
  for (int g = g0; g < g1; ++g) {
    s_pref[g] = run;
    const int64_t rows = g < a.n_routed ? (a.offsets[g + 1] - a.offsets[g]) : a.T_sh;
    run += static_cast<int>((rows + BM - 1) / BM);
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
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
// One wave instruction moves 8 tile rows x 128 bytes straight from global
// memory into LDS: lane L lands at byte 16*L of the 1 KB block, i.e. row L/8,
// chunk position L%8.  Position p of row r must hold logical chunk p ^ (r%8)
// (the XOR swizzle the fragment reads expect), so lane L fetches chunk
// (L%8) ^ (L/8) of its row; the 128-byte row segment stays fully used.
__device__ __forceinline__ void load_rows_to_lds(const uint16_t *src, uint16_t *lds_block) {
  __builtin_amdgcn_global_load_lds(src, lds_block, 16, 0, 0);
}

// Issue the global->LDS loads of K-step kb into one stage.
template <int A_INS, int B_INS, int NW, int BM, int BK>
__device__ __forceinline__ void issue_stage(uint16_t *sa, const uint16_t *const (&a_src)[A_INS],
                                            const uint16_t *const (&b_src)[B_INS], int kb,
                                            int wave) {
  uint16_t *sb = sa + BM * BK;
#pragma unroll
  for (int j = 0; j < A_INS; ++j) load_rows_to_lds(a_src[j] + kb * BK, sa + (j * NW + wave) * 8 * BK);
#pragma unroll
  for (int j = 0; j < B_INS; ++j) load_rows_to_lds(b_src[j] + kb * BK, sb + (j * NW + wave) * 8 * BK);
}

// Fragments of one 16-wide K slice: lane l holds 8 consecutive k of row l%32
// (k offset 8*(l/32)) for each 32-row block of the wave's rows.
template <int TM, int TN, int BM, int BK, int WTM, int WTN>
__device__ __forceinline__ void load_frags(const uint16_t *sa, bf16x8_t (&fa)[TM],
                                           bf16x8_t (&fb)[TN], int ks, int wm, int wn,
                                           int lane) {
  const uint16_t *sb = sa + BM * BK;
  const int c = ks * 2 + (lane >> 5);
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    const int row = wm * WTM + mi * 32 + (lane & 31);
    fa[mi] = *reinterpret_cast<const bf16x8_t *>(sa + row * BK + ((c ^ (row & 7)) << 3));
  }
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
    const int row = wn * WTN + ni * 32 + (lane & 31);
    fb[ni] = *reinterpret_cast<const bf16x8_t *>(sb + row * BK + ((c ^ (row & 7)) << 3));
  }
}

// Multiply one staged K-step into the wave's accumulators.  The fragments of
// slice ks+1 are read while the MFMAs of slice ks run (two register sets).
template <int TM, int TN, int BM, int BK, int WTM, int WTN>
__device__ __forceinline__ void mma_stage(const uint16_t *sa, f32x16_t (&acc)[TN][TM], int wm,
                                          int wn, int lane) {
  constexpr int NS = BK / 16;
  bf16x8_t fa[2][TM], fb[2][TN];
  load_frags<TM, TN, BM, BK, WTM, WTN>(sa, fa[0], fb[0], 0, wm, wn, lane);
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) {
    if (ks + 1 < NS)
      load_frags<TM, TN, BM, BK, WTM, WTN>(sa, fa[(ks + 1) & 1], fb[(ks + 1) & 1], ks + 1, wm, wn,
                                           lane);
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][ni], fa[ks & 1][mi],
                                                              acc[ni][mi], 0, 0, 0);
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int GM>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void grouped_gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int BK = 64;                 // 8 chunks of 16 B per row
  constexpr int WTM = BM / WAVES_M;      // rows (tokens) per wave
  constexpr int WTN = BN / WAVES_N;      // output features per wave
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int NW = NT / 64;
  constexpr int A_INS = BM / 8 / NW;     // 8-row global->LDS loads per wave per stage
  constexpr int B_INS = BN / 8 / NW;
  constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be MFMA-aligned");
  static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "row blocks must divide evenly");

  // Two stages as distinct objects, so the compiler can tell the loads into
  // one from the reads of the other and need not wait between them.
  __shared__ __attribute__((aligned(16))) uint16_t s_st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s_st1[STAGE];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int n_groups = a.n_routed + a.n_shared;

  const int total_m = build_tile_prefix<NT, BM>(a, s_pref, s_tmp);
  const int n_nt = (a.Nout + BN - 1) / BN;
  const int total = total_m * n_nt;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int part = (total + kXcds - 1) / kXcds;
  const int begin = xcd * part;
  const int end = min(total, begin + part);
  const int nk = a.K / BK;
  const int lrow = lane >> 3;                       // row within an 8-row block
  const int lchunk = (lane & 7) ^ lrow;             // logical chunk this lane fetches

  for (int L = begin + slot; L < end; L += nslots) {
    int mt, nt;
    decode_tile<GM>(L, total_m, n_nt, &mt, &nt);
    const int g = find_group(s_pref, n_groups, mt);
    const TileView<uint16_t> v = tile_view<uint16_t>(a, g, mt - s_pref[g], BM);
    const int n0 = nt * BN;

    const uint16_t *a_src[A_INS];
    const uint16_t *b_src[B_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int row = (j * NW + wave) * 8 + lrow;
      a_src[j] = a_row_ptr(a, v, v.row0 + row) + lchunk * 8;
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      int n = n0 + (j * NW + wave) * 8 + lrow;
      if (n >= a.Nout) n = a.Nout - 1;
      b_src[j] = v.W + static_cast<int64_t>(n) * a.K + lchunk * 8;
    }
    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Two LDS stages: the loads of step kb+1 land in one while step kb is
    // multiplied out of the other; the barrier at the end of each step both
    // publishes the new stage and frees the old one.
    issue_stage<A_INS, B_INS, NW, BM, BK>(s_st0, a_src, b_src, 0, wave);
    __syncthreads();
    int kb = 0;
    for (; kb + 1 < nk; kb += 2) {
      issue_stage<A_INS, B_INS, NW, BM, BK>(s_st1, a_src, b_src, kb + 1, wave);
      mma_stage<TM, TN, BM, BK, WTM, WTN>(s_st0, acc, wm, wn, lane);
      __syncthreads();
      if (kb + 2 < nk) issue_stage<A_INS, B_INS, NW, BM, BK>(s_st0, a_src, b_src, kb + 2, wave);
      mma_stage<TM, TN, BM, BK, WTM, WTN>(s_st1, acc, wm, wn, lane);
      __syncthreads();
    }
    if (kb < nk) {   // odd number of K-steps: the last one sits in stage 0
      mma_stage<TM, TN, BM, BK, WTM, WTN>(s_st0, acc, wm, wn, lane);
      __syncthreads();
    }

    // Epilogue through LDS: bias, SiLU and bf16 rounding per accumulator,
    // into a [BM][BN] bf16 tile whose 16-byte chunks are XOR-swizzled by row
    // (acc[ni][mi][q*4 + j] holds feature wn*WTN + ni*32 + q*8 + (lane/32)*4 + j
    // of row wm*WTM + mi*32 + lane%32); then whole rows leave in 16-byte stores.
    // Opaque copies of the lane coordinates keep the epilogue's address
    // arithmetic below the K loop instead of live across it.
    int el = lane, ewm = wm, ewn = wn, etid = tid;
    asm volatile("" : "+v"(el), "+v"(etid), "+s"(ewm), "+s"(ewn));
    constexpr int CH = BN / 8;                       // 16-byte chunks per tile row
    constexpr int XM = (CH < 32 ? CH : 32) - 1;      // swizzle mask
    // the C tile takes stage 0, spilling its second half of rows into stage 1
    constexpr bool kSplitC = BM * BN > STAGE;
    static_assert(!kSplitC || (BM * BN) / 2 <= STAGE, "C tile must fit in the LDS stages");
#define MOE_CROW(r) ((kSplitC && (r) >= BM / 2) ? s_st1 + ((r) - BM / 2) * BN : s_st0 + (r) * BN)
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
            if (EPI == kEpiBiasSilu) o[j] = silu(o[j]);
          }
          uint2 packed;
          packed.x = f32_to_bf16(o[0]) | (static_cast<uint32_t>(f32_to_bf16(o[1])) << 16);
          packed.y = f32_to_bf16(o[2]) | (static_cast<uint32_t>(f32_to_bf16(o[3])) << 16);
          const int pos = (nl >> 3) ^ (ml & XM);
          *reinterpret_cast<uint2 *>(MOE_CROW(ml) + pos * 8 + ((nl >> 2) & 1) * 4) = packed;
        }
      }
    }
    __syncthreads();
    for (int i = etid; i < BM * CH; i += NT) {
      const int r = i / CH, c = i % CH;
      const int64_t row = v.row0 + r;
      const int n = n0 + c * 8;
      if (row < v.rows && n < a.Nout) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t *>(MOE_CROW(r) + ((c ^ (r & XM)) << 3));
        *reinterpret_cast<u32x4_t *>(v.C + (v.out_base + row) * a.Nout + n) = val;
      }
    }
#undef MOE_CROW
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, deep pipeline: 256x256 tiles, four 128x128 wave tiles,
// K-steps of 32 in four LDS stages (32 KB each), loads issued three steps
// ahead.  Each step ends with a wait for just the stage needed next
// (s_waitcnt vmcnt(N) on this wave's own loads) and a plain s_barrier, so the
// loads of the two younger stages stay in flight across it.
// ---------------------------------------------------------------------------
namespace deep {
constexpr int BM = 256, BN = 256, BK = 32, NT = 256, NW = 4, WTM = 128, WTN = 128;
constexpr int TM = WTM / 32, TN = WTN / 32;
constexpr int ROWS_PER_INS = 16;                       // 1 KB per wave instruction
constexpr int A_INS = BM / ROWS_PER_INS / NW;          // 4
constexpr int B_INS = BN / ROWS_PER_INS / NW;          // 4
constexpr int LOADS_PER_STAGE = A_INS + B_INS;         // per wave
constexpr int STAGE = (BM + BN) * BK;                  // 16384 bf16 = 32 KB
static_assert(STAGE == 64 * BN, "each stage holds 64 rows of the C tile");

// 64-byte rows, 4 chunks of 16 B; chunk c of row r sits at c ^ ((r >> 1) & 3),
// which keeps 8 consecutive rows read at one logical chunk on distinct banks.
__device__ __forceinline__ int pos(int r, int c) { return c ^ ((r >> 1) & 3); }

// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// One wave-wide LDS DMA (64 lanes x 16 B) written as inline assembly, so the
// compiler does not treat every later LDS read as a possible alias of it and
// drain all loads in flight; the wait before each barrier covers it instead.
// M0 carries the LDS byte address of the 1 KB block (wave-uniform).
__device__ __forceinline__ void dma16(const uint16_t *src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

// Loads of K-step kb into the stage at LDS byte address `stage` (A rows first,
// then B rows; 16 rows of 64 B per instruction).
__device__ __forceinline__ void issue(uint32_t stage, const uint16_t *const (&a_src)[A_INS],
                                      const uint16_t *const (&b_src)[B_INS], int kb, int wave) {
  constexpr uint32_t kBlock = ROWS_PER_INS * BK * 2;   // bytes per instruction
#pragma unroll
  for (int j = 0; j < A_INS; ++j)
    dma16(a_src[j] + kb * BK, stage + (j * NW + wave) * kBlock);
#pragma unroll
  for (int j = 0; j < B_INS; ++j)
    dma16(b_src[j] + kb * BK, stage + BM * BK * 2 + (j * NW + wave) * kBlock);
}

// Fragments of one K-step (two 16-wide slices): lane l holds 8 consecutive k
// of row l%32 of each 32-row block (k offset 8*(l/32) within the slice).
struct Frags {
  bf16x8_t a[2][TM];
  bf16x8_t b[2][TN];
};

__device__ __forceinline__ void read_frags(const uint16_t *sa, Frags &f, int wm, int wn, int lane) {
  const uint16_t *sb = sa + BM * BK;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int row = wm * WTM + mi * 32 + (lane & 31);
      f.a[ks][mi] = *reinterpret_cast<const bf16x8_t *>(sa + row * BK + (pos(row, c) << 3));
    }
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
      const int row = wn * WTN + ni * 32 + (lane & 31);
      f.b[ks][ni] = *reinterpret_cast<const bf16x8_t *>(sb + row * BK + (pos(row, c) << 3));
    }
  }
}

__device__ __forceinline__ void mfma_frags(const Frags &f, f32x16_t (&acc)[TN][TM]) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
      for (int mi = 0; mi < TM; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ks][ni], f.a[ks][mi], acc[ni][mi],
                                                              0, 0, 0);
}

// Interleave the next step's 16 fragment reads with this step's 32 MFMAs.
__device__ __forceinline__ void interleave_reads_with_mfma() {
#pragma unroll
  for (int i = 0; i < (BK / 16) * (TM + TN); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
  }
}

// Wait until at most N of this wave's loads are in flight and its LDS reads
// are done, then meet the other waves.  The empty asm statements keep the
// compiler from moving memory operations across the barrier.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace deep

template <int EPI, int GM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_deep_kernel(GemmArgs a) {
  using namespace deep;
  __shared__ __attribute__((aligned(16))) uint16_t s0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s2[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s3[STAGE];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int n_groups = a.n_routed + a.n_shared;
  const int total_m = build_tile_prefix<NT, BM>(a, s_pref, s_tmp);
  const int n_nt = (a.Nout + BN - 1) / BN;
  const int total = total_m * n_nt;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int part = (total + kXcds - 1) / kXcds;
  const int begin = xcd * part;
  const int end = min(total, begin + part);
  const int nk = a.K / BK;                     // multiple of 2 (K % 64 == 0)
  const int lrow = lane >> 2;                  // row within a 16-row block
  const int lchunk = (lane & 3) ^ ((lane >> 3) & 3);
  const uint32_t a0 = uniform(static_cast<int>(lds_addr(s0)));
  const uint32_t a1 = uniform(static_cast<int>(lds_addr(s1)));
  const uint32_t a2 = uniform(static_cast<int>(lds_addr(s2)));
  const uint32_t a3 = uniform(static_cast<int>(lds_addr(s3)));

  for (int L = begin + slot; L < end; L += nslots) {
    int mt, nt;
    decode_tile<GM>(L, total_m, n_nt, &mt, &nt);
    const int g = find_group(s_pref, n_groups, mt);
    const TileView<uint16_t> v = tile_view<uint16_t>(a, g, mt - s_pref[g], BM);
    const int n0 = nt * BN;
    const uint16_t *a_src[A_INS];
    const uint16_t *b_src[B_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j)
      a_src[j] = a_row_ptr(a, v, v.row0 + (j * NW + wave) * ROWS_PER_INS + lrow) + lchunk * 8;
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      int n = n0 + (j * NW + wave) * ROWS_PER_INS + lrow;
      if (n >= a.Nout) n = a.Nout - 1;
      b_src[j] = v.W + static_cast<int64_t>(n) * a.K + lchunk * 8;
    }
    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Schedule of step kb (stage kb%4 holds step kb, its fragments are in
    // registers already): barrier (step kb+1 has landed, every wave has read
    // stage kb%4), issue step kb+4 into stage kb%4, then read step kb+1's
    // fragments from stage (kb+1)%4 while the MFMAs of step kb run.
    Frags f0, f1;
    issue(a0, a_src, b_src, 0, wave);
    if (nk > 1) issue(a1, a_src, b_src, 1, wave);
    if (nk > 2) issue(a2, a_src, b_src, 2, wave);
    if (nk > 3) issue(a3, a_src, b_src, 3, wave);
    if (nk > 3) wait_and_barrier<3 * LOADS_PER_STAGE>();
    else wait_and_barrier<0>();
    read_frags(s0, f0, wm, wn, lane);

#define MOE_DEEP_FULL(DMA_AT, NEXT_STAGE, FCUR, FNXT, KB)                                     \
    {                                                                                        \
      wait_and_barrier<2 * LOADS_PER_STAGE>();                                               \
      issue(DMA_AT, a_src, b_src, (KB) + 4, wave);                                           \
      read_frags(NEXT_STAGE, FNXT, wm, wn, lane);                                            \
      mfma_frags(FCUR, acc);                                                                 \
      interleave_reads_with_mfma();                                                          \
    }
    int kb = 0;
    for (; kb + 7 < nk; kb += 4) {
      MOE_DEEP_FULL(a0, s1, f0, f1, kb)
      MOE_DEEP_FULL(a1, s2, f1, f0, kb + 1)
      MOE_DEEP_FULL(a2, s3, f0, f1, kb + 2)
      MOE_DEEP_FULL(a3, s0, f1, f0, kb + 3)
    }
#undef MOE_DEEP_FULL
    // tail: the last steps, with every wait covering all loads in flight
#define MOE_DEEP_TAIL(DMA_AT, NEXT_STAGE, FCUR, FNXT, KB)                                     \
    {                                                                                        \
      const int kb_ = (KB);                                                                  \
      wait_and_barrier<0>();                                                                 \
      if (kb_ + 4 < nk) issue(DMA_AT, a_src, b_src, kb_ + 4, wave);                          \
      if (kb_ + 1 < nk) read_frags(NEXT_STAGE, FNXT, wm, wn, lane);                          \
      mfma_frags(FCUR, acc);                                                                 \
    }
    for (; kb < nk; kb += 4) {
      MOE_DEEP_TAIL(a0, s1, f0, f1, kb)
      if (kb + 1 < nk) MOE_DEEP_TAIL(a1, s2, f1, f0, kb + 1)
      if (kb + 2 < nk) MOE_DEEP_TAIL(a2, s3, f0, f1, kb + 2)
      if (kb + 3 < nk) MOE_DEEP_TAIL(a3, s0, f1, f0, kb + 3)
    }
#undef MOE_DEEP_TAIL
    __syncthreads();

    // Epilogue through LDS: the C tile takes 64 rows per stage.
    int el = lane, ewm = wm, ewn = wn, etid = tid;
    asm volatile("" : "+v"(el), "+v"(etid), "+s"(ewm), "+s"(ewn));
    constexpr int CH = BN / 8;
#define MOE_DEEP_CROW(r)                                                                      \
    (((r) >> 6) == 0 ? s0 : ((r) >> 6) == 1 ? s1 : ((r) >> 6) == 2 ? s2 : s3) + ((r) & 63) * BN
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
            if (EPI == kEpiBiasSilu) o[j] = silu(o[j]);
          }
          uint2 packed;
          packed.x = f32_to_bf16(o[0]) | (static_cast<uint32_t>(f32_to_bf16(o[1])) << 16);
          packed.y = f32_to_bf16(o[2]) | (static_cast<uint32_t>(f32_to_bf16(o[3])) << 16);
          const int p = (nl >> 3) ^ (ml & 31);
          *reinterpret_cast<uint2 *>(MOE_DEEP_CROW(ml) + p * 8 + ((nl >> 2) & 1) * 4) = packed;
        }
      }
    }
    __syncthreads();
    for (int i = etid; i < BM * CH; i += NT) {
      const int r = i / CH, c = i % CH;
      const int64_t row = v.row0 + r;
      const int n = n0 + c * 8;
      if (row < v.rows && n < a.Nout) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t *>(MOE_DEEP_CROW(r) + ((c ^ (r & 31)) << 3));
        *reinterpret_cast<u32x4_t *>(v.C + (v.out_base + row) * a.Nout + n) = val;
      }
    }
#undef MOE_DEEP_CROW
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, register-staged pipeline: 256x256 tiles, four 128x128
// wave tiles, one LDS buffer of one 64-wide K-step.  Global loads run two
// K-steps ahead into registers; each step's fragments (all four 16-wide
// slices) are read from LDS into registers once, so the MFMAs of step kb
// overlap the LDS writes and global loads of the following steps and the
// fragment reads of step kb+1.
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

__device__ __forceinline__ void gload(u32x4_t (&ra)[A_CH], u32x4_t (&rb)[B_CH],
                                      const uint16_t *const (&a_src)[A_CH],
                                      const uint16_t *const (&b_src)[B_CH], int kb) {
#pragma unroll
  for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4_t *>(a_src[i] + kb * BK);
#pragma unroll
  for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4_t *>(b_src[i] + kb * BK);
}

// chunk kc of tile row r at chunk position kc ^ ((r / 2) % 8) of its 128-byte
// row: with 64 four-byte banks serving 16 lanes of 16 bytes at a time, the
// 16 rows read together (same logical chunk) then cover all banks once.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void lstore(uint16_t *tile, const u32x4_t (&ra)[A_CH],
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

// Instruction order of one steady-state step (64 MFMAs): each global load
// and LDS write shares a slot with three MFMAs, then two fragment reads
// precede each of the last sixteen MFMAs.
__device__ __forceinline__ void schedule_step() {
#pragma unroll
  for (int i = 0; i < A_CH + B_CH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
  }
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

template <int EPI, int GM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_rs_kernel(GemmArgs a) {
  using namespace rs;
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[TILE];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int n_groups = a.n_routed + a.n_shared;
  const int total_m = build_tile_prefix<NT, BM>(a, s_pref, s_tmp);
  const int n_nt = (a.Nout + BN - 1) / BN;
  const int total = total_m * n_nt;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int part = (total + kXcds - 1) / kXcds;
  const int begin = xcd * part;
  const int end = min(total, begin + part);
  const int nk = a.K / BK;
  const int kc = tid & 7;

  for (int L = begin + slot; L < end; L += nslots) {
    int mt, nt;
    decode_tile<GM>(L, total_m, n_nt, &mt, &nt);
    const int g = find_group(s_pref, n_groups, mt);
    const TileView<uint16_t> v = tile_view<uint16_t>(a, g, mt - s_pref[g], BM);
    const int n0 = nt * BN;
    const uint16_t *a_src[A_CH];
    const uint16_t *b_src[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      a_src[i] = a_row_ptr(a, v, v.row0 + (tid >> 3) + i * (NT / 8)) + kc * 8;
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int n = n0 + (tid >> 3) + i * (NT / 8);
      if (n >= a.Nout) n = a.Nout - 1;
      b_src[i] = v.W + static_cast<int64_t>(n) * a.K + kc * 8;
    }
    f32x16_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4_t ra[A_CH], rb[B_CH];
    Frags f;
    gload(ra, rb, a_src, b_src, 0);
    lstore(s_tile, ra, rb, tid);
    if (nk > 1) gload(ra, rb, a_src, b_src, 1);
    __syncthreads();
    read_frags(s_tile, f, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
    // steady state (no branches, so each step is one scheduling region)
    int kb = 0;
    for (; kb + 2 < nk; ++kb) {
      lds_barrier();                        // every wave has its fragments of step kb
      lstore(s_tile, ra, rb, tid);          // step kb+1 into LDS
      gload(ra, rb, a_src, b_src, kb + 2);  // step kb+2 into registers
      mfma_all(f, acc);                     // step kb
      lds_barrier();                        // step kb+1 is in LDS
      read_frags(s_tile, f, wm, wn, lane);
      schedule_step();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kb + 1 < nk) {                      // step nk-2: nothing left to load
      lds_barrier();
      lstore(s_tile, ra, rb, tid);
      mfma_all(f, acc);
      lds_barrier();
      read_frags(s_tile, f, wm, wn, lane);
    }
    mfma_all(f, acc);                       // last step
    __syncthreads();

    // Epilogue through LDS in two passes of 128 rows (the tile buffer holds
    // 128 x 256 bf16): in pass p every wave stores its row blocks mi = 2p,
    // 2p+1, so all four waves work in both passes.
    int el = lane, ewm = wm, ewn = wn, etid = tid;
    asm volatile("" : "+v"(el), "+v"(etid), "+s"(ewm), "+s"(ewn));
    constexpr int CH = BN / 8;
    static_assert(TILE >= 128 * BN, "128 C-tile rows must fit");
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
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
          for (int mm = 0; mm < 2; ++mm) {
            const int mi = pass * 2 + mm;
            const int ml = ewm * 64 + mm * 32 + (el & 31);   // row within the pass
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              o[j] = acc[ni][mi][q * 4 + j] + bv[j];
              if (EPI == kEpiBiasSilu) o[j] = silu_fast(o[j]);
            }
            uint2 packed;
            packed.x = f32_to_bf16(o[0]) | (static_cast<uint32_t>(f32_to_bf16(o[1])) << 16);
            packed.y = f32_to_bf16(o[2]) | (static_cast<uint32_t>(f32_to_bf16(o[3])) << 16);
            const int p = (nl >> 3) ^ (ml & 31);
            *reinterpret_cast<uint2 *>(s_tile + ml * BN + p * 8 + ((nl >> 2) & 1) * 4) = packed;
          }
        }
      }
      __syncthreads();
      // LDS row ml of the pass is tile row (ml/64)*128 + pass*64 + ml%64
      for (int i = etid; i < 128 * CH; i += NT) {
        const int r = i / CH, c = i % CH;
        const int64_t row = v.row0 + (r >> 6) * 128 + pass * 64 + (r & 63);
        const int n = n0 + c * 8;
        if (row < v.rows && n < a.Nout) {
          const u32x4_t val = *reinterpret_cast<const u32x4_t *>(s_tile + r * BN + ((c ^ (r & 31)) << 3));
          *reinterpret_cast<u32x4_t *>(v.C + (v.out_base + row) * a.Nout + n) = val;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel (also accepts bf16 operands): 64x64 tiles, 256 threads
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

template <int BM, int BN, int WM, int WN, int GM>
hipError_t launch_bf16(const GemmArgs &a, const GemmGroups &g, Epilogue epi, int per_cu,
                       hipStream_t s) {
  const unsigned grid = persistent_grid(tiles_upper_bound(g, BM, BN), per_cu);
  const dim3 block(WM * WN * 64);
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, WM, WN, kEpiBiasSilu, GM>), dim3(grid),
                       block, 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, WM, WN, kEpiBias, GM>), dim3(grid),
                       block, 0, s, a);
  return hipGetLastError();
}

template <int GM>
hipError_t launch_bf16_deep(const GemmArgs &a, const GemmGroups &g, Epilogue epi, hipStream_t s) {
  const unsigned grid = persistent_grid(tiles_upper_bound(g, 256, 256), 1);
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((grouped_gemm_bf16_deep_kernel<kEpiBiasSilu, GM>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_deep_kernel<kEpiBias, GM>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int GM>
hipError_t launch_bf16_rs(const GemmArgs &a, const GemmGroups &g, Epilogue epi, hipStream_t s) {
  const unsigned grid = persistent_grid(tiles_upper_bound(g, 256, 256), 1);
  if (epi == kEpiBiasSilu)
    hipLaunchKernelGGL((grouped_gemm_bf16_rs_kernel<kEpiBiasSilu, GM>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_rs_kernel<kEpiBias, GM>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(bool bf16, const GemmGroups &g, Epilogue epi, hipStream_t s) {
  const GemmArgs a = make_args(g);
  if (g.n_routed + g.n_shared <= 0 || g.Nout <= 0) return hipSuccess;
  if (bf16 && g.K % 64 == 0 && g.Nout % 4 == 0) {
    // rows per routed group decide the tile: few rows -> stream weights with a
    // short M tile; many rows -> square tiles for operand reuse
    const int64_t groups = g.n_routed > 0 ? g.n_routed : 1;
    const int64_t mean_rows = g.max_routed_rows / groups;
    if (mean_rows <= 48 && g.T_sh <= 256)
      return launch_bf16<32, 128, 1, 4, 8>(a, g, epi, 2, s);
    if (mean_rows >= 384) return launch_bf16_rs<8>(a, g, epi, s);
    return launch_bf16<128, 128, 2, 2, 8>(a, g, epi, 2, s);
  }
  const unsigned grid = persistent_grid(tiles_upper_bound(g, 64, 64), 4);
  if (bf16) {
    if (epi == kEpiBiasSilu)
      hipLaunchKernelGGL((grouped_gemm_valu_kernel<uint16_t, kEpiBiasSilu>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((grouped_gemm_valu_kernel<uint16_t, kEpiBias>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (epi == kEpiBiasSilu)
      hipLaunchKernelGGL((grouped_gemm_valu_kernel<float, kEpiBiasSilu>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((grouped_gemm_valu_kernel<float, kEpiBias>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
