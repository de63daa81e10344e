// Host side of the C interface declared in include/moe_mi355x.h: argument
// validation, workspace layout and kernel launches on the caller's stream.
// No call allocates device memory, synchronises, or copies device data back.
#include <math.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "moe_common.h"
#include "moe_mi355x.h"

namespace {

using moe::GemmGroups;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t b) { return (b + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every device pointer the header declares must be 16-byte aligned (the
// kernels read operands as 16-byte vectors, biases as 8-byte pairs); NULL
// passes here and is checked where it is not allowed.
bool all_aligned16(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

size_t act_bytes(const moe_config *c) { return c->dtype == MOE_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.  `need_route` adds the routing
// limits (N, K); `need_ffn` adds the expert widths.
int check_config(const moe_config *c, bool need_route, bool need_ffn) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d_model <= 0) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  const int mult = c->dtype == MOE_BF16 ? 64 : 16;
  if (c->d_model % mult != 0) return MOE_ERR_UNSUPPORTED;
  if (need_route) {
    if (c->n_routed <= 0 || c->top_k <= 0 || c->top_k > c->n_routed) return MOE_ERR_INVALID_ARG;
    if (c->n_routed > moe::kMaxRouted || c->top_k > 64) return MOE_ERR_UNSUPPORTED;
    if (c->T * static_cast<int64_t>(c->top_k) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    if (c->capacity < -1) return MOE_ERR_INVALID_ARG;
    if (c->bias_mode != MOE_BIAS_IN_LOGIT && c->bias_mode != MOE_BIAS_SELECTION_ONLY)
      return MOE_ERR_INVALID_ARG;
  }
  if (c->dispatch != MOE_DISPATCH_BF16 && c->dispatch != MOE_DISPATCH_FP8)
    return MOE_ERR_INVALID_ARG;
  if (c->dispatch == MOE_DISPATCH_FP8 && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (need_ffn) {
    if (c->d_ff <= 0) return MOE_ERR_INVALID_ARG;
    if (c->d_ff % mult != 0) return MOE_ERR_UNSUPPORTED;
    if (c->n_shared < 0) return MOE_ERR_INVALID_ARG;
    if (c->n_shared > moe::kMaxShared) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int64_t capacity_of(const moe_config *c) {
  if (c->capacity >= 0) return c->capacity;
  if (!(c->capacity_factor > 0.0f)) return -1;
  const double v = static_cast<double>(c->capacity_factor) * static_cast<double>(c->T) *
                   static_cast<double>(c->top_k) / static_cast<double>(c->n_routed);
  return static_cast<int64_t>(ceil(v));
}

// Workspace of the whole layer, carved in this order (each piece 256-aligned).
struct LayerWs {
  float *logits;
  int32_t *idx;
  float *gates;
  int32_t *counts;
  int32_t *offsets;
  int32_t *n_dropped;
  int32_t *row_token;
  int32_t *slot_row;
  void *dispatch_ws;
  void *h;       // routed hidden [T*K][f]
  void *h_sh;    // shared hidden [Ks][T][f]
  void *y_rows;  // routed outputs [T*K][d]
  void *s_out;   // shared outputs [Ks][T][d]
  void *split;   // k-split scratch of the expert GEMMs (may be empty)
  size_t split_bytes;
  uint8_t *xq;     // FP8 dispatch: E4M3 codes [T][d] (else null)
  int32_t *xexp;   // FP8 dispatch: scale exponents [T] (else null)
  void *xw;        // FP8 dispatch: the codes widened back to bf16 [T][d] (else null)
  size_t bytes;
};

// Row bounds the dispatch guarantees: a routed group holds at most T rows
// (a token meets an expert once) and at most C; all groups at most T*K and
// N*C rows together.
int64_t routed_rows_bound(const moe_config *c) {
  const int64_t C = capacity_of(c);
  const int64_t tk = c->T * c->top_k;
  return C >= 0 && C * c->n_routed < tk ? C * c->n_routed : tk;
}
int64_t group_rows_bound(const moe_config *c) {
  const int64_t C = capacity_of(c);
  return C >= 0 && C < c->T ? C : c->T;
}

// Split scratch the layer's two expert GEMMs may use (shared by both).
size_t layer_split_bytes(const moe_config *c) {
  if (c->dtype != MOE_BF16) return 0;
  GemmGroups g{};
  g.n_routed = c->n_routed;
  g.n_shared = c->n_shared;
  g.T_sh = c->T;
  g.max_routed_rows = routed_rows_bound(c);
  g.Nout = c->d_ff > c->d_model ? c->d_ff : c->d_model;
  return moe::grouped_gemm_split_bytes(g);
}

// The layer's workspace carved from base (NULL: sizes only).  The K-split
// scratch of the expert GEMMs is the last piece, at most split_cap bytes:
// with less than they could use, the GEMMs split fewer products (same
// results within the tolerance, possibly slower).
LayerWs layer_ws(const moe_config *c, void *base, size_t split_cap = SIZE_MAX) {
  LayerWs w;
  char *p = static_cast<char *>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char *q = p ? p + off : nullptr;
    off += align_up(b);
    return static_cast<void *>(q);
  };
  const int64_t T = c->T, K = c->top_k, N = c->n_routed, Ks = c->n_shared;
  const size_t ab = act_bytes(c);
  w.logits = static_cast<float *>(take(sizeof(float) * T * N));
  w.idx = static_cast<int32_t *>(take(sizeof(int32_t) * T * K));
  w.gates = static_cast<float *>(take(sizeof(float) * T * K));
  w.counts = static_cast<int32_t *>(take(sizeof(int32_t) * N));
  w.offsets = static_cast<int32_t *>(take(sizeof(int32_t) * (N + 1)));
  w.n_dropped = static_cast<int32_t *>(take(sizeof(int32_t)));
  w.row_token = static_cast<int32_t *>(take(sizeof(int32_t) * T * K));
  w.slot_row = static_cast<int32_t *>(take(sizeof(int32_t) * T * K));
  w.dispatch_ws = take(moe::dispatch_workspace_bytes(T, static_cast<int>(K), static_cast<int>(N)));
  w.h = take(ab * T * K * c->d_ff);
  w.h_sh = take(ab * Ks * T * c->d_ff);
  w.y_rows = take(ab * T * K * c->d_model);
  w.s_out = take(ab * Ks * T * c->d_model);
  const bool fp8 = c->dispatch == MOE_DISPATCH_FP8;
  w.xq = fp8 ? static_cast<uint8_t *>(take(static_cast<size_t>(T) * c->d_model)) : nullptr;
  w.xexp = fp8 ? static_cast<int32_t *>(take(sizeof(int32_t) * T)) : nullptr;
  w.xw = fp8 ? take(ab * T * c->d_model) : nullptr;
  size_t sb = layer_split_bytes(c);
  if (sb > split_cap) sb = split_cap & ~(kAlign - 1);
  w.split = sb ? take(sb) : nullptr;
  w.split_bytes = sb;
  w.bytes = off;
  return w;
}

// Pointer checks of the layer entry points (after check_config).
int check_layer_args(const moe_weights *w, const moe_config *cfg, const void *x, const void *y,
                     const int32_t *topk_idx, const float *topk_gate, const int32_t *counts) {
  if (!x || !y || !w->w_router || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > 0 && (!w->ws1 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({x, y, w->w_router, w->router_bias, w->w1, w->b1, w->w2, w->b2, w->ws1,
                      w->bs1, w->ws2, w->bs2, topk_idx, topk_gate, counts}))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int run_layer(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
              int32_t *topk_idx, float *topk_gate, int32_t *counts, const LayerWs &L,
              void *const *stage_events, hipStream_t s);

}  // namespace

// Workspace of moe_layer_forward_noalloc: a file-scope device array, so
// that entry point needs no allocation.  Every GPU the library runs on gets
// its own copy when the code object is loaded there, held until the process
// ends.  In host code `scratch` is only a handle: its device address is
// looked up once per device (noalloc_scratch) and used everywhere instead.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's `scratch`, found with the device current
// on the first call there and kept per device.
int noalloc_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_version(void) { return MOE_VERSION; }

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t moe_capacity(const moe_config *cfg) {
  if (!cfg || cfg->n_routed <= 0) return -1;
  return capacity_of(cfg);
}

int moe_route(const moe_config *cfg, const void *x, const float *w_router,
              const float *router_bias, float *logits, int32_t *topk_idx, float *topk_gate,
              void *stream) {
  int st = check_config(cfg, true, false);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !w_router || !logits || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({x, w_router, router_bias, logits, topk_idx, topk_gate}))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = cfg->dtype == MOE_BF16;
  const bool sel_only = cfg->bias_mode == MOE_BIAS_SELECTION_ONLY;
  st = hip_status(moe::launch_router_logits(bf16, x, w_router, sel_only ? nullptr : router_bias,
                                            logits, cfg->T, cfg->d_model, cfg->n_routed, s));
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_topk_gates(logits, sel_only ? router_bias : nullptr, cfg->T,
                                           cfg->n_routed, cfg->top_k, topk_idx, topk_gate, s));
}

size_t moe_balance_stats_workspace_size(const moe_config *cfg) {
  if (check_config(cfg, true, false) != MOE_OK) return 0;
  return moe::balance_workspace_bytes(cfg->T, cfg->n_routed);
}

int moe_balance_stats(const moe_config *cfg, const float *logits, const int32_t *topk_idx,
                      float alpha, float *f, float *P, float *loss, void *ws, size_t ws_bytes,
                      void *stream) {
  int st = check_config(cfg, true, false);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!logits || !topk_idx || !f || !P || !loss) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({logits, topk_idx, f, P, loss, ws})) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe::balance_workspace_bytes(cfg->T, cfg->n_routed))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_balance_stats(logits, topk_idx, cfg->T, cfg->n_routed,
                                              cfg->top_k, alpha, f, P, loss, ws,
                                              static_cast<hipStream_t>(stream)));
}

size_t moe_permute_workspace_size(const moe_config *cfg) {
  if (check_config(cfg, true, false) != MOE_OK) return 0;
  return moe::dispatch_workspace_bytes(cfg->T, cfg->top_k, cfg->n_routed);
}

int moe_permute(const moe_config *cfg, const int32_t *topk_idx, const void *x, int32_t *counts,
                int32_t *offsets, int32_t *row_token, int32_t *slot_row, int32_t *n_dropped,
                void *x_perm, void *ws, size_t ws_bytes, void *stream) {
  int st = check_config(cfg, true, false);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !row_token || !slot_row || !n_dropped)
    return MOE_ERR_INVALID_ARG;
  if (x_perm && !x) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({topk_idx, counts, offsets, row_token, slot_row, n_dropped, ws,
                      x_perm ? x : nullptr, x_perm}))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::dispatch_workspace_bytes(cfg->T, cfg->top_k, cfg->n_routed);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(moe::launch_dispatch(topk_idx, cfg->T, cfg->top_k, cfg->n_routed,
                                       capacity_of(cfg), counts, offsets, row_token, slot_row,
                                       n_dropped, ws, s));
  if (st != MOE_OK || !x_perm) return st;
  return hip_status(moe::launch_gather_rows(cfg->dtype == MOE_BF16, x, row_token,
                                            offsets + cfg->n_routed, cfg->T * cfg->top_k,
                                            cfg->d_model, x_perm, s));
}

size_t moe_grouped_ffn_workspace_size(const moe_config *cfg, int32_t n_groups, int64_t max_rows) {
  if (check_config(cfg, false, true) != MOE_OK || n_groups <= 0 || max_rows < 0) return 0;
  if (cfg->dtype != MOE_BF16) return 0;
  GemmGroups g{};
  g.n_routed = n_groups;
  g.max_routed_rows = max_rows;
  g.Nout = cfg->d_ff > cfg->d_model ? cfg->d_ff : cfg->d_model;
  return moe::grouped_gemm_split_bytes(g);
}

int moe_grouped_ffn(const moe_config *cfg, int32_t n_groups, const void *x_rows,
                    const int32_t *offsets, int64_t max_rows, const void *w1, const void *b1,
                    const void *w2, const void *b2, void *h, void *y_rows, void *ws,
                    size_t ws_bytes, void *stream) {
  int st = check_config(cfg, false, true);
  if (st != MOE_OK) return st;
  if (n_groups <= 0 || max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (n_groups > moe::kMaxRouted + moe::kMaxShared) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  if (max_rows >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!x_rows || !offsets || !w1 || !w2 || !h || !y_rows) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({x_rows, offsets, w1, b1, w2, b2, h, y_rows, ws}))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe_grouped_ffn_workspace_size(cfg, n_groups, max_rows);
  if (ws && ws_bytes < need) return MOE_ERR_WORKSPACE;
  const bool bf16 = cfg->dtype == MOE_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmGroups g{};
  g.offsets = offsets;
  g.n_routed = n_groups;
  g.A = x_rows;
  g.W = w1;
  g.bias = b1;
  g.C = h;
  g.Nout = cfg->d_ff;
  g.K = cfg->d_model;
  g.max_routed_rows = max_rows;
  g.max_group_rows = max_rows;
  g.split_ws = ws && need ? ws : nullptr;
  g.split_bytes = g.split_ws ? need : 0;
  st = hip_status(moe::launch_grouped_gemm(bf16, g, moe::kEpiBiasSilu, s));
  if (st != MOE_OK) return st;
  g.A = h;
  g.W = w2;
  g.bias = b2;
  g.C = y_rows;
  g.Nout = cfg->d_model;
  g.K = cfg->d_ff;
  return hip_status(moe::launch_grouped_gemm(bf16, g, moe::kEpiBias, s));
}

int moe_combine(const moe_config *cfg, const void *y_rows, const int32_t *slot_row,
                const float *topk_gate, const void *shared_out, void *y, void *stream) {
  int st = check_config(cfg, true, false);
  if (st != MOE_OK) return st;
  if (cfg->n_shared < 0) return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > moe::kMaxShared) return MOE_ERR_UNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!y_rows || !slot_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (cfg->n_shared > 0 && !shared_out) return MOE_ERR_INVALID_ARG;
  if (!all_aligned16({y_rows, slot_row, topk_gate, shared_out, y})) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(cfg->dtype == MOE_BF16, y_rows, slot_row, topk_gate,
                                        cfg->n_shared > 0 ? shared_out : nullptr, cfg->n_shared,
                                        cfg->T, cfg->top_k, cfg->d_model, y,
                                        static_cast<hipStream_t>(stream)));
}

size_t moe_workspace_size(const moe_config *cfg) {
  if (check_config(cfg, true, true) != MOE_OK) return 0;
  return layer_ws(cfg, nullptr).bytes;
}

int moe_workspace_layout(const moe_config *cfg, moe_ws_layout *out) {
  const int st = check_config(cfg, true, true);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID_ARG;
  // carve from a base of 256 (not NULL, which the carver reads as "sizes only")
  char *const base = reinterpret_cast<char *>(static_cast<uintptr_t>(kAlign));
  const LayerWs L = layer_ws(cfg, base);
  auto off = [&](const void *p) { return static_cast<size_t>(static_cast<const char *>(p) - base); };
  out->logits = off(L.logits);
  out->topk_idx = off(L.idx);
  out->topk_gate = off(L.gates);
  out->counts = off(L.counts);
  out->offsets = off(L.offsets);
  out->n_dropped = off(L.n_dropped);
  out->row_token = off(L.row_token);
  out->slot_row = off(L.slot_row);
  out->x_fp8 = L.xq ? off(L.xq) : 0;
  out->x_fp8_exp = L.xexp ? off(L.xexp) : 0;
  out->x_fp8_wide = L.xw ? off(L.xw) : 0;
  out->total = L.bytes;
  return MOE_OK;
}

int moe_layer_forward(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                      int32_t *topk_idx, float *topk_gate, int32_t *counts, void *ws,
                      size_t ws_bytes, void *stream) {
  return moe_layer_forward_events(cfg, w, x, y, topk_idx, topk_gate, counts, ws, ws_bytes,
                                  nullptr, stream);
}

int moe_layer_forward_events(const moe_config *cfg, const moe_weights *w, const void *x,
                             void *y, int32_t *topk_idx, float *topk_gate, int32_t *counts,
                             void *ws, size_t ws_bytes, void *const *stage_events,
                             void *stream) {
  int st = check_config(cfg, true, true);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  if ((st = check_layer_args(w, cfg, x, y, topk_idx, topk_gate, counts)) != MOE_OK) return st;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  const LayerWs L = layer_ws(cfg, ws);
  if (!ws || ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  return run_layer(cfg, w, x, y, topk_idx, topk_gate, counts, L, stage_events,
                   static_cast<hipStream_t>(stream));
}

int moe_layer_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                              void *y, int32_t *topk_idx, float *topk_gate, int32_t *counts,
                              void *stream) {
  int st = check_config(cfg, true, true);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  if ((st = check_layer_args(w, cfg, x, y, topk_idx, topk_gate, counts)) != MOE_OK) return st;
  // everything but the K-split scratch must fit; that scratch gets the rest
  const size_t need = layer_ws(cfg, nullptr, 0).bytes;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *base = nullptr;
  if ((st = noalloc_scratch(&base)) != MOE_OK) return st;
  const LayerWs L = layer_ws(cfg, base, MOE_NOALLOC_SCRATCH_BYTES - need);
  if (L.bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;   // not reached
  return run_layer(cfg, w, x, y, topk_idx, topk_gate, counts, L, nullptr,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int run_layer(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
              int32_t *topk_idx, float *topk_gate, int32_t *counts, const LayerWs &L,
              void *const *stage_events, hipStream_t s) {
  int st = MOE_OK;
  const bool bf16 = cfg->dtype == MOE_BF16;
  const int64_t T = cfg->T;
  const int K = cfg->top_k, N = cfg->n_routed, Ks = cfg->n_shared;
  int32_t *idx = topk_idx ? topk_idx : L.idx;
  float *gates = topk_gate ? topk_gate : L.gates;
  int32_t *cnt = counts ? counts : L.counts;
  auto mark = [&](int i) -> int {
    if (!stage_events) return MOE_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s));
  };

  if ((st = mark(MOE_STAGE_ROUTER)) != MOE_OK) return st;
  const bool sel_only = cfg->bias_mode == MOE_BIAS_SELECTION_ONLY;
  st = hip_status(moe::launch_router_logits(bf16, x, w->w_router,
                                            sel_only ? nullptr : w->router_bias, L.logits, T,
                                            cfg->d_model, N, s));
  if (st != MOE_OK) return st;
  if ((st = mark(MOE_STAGE_TOPK)) != MOE_OK) return st;
  st = hip_status(moe::launch_topk_gates(L.logits, sel_only ? w->router_bias : nullptr, T, N, K,
                                         idx, gates, s));
  if (st != MOE_OK) return st;
  if ((st = mark(MOE_STAGE_DISPATCH)) != MOE_OK) return st;
  st = hip_status(moe::launch_dispatch(idx, T, K, N, capacity_of(cfg), cnt, L.offsets,
                                       L.row_token, L.slot_row, L.n_dropped, L.dispatch_ws, s));
  if (st != MOE_OK) return st;

  // First Linear + SiLU: routed rows gather their token's x directly.
  GemmGroups g{};
  g.offsets = L.offsets;
  g.n_routed = N;
  g.A = x;
  g.a_index = L.row_token;
  g.n_shared = Ks;
  g.T_sh = T;
  g.A_sh = x;
  g.a_sh_stride = 0;
  g.W = w->w1;
  g.bias = w->b1;
  g.W_sh = w->ws1;
  g.bias_sh = w->bs1;
  g.C = L.h;
  g.C_sh = L.h_sh;
  g.Nout = cfg->d_ff;
  g.K = cfg->d_model;
  g.max_routed_rows = routed_rows_bound(cfg);
  g.max_group_rows = group_rows_bound(cfg);
  g.split_ws = L.split;
  g.split_bytes = L.split ? L.split_bytes : 0;
  if ((st = mark(MOE_STAGE_UP)) != MOE_OK) return st;
  if (cfg->dispatch == MOE_DISPATCH_FP8) {
    // FP8 dispatch: the token rows go out as E4M3 codes with a per-row scale
    // (L.xq, L.xexp) and arrive widened back to bf16 (L.xw), in one pass; the
    // routed groups read the arrived rows, the shared experts, which are not
    // dispatched, read x, in the same launch
    st = hip_status(moe::launch_quantize_fp8(x, T, cfg->d_model, L.xq, L.xexp, L.xw, s));
    if (st != MOE_OK) return st;
    g.A = L.xw;
  }
  st = hip_status(moe::launch_grouped_gemm(bf16, g, moe::kEpiBiasSilu, s));
  if (st != MOE_OK) return st;

  // Second Linear.
  g.A = L.h;
  g.a_index = nullptr;
  g.A_sh = L.h_sh;
  g.a_sh_stride = T * cfg->d_ff;
  g.W = w->w2;
  g.bias = w->b2;
  g.W_sh = w->ws2;
  g.bias_sh = w->bs2;
  g.C = L.y_rows;
  g.C_sh = L.s_out;
  g.Nout = cfg->d_model;
  g.K = cfg->d_ff;
  if ((st = mark(MOE_STAGE_DOWN)) != MOE_OK) return st;
  st = hip_status(moe::launch_grouped_gemm(bf16, g, moe::kEpiBias, s));
  if (st != MOE_OK) return st;

  if ((st = mark(MOE_STAGE_COMBINE)) != MOE_OK) return st;
  st = hip_status(moe::launch_combine(bf16, L.y_rows, L.slot_row, gates,
                                      Ks > 0 ? L.s_out : nullptr, Ks, T, K, cfg->d_model, y, s));
  if (st != MOE_OK) return st;
  return mark(MOE_STAGE_COUNT);
}

}  // namespace
