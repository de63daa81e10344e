/*
 * moe_mi355x.h — C interface of the sparse top-K routed MoE FFN forward
 * (renormalised gates, optional always-on shared experts) for MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [TopK]  "Sparse MoE Top-Kルーティング" glossary page (jisaku.com):
 *           section ルーティングの仕組み (router scores for every expert, keep
 *           the K best, masked re-softmax gives the gates, gate-weighted sum);
 *           section 解決策2: エキスパートキャパシティファクター (per-expert token
 *           limit, overflow tokens dropped / left to the residual).
 *   [DSMoE] "論文解説: DeepSeekMoE — 細粒度エキスパート分割と共有エキスパートによる
 *           MoE効率化" (0h-n0.github.io): section 共有エキスパート機構 (output
 *           equation: sum of shared experts plus gate-weighted routed experts);
 *           section ルーティングとバランス損失 (gate equation
 *           g_j = s_j / sum_{k in TopK} s_k, s = softmax(W_r x)); section
 *           アルゴリズム (layer arguments d_model, n_routed, n_shared, top_k,
 *           d_ff; router Linear without bias; expert Linear-SiLU-Linear).
 *   [EP]    "エキスパート並列（Expert Parallelism）" glossary page (jisaku.com):
 *           section 推論フロー (gate selects experts, tokens are sent to their
 *           experts, results are sent back); on one GPU that exchange is the
 *           on-device permutation below.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument of type void*, float*, int32_t* that names a
 *     tensor is a DEVICE pointer owned by the caller; the library allocates
 *     nothing and keeps no state between calls.  `cfg` and `w` (the structs)
 *     are HOST pointers read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it; none synchronises with the host and none
 *     copies device data to the host.  Results are ready when the stream is.
 *   - Tensors are dense and row-major in the shapes given; "act" denotes the
 *     activation / expert-weight type chosen by cfg->dtype (MOE_F32: float,
 *     MOE_BF16: bfloat16 bits).  Router weights, router bias, logits and
 *     gates are always float32.  Every device pointer must be 16-byte aligned.
 *   - Return value: MOE_OK, or a negative moe_status.  Argument errors are
 *     detected on the host before anything is enqueued.  Launch failures
 *     return MOE_ERR_HIP.  Device-side contents (for example an expert index
 *     outside [0, N) handed to moe_permute) are not validated; behaviour is
 *     then undefined.  No C++ exception crosses this interface.
 *   - T == 0 is a successful no-op.
 *   - Supported sizes: 1 <= top_k <= n_routed (top_k > n_routed or
 *     top_k < 1 is MOE_ERR_INVALID_ARG); n_routed <= 1024 and top_k <= 64
 *     (the top-K kernel keeps slot k of a token in lane k of one 64-wide
 *     wave, and the combine stages a token's slot rows in 64 entries);
 *     n_shared <= 64; d_model and d_ff multiples of 64 for MOE_BF16 (one
 *     64-element reduction step of the matrix-core kernels, 128 bytes) and of
 *     16 for MOE_F32; T * top_k < 2^31.  Sizes outside these limits return
 *     MOE_ERR_UNSUPPORTED.
 *
 * Numerical contract
 *   - Logits: float32, per (t, e) one fused multiply-add chain over k
 *     ascending starting at +0, then + router_bias[e] with one rounding
 *     (with MOE_BIAS_SELECTION_ONLY the bias is added to the selection key
 *     only).
 *   - Selection: the K largest logits, key (logit desc, expert id asc); slot
 *     k of a token holds its k-th best expert.
 *   - Gates: softmax over the K kept logits (float32), which equals
 *     s_j / sum_{k in TopK} s_k of [DSMoE] gate equation.
 *   - Capacity: C = cfg->capacity when >= 0, else ceil(cf * T * K / N)
 *     evaluated in double as ((cf * T) * K) / N when cf > 0, else no limit.
 *     An expert keeps its first C tokens in token order; a dropped
 *     (token, slot) contributes nothing; gates are not renormalised again.
 *   - Output: y_t = sum_i S_i(x_t) + sum_{k kept} g[t,k] * E_{idx[t,k]}(x_t),
 *     accumulated in float32, shared experts first, then k ascending; no
 *     residual term (that add belongs to the caller).
 *   - Expert E(z) = W2 SiLU(W1 z + b1) + b2; bf16 configurations round the
 *     hidden activations and the expert outputs to bf16, accumulate in fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* NULL where required, negative size, K > N ... */
    MOE_ERR_UNSUPPORTED = -2,   /* sizes outside the supported ranges above      */
    MOE_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required    */
    MOE_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed    */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape ([DSMoE] アルゴリズム: d_model, n_routed, n_shared, top_k, d_ff). */
typedef struct {
    int64_t T;                /* tokens (batch * seq_len, flattened)              */
    int32_t d_model;          /* d                                                 */
    int32_t n_routed;         /* N routed experts                                  */
    int32_t top_k;            /* K experts kept per token                          */
    int32_t n_shared;         /* K_s always-active shared experts (may be 0)       */
    int32_t d_ff;             /* f, hidden width of every expert                   */
    int32_t dtype;            /* moe_dtype of x, expert weights/biases, hidden, y  */
    float capacity_factor;    /* <= 0: no factor-derived limit                     */
    int32_t capacity;         /* >= 0: explicit per-expert limit; -1: use factor   */
    int32_t bias_mode;        /* MOE_BIAS_IN_LOGIT or MOE_BIAS_SELECTION_ONLY      */
    int32_t dispatch;         /* MOE_DISPATCH_BF16 or MOE_DISPATCH_FP8             */
} moe_config;

/* Precision of the token rows the routed experts receive (the dispatch).
 *   MOE_DISPATCH_BF16: the rows as given (act dtype).
 *   MOE_DISPATCH_FP8: the FP8 dispatch of [DeepEP] ("DeepEP とは？" item 5;
 *     "DeepEP の性能": FP8 dispatch, BF16 combine).  Each token row is sent as
 *     OCP FP8 E4M3 codes (bias 7, 3 mantissa bits, largest value 448) with one
 *     power-of-two scale 2^E per row, E the smallest integer with
 *     max|x[t]| <= 448 * 2^E (0 for an all-zero row); codes are x / 2^E
 *     rounded to nearest, ties to even.  The pass that makes the codes (the
 *     payload an exchange between GPUs would carry) also widens them back,
 *     as the receiving side would, to bf16 rows of exactly 2^E * code value,
 *     and the routed experts' first Linear reads those rows through the
 *     dispatch permutation; the router and the shared experts use x; the
 *     combine is unchanged (bf16).  MOE_BF16 layers only
 *     (MOE_ERR_UNSUPPORTED otherwise); honoured by moe_layer_forward and
 *     moe_layer_forward_noalloc, ignored by the other entry points. */
enum { MOE_DISPATCH_BF16 = 0, MOE_DISPATCH_FP8 = 1 };

/* How router_bias enters the routing.
 *   MOE_BIAS_IN_LOGIT: the bias is part of the logit, for selection and gates.
 *   MOE_BIAS_SELECTION_ONLY: the bias-based balancing of [TopK] section
 *     負荷均衡 (steers the load without changing the loss): selection uses the
 *     key fl32(logit + bias[e]); the gates are the softmax over the K kept
 *     unbiased logits, and the logits written are the unbiased ones. */
enum { MOE_BIAS_IN_LOGIT = 0, MOE_BIAS_SELECTION_ONLY = 1 };

/* Expert and router weights, nn.Linear layout (out_features, in_features). */
typedef struct {
    const float *w_router;    /* [N][d] float32                                   */
    const float *router_bias; /* [N] float32 or NULL                              */
    const void *w1;           /* [N][f][d] act                                    */
    const void *b1;           /* [N][f] act or NULL                               */
    const void *w2;           /* [N][d][f] act                                    */
    const void *b2;           /* [N][d] act or NULL                               */
    const void *ws1;          /* [K_s][f][d] act (NULL when K_s == 0)             */
    const void *bs1;          /* [K_s][f] act or NULL                             */
    const void *ws2;          /* [K_s][d][f] act (NULL when K_s == 0)             */
    const void *bs2;          /* [K_s][d] act or NULL                             */
} moe_weights;

/*
 * moe_route — router scores, top-K selection and renormalised gates
 * ([TopK] ルーティングの仕組み; [DSMoE] gate equation).
 *   x           [T][d] act
 *   w_router    [N][d] float32;  router_bias [N] float32 or NULL (part of the
 *               logit for both selection and gates)
 *   logits      [T][N] float32 output, required: the top-K pass reads the
 *               logits back from here.  The logits of one token are computed
 *               by many workgroups (one logit per lane, each a d-long fixed
 *               order chain), so no single workgroup holds a token's N
 *               logits on chip; a pass that did would serialise N/64 of those
 *               chains per wave, far slower than this T*N*4-byte round trip
 *               (4 MB, under a microsecond of HBM time, at 4096 tokens and
 *               256 experts).
 *   topk_idx    [T][K] int32 output, expert ids in slot order
 *   topk_gate   [T][K] float32 output, sums to 1 per token
 */
int moe_route(const moe_config *cfg, const void *x, const float *w_router,
              const float *router_bias, float *logits, int32_t *topk_idx,
              float *topk_gate, void *stream);

/*
 * moe_permute — dispatch as an on-device permutation: per-expert histogram,
 * capacity clip, exclusive scan, stable scatter ([EP] 推論フロー steps 2-3 on
 * one GPU; [TopK] capacity section).
 *   topk_idx    [T][K] int32 input, values in [0, N)
 *   x           [T][d] act input, read only when x_perm != NULL
 *   counts      [N] int32 output: kept rows per expert
 *   offsets     [N+1] int32 output: exclusive scan of counts
 *   row_token   [T*K] int32 output: rows 0..offsets[N]-1 hold the token of
 *               each row, experts in order, tokens ascending within one
 *   slot_row    [T*K] int32 output: row of (t, k), or -1 when dropped
 *   n_dropped   [1] int32 output
 *   x_perm      [T*K][d] act output (rows 0..offsets[N]-1) or NULL to skip
 *   ws          device workspace of moe_permute_workspace_size(cfg) bytes
 */
int moe_permute(const moe_config *cfg, const int32_t *topk_idx, const void *x,
                int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *slot_row,
                int32_t *n_dropped, void *x_perm, void *ws, size_t ws_bytes, void *stream);
size_t moe_permute_workspace_size(const moe_config *cfg);

/*
 * moe_grouped_ffn — every group's expert FFN over its contiguous rows:
 * rows offsets[g] .. offsets[g+1]-1 get E_g(x_rows[r]) ([DSMoE] アルゴリズム,
 * expert Linear(d, f) - SiLU - Linear(f, d)).
 *   n_groups    number of experts in w1/w2 (>= 1)
 *   x_rows      [max_rows][d] act input
 *   offsets     [n_groups+1] int32 DEVICE array, non-decreasing, offsets[0]=0
 *   max_rows    host-side upper bound on offsets[n_groups].  The offsets
 *               stay on the device (no call copies them back), so the host
 *               sizes the persistent launch and the split scratch from this
 *               bound; the kernels read the true row counts on the device.
 *               Rows at or beyond offsets[n_groups] are neither read nor
 *               written; offsets[n_groups] > max_rows is undefined.
 *   w1 [G][f][d], b1 [G][f] or NULL, w2 [G][d][f], b2 [G][d] or NULL (act)
 *   h           [max_rows][f] act output (hidden activations)
 *   y_rows      [max_rows][d] act output
 *   ws          optional device scratch of moe_grouped_ffn_workspace_size
 *               bytes (NULL allowed); with it, products with too few row
 *               blocks to fill the GPU are split along their reduction
 *               dimension and the parts summed in a fixed order.  A non-NULL
 *               ws smaller than that size is MOE_ERR_WORKSPACE.
 * Only cfg->d_model, cfg->d_ff and cfg->dtype are read.
 */
int moe_grouped_ffn(const moe_config *cfg, int32_t n_groups, const void *x_rows,
                    const int32_t *offsets, int64_t max_rows, const void *w1, const void *b1,
                    const void *w2, const void *b2, void *h, void *y_rows, void *ws,
                    size_t ws_bytes, void *stream);
size_t moe_grouped_ffn_workspace_size(const moe_config *cfg, int32_t n_groups,
                                      int64_t max_rows);

/*
 * moe_combine — y_t = sum_i S_i[t] + sum_{k: slot_row[t,k] >= 0}
 * g[t,k] * y_rows[slot_row[t,k]] ([DSMoE] 共有エキスパート機構 equation).
 *   y_rows      [*][d] act, indexed by slot_row
 *   slot_row    [T][K] int32, topk_gate [T][K] float32
 *   shared_out  [K_s][T][d] act or NULL (K_s from cfg->n_shared)
 *   y           [T][d] act output
 */
int moe_combine(const moe_config *cfg, const void *y_rows, const int32_t *slot_row,
                const float *topk_gate, const void *shared_out, void *y, void *stream);

/*
 * moe_layer_forward — the whole layer of [DSMoE] 共有エキスパート機構 (output
 * equation: the shared experts' sum plus the gate-weighted routed experts),
 * with the routing of [TopK] ルーティングの仕組み and [DSMoE] gate equation and
 * the capacity limit of [TopK] 解決策2: route, permute (the gather is fused
 * into the first expert GEMM), routed and shared expert FFNs, combine.
 *   x [T][d] act input, y [T][d] act output.
 *   topk_idx, topk_gate ([T][K]) and counts ([N]) are optional outputs of the
 *   routing (NULL to skip).  When one is given, the layer writes that array
 *   there instead of into its workspace region.
 *   ws          device workspace of moe_workspace_size(cfg) bytes.  After the
 *               call has run on the stream, the regions named by
 *               moe_workspace_layout hold the layer's routing: logits,
 *               offsets, n_dropped, row_token and slot_row always, and
 *               topk_idx, topk_gate and counts when their optional output is
 *               NULL.  The rest of ws is scratch.
 */
int moe_layer_forward(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                      int32_t *topk_idx, float *topk_gate, int32_t *counts,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_forward_noalloc — moe_layer_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same stages and kernels, with the
 * workspace taken from a library-owned device array instead of `ws`.
 *   - The array holds MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, from the
 *     first use of the library on that GPU until the process ends.  The
 *     call allocates nothing (no hipMalloc, hipFree or allocating library
 *     routine); its first call on a device looks up the array's address there.
 *   - A layer whose workspace, without the expert GEMMs' optional K-split
 *     scratch, exceeds that size returns MOE_ERR_WORKSPACE before anything is
 *     enqueued.  The K-split scratch gets what is left (a DeepSeek-V3-shaped
 *     decode layer of 128 tokens needs about 22 MB plus 32 MB of it); with
 *     less, fewer products are split.  Batches of a few hundred tokens at
 *     DeepSeek-V3 widths fit; 4096-token prefill layers do not.
 *   - Every call on one GPU uses that GPU's one array.  Calls that overlap on
 *     one GPU (on different streams, or from several host threads without
 *     ordering) race and give undefined results; calls on one stream are
 *     ordered and safe.  Each call writes every part of the array it later
 *     reads, so nothing left by an earlier call is used.
 *   Arguments as moe_layer_forward; the routing arrays are not readable
 *   through moe_workspace_layout here (pass topk_idx, topk_gate, counts).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                              void *y, int32_t *topk_idx, float *topk_gate, int32_t *counts,
                              void *stream);

/* Bytes of device workspace moe_layer_forward needs for cfg (0 when cfg is
 * invalid or unsupported). */
size_t moe_workspace_size(const moe_config *cfg);

/* Byte offsets, from the start of moe_layer_forward's workspace, of the
 * routing arrays the layer leaves there (shapes as in moe_permute; every
 * offset is a multiple of 256). */
typedef struct {
    size_t logits;      /* [T][N] float32                                     */
    size_t topk_idx;    /* [T][K] int32                                       */
    size_t topk_gate;   /* [T][K] float32                                     */
    size_t counts;      /* [N] int32: kept rows per expert                    */
    size_t offsets;     /* [N+1] int32                                        */
    size_t n_dropped;   /* [1] int32                                          */
    size_t row_token;   /* [T*K] int32 (rows 0 .. offsets[N]-1 hold tokens)   */
    size_t slot_row;    /* [T][K] int32 (-1 = dropped)                        */
    size_t x_fp8;       /* MOE_DISPATCH_FP8: [T][d] uint8 E4M3 codes, else 0  */
    size_t x_fp8_exp;   /* MOE_DISPATCH_FP8: [T] int32 scale exponents, else 0 */
    size_t x_fp8_wide;  /* MOE_DISPATCH_FP8: [T][d] bf16, the codes widened back
                           (2^E times each code's value: the rows the first
                           Linear reads), else 0                             */
    size_t total;       /* moe_workspace_size(cfg)                            */
} moe_ws_layout;

/* Fills *out for cfg; MOE_OK, or the status moe_layer_forward would return
 * for cfg's shape. */
int moe_workspace_layout(const moe_config *cfg, moe_ws_layout *out);

/* Stages of moe_layer_forward, in launch order. */
enum {
    MOE_STAGE_ROUTER = 0,   /* router logits                                   */
    MOE_STAGE_TOPK = 1,     /* top-K selection and gates                       */
    MOE_STAGE_DISPATCH = 2, /* histogram, scan, scatter                        */
    MOE_STAGE_UP = 3,       /* first Linear + SiLU, routed and shared experts  */
    MOE_STAGE_DOWN = 4,     /* second Linear, routed and shared experts        */
    MOE_STAGE_COMBINE = 5,  /* gate-weighted sum + shared outputs              */
    MOE_STAGE_COUNT = 6
};

/*
 * moe_layer_forward_events — moe_layer_forward that also records caller-owned
 * HIP events on `stream` at every stage boundary, for timing the stages on the
 * stream they run on.  stage_events points to MOE_STAGE_COUNT + 1 hipEvent_t
 * handles (as void*): event i is recorded just before stage i is launched and
 * event MOE_STAGE_COUNT after the last one.  NULL behaves like
 * moe_layer_forward.  The events are only recorded, never waited on.
 */
int moe_layer_forward_events(const moe_config *cfg, const moe_weights *w, const void *x,
                             void *y, int32_t *topk_idx, float *topk_gate, int32_t *counts,
                             void *ws, size_t ws_bytes, void *const *stage_events,
                             void *stream);

/*
 * moe_balance_stats — load statistics of one routing ([DSMoE] section
 * ルーティングとバランス損失, balance-loss equation):
 *   f[j]  = (number of (t, k) with topk_idx[t][k] == j) / (T * K)
 *   P[j]  = (1/T) * sum_t softmax(logits[t])_j   (softmax over all N)
 *   *loss = alpha * N * sum_j f[j] * P[j]
 *   logits      [T][N] float32 (as written by moe_route)
 *   topk_idx    [T][K] int32, values in [0, N)
 *   f, P        [N] float32 outputs; loss [1] float32 output (device)
 *   ws          device workspace of moe_balance_stats_workspace_size(cfg) bytes
 * Counts are exact; P and the loss are float32 sums in a fixed order, so the
 * results do not depend on timing.  Only T, n_routed and top_k are read.
 */
int moe_balance_stats(const moe_config *cfg, const float *logits, const int32_t *topk_idx,
                      float alpha, float *f, float *P, float *loss, void *ws, size_t ws_bytes,
                      void *stream);
size_t moe_balance_stats_workspace_size(const moe_config *cfg);

/* Per-expert capacity the library applies for cfg (-1 = unlimited). */
int64_t moe_capacity(const moe_config *cfg);

/* Static text for a moe_status value. */
const char *moe_status_string(int status);

/* Interface version, 0x00MMmmpp: the library returns MOE_VERSION of the
 * header it was built with; a caller built against another version should not
 * use it (struct layouts may differ). */
#define MOE_VERSION 0x000200
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
