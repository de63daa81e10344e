/*
 * Oracle helper: router logits in one fixed float32 order.
 *
 * TEST INFRASTRUCTURE ONLY.  Called by the CPU oracle (oracle/moe_oracle.py);
 * the HIP library neither links nor calls it.
 *
 * What it computes (the router score of the MoE layer: a bias-free linear map
 * of the token embedding, one score per expert, as in the "Sparse MoE Top-K
 * routing" glossary page, section on the routing mechanism, and the DeepSeekMoE
 * explainer page, gate equation s = softmax(W_r x)):
 *
 *     acc = +0.0f
 *     for k = 0 .. d-1:   acc = fmaf(x[t,k], w[e,k], acc)   (one rounding per step)
 *     logit[t,e] = acc               (no bias)
 *     logit[t,e] = acc + bias[e]     (one float32 rounding, when a bias is given)
 *
 * The pages leave the summation order open; this fixed order (k ascending,
 * fused multiply-add, bias last) is the reading both sides implement so that
 * expert selection can be compared bit for bit.
 *
 * fmaf is correctly rounded by the C standard, in scalar or vector form, so the
 * AVX2/FMA variant below produces the same bits as the portable one; only the
 * loop order (experts innermost, over a transposed weight copy) differs, and
 * each logit still sees its terms in ascending k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static void logits_portable(const float *x, const float *wt, const float *bias,
                            int64_t T, int64_t d, int64_t N, float *out) {
    float *acc = (float *)malloc(sizeof(float) * (size_t)N);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < N; ++e) acc[e] = 0.0f;
        for (int64_t k = 0; k < d; ++k) {
            const float xv = x[t * d + k];
            const float *wrow = wt + k * N;
            for (int64_t e = 0; e < N; ++e) acc[e] = fmaf(xv, wrow[e], acc[e]);
        }
        for (int64_t e = 0; e < N; ++e) {
            float v = acc[e];
            if (bias) v = v + bias[e];
            out[t * N + e] = v;
        }
    }
    free(acc);
}

__attribute__((target("avx2,fma")))
static void logits_fma(const float *x, const float *wt, const float *bias,
                       int64_t T, int64_t d, int64_t N, float *out) {
    float *acc = (float *)aligned_alloc(64, sizeof(float) * (size_t)((N + 15) & ~15));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < N; ++e) acc[e] = 0.0f;
        for (int64_t k = 0; k < d; ++k) {
            const float xv = x[t * d + k];
            const float *wrow = wt + k * N;
            for (int64_t e = 0; e < N; ++e) acc[e] = fmaf(xv, wrow[e], acc[e]);
        }
        for (int64_t e = 0; e < N; ++e) {
            float v = acc[e];
            if (bias) v = v + bias[e];
            out[t * N + e] = v;
        }
    }
    free(acc);
}

/* x: [T][d] float32, w: [N][d] float32, bias: [N] or NULL, out: [T][N]. */
int oracle_router_logits(const float *x, const float *w, const float *bias,
                         int64_t T, int64_t d, int64_t N, float *out) {
    if (T < 0 || d < 0 || N <= 0) return -1;
    float *wt = (float *)malloc(sizeof(float) * (size_t)(d * N + 1));
    if (!wt) return -2;
    for (int64_t e = 0; e < N; ++e)
        for (int64_t k = 0; k < d; ++k) wt[k * N + e] = w[e * d + k];
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
        logits_fma(x, wt, bias, T, d, N, out);
    else
        logits_portable(x, wt, bias, T, d, N, out);
    free(wt);
    return 0;
}

/* Scalar fmaf, exposed so the tests can pin it against exact rational arithmetic. */
void oracle_fmaf_array(const float *a, const float *b, const float *c, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = fmaf(a[i], b[i], c[i]);
}
