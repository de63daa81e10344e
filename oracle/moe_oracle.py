"""Plain CPU oracle of the sparse top-K MoE FFN forward with renormalised gates.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  It shares no code with the HIP library
and never calls it; its only native piece is ``fixed_order_logits.c`` (gcc).
Everything is written to be checked by eye against the pages, in float64
unless a step is defined in float32 (the router logits).

Pages (cited by title and section):

* [TopK] "Sparse MoE Top-Kルーティング" glossary page (jisaku.com), section
  "ルーティングの仕組み" (routing mechanism: score every expert, keep the K
  best, mask the rest and re-apply softmax, gate-weighted sum) and section
  "解決策2: エキスパートキャパシティファクター" (per-expert token limit; tokens
  over it are dropped or pass through the residual).
* [DSMoE] "論文解説: DeepSeekMoE — 細粒度エキスパート分割と共有エキスパートによる
  MoE効率化" (0h-n0.github.io), section "共有エキスパート機構" (output equation
  h_t = sum_i E_s,i(x_t) + sum_{j in TopK} g_j(x_t) E_r,j(x_t)), section
  "ルーティングとバランス損失" (gate equation g_j = s_j / sum_{k in TopK} s_k,
  s = softmax(W_r x); balance loss), section "アルゴリズム" (reference layer:
  router Linear without bias, experts Linear(d, d_ff) - SiLU - Linear(d_ff, d)).
* [EP] "エキスパート並列（Expert Parallelism）" glossary page (jisaku.com),
  section "MoEアーキテクチャの概要" (active parameters = K/N of expert parameters).

Readings taken where the pages are silent or disagree (each is also listed in
the design notes):

1. Masking before the re-softmax sets the dropped experts' probabilities to 0
   (logits to -inf), so the re-softmax is a softmax over the K kept logits and
   equals s_j / sum_TopK s_k exactly in real arithmetic.
2. Experts are selected on the float32 (biased) logit, key (logit desc,
   expert id asc): ties go to the lower expert id.  Slots are in that order.
3. Logits use one fixed float32 order: fused multiply-add over k ascending
   from +0, then the router bias added with one rounding.
4. A router bias, when present, is part of the logit for selection and gates.
5. Capacity C = ceil(cf * T * K / N) evaluated in float64 as
   ((cf * T) * K) / N; an expert keeps its first C tokens in token order and
   drops the rest; dropped assignments contribute 0; gates are not
   re-normalised over the kept ones; the residual add is the caller's.
6. Expert FFN E(z) = W2 SiLU(W1 z + b1) + b2, SiLU(z) = z / (1 + e^-z).
7. Output y_t = sum of shared experts + sum of kept gate-weighted routed
   experts; no residual term.
8. Selection-only bias (the bias-based balancing of [TopK] section 負荷均衡,
   which steers the load without changing the loss): when asked for, the
   bias enters only the selection key fl32(logit + bias[e]); the gates are
   the softmax over the K kept unbiased logits, and the logits returned are
   the unbiased ones.
9. Balance statistics ([DSMoE] balance-loss equation): f_j is the share of
   the T*K routed assignments that go to expert j (so the f_j sum to 1 and a
   perfectly even routing gives L = alpha), P_j the mean over tokens of the
   full softmax over all N logits.
10. FP8 dispatch ([DeepEP] section "DeepEP とは？", item 5, native FP8 data
    dispatch that cuts transfer volume; section "DeepEP の性能", settings with
    FP8 dispatch and BF16 combine).  The pages fix neither the FP8 format nor
    the scaling, so: the dispatched token rows are OCP FP8 E4M3 (E4M3FN: sign,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; largest finite value 448; no infinities), with one
    power-of-two scale per token row, 2^E with E the smallest integer such
    that max_k |x[t,k]| <= 448 * 2^E (E = 0 for an all-zero row).  Codes are
    x / 2^E rounded to the nearest E4M3 value, ties to the even mantissa.
    The routed experts consume the dispatched rows x~ = 2^E * value(code);
    the router and the shared experts (which the pages keep on every device,
    never dispatched) use x itself; the combine is unchanged (BF16).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Callable, Dict, Optional, Sequence

import numpy as np

from . import build as _build

__all__ = [
    "router_logits", "select_top_k", "renormalised_gates", "capacity_limit",
    "dispatch", "gather_rows", "silu", "expert_ffn", "grouped_ffn",
    "combine", "route", "layer_forward", "dense_masked_forward",
    "balance_statistics", "fmaf_array",
    "e4m3_values", "round_e4m3", "fp8_scale_exponent", "quantize_fp8_rows",
    "dequantize_fp8_rows",
]

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        lib.oracle_router_logits.restype = ctypes.c_int
        lib.oracle_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p]
        lib.oracle_fmaf_array.restype = None
        lib.oracle_fmaf_array.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def _f32c(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def fmaf_array(a, b, c) -> np.ndarray:
    """Elementwise C ``fmaf`` (one rounding), used by the router and by its pins."""
    a, b, c = _f32c(a), _f32c(b), _f32c(c)
    out = np.empty_like(a)
    _lib().oracle_fmaf_array(a.ctypes.data, b.ctypes.data, c.ctypes.data, a.size, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# Router: [TopK] routing mechanism; [DSMoE] gate equation, s = softmax(W_r x)
# ---------------------------------------------------------------------------

def router_logits(x, w_r, bias=None) -> np.ndarray:
    """float32 logits [T, N] = W_r x_t (+ bias), in the fixed order of reading 3."""
    x = _f32c(x)
    w_r = _f32c(w_r)
    T, d = x.shape
    N, d2 = w_r.shape
    assert d == d2
    out = np.empty((T, N), dtype=np.float32)
    bptr = None
    if bias is not None:
        bias = _f32c(bias)
        assert bias.shape == (N,)
        bptr = bias.ctypes.data
    rc = _lib().oracle_router_logits(x.ctypes.data, w_r.ctypes.data, bptr, T, d, N, out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_router_logits failed: {rc}")
    return out


def select_top_k(logits: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest logits per token, key (logit desc, expert id asc).

    A stable sort of the negated logits keeps equal keys in ascending expert
    order, which is reading 2's tie rule.
    """
    logits = np.asarray(logits, dtype=np.float32)
    N = logits.shape[1]
    assert 1 <= K <= N
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def renormalised_gates(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g[t,k] = softmax over the K kept logits (float64), reading 1.

    exp(l_k - l_max) / sum_j exp(l_j - l_max) over the kept slots; the largest
    kept logit is subtracted only to keep exp in range.
    """
    kept = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx.astype(np.int64), axis=1)
    m = kept.max(axis=1, keepdims=True)
    p = np.exp(kept - m)
    return p / p.sum(axis=1, keepdims=True)


def route(x, w_r, bias, K: int, selection_only_bias: bool = False):
    """Router + top-K + renormalised gates: (logits f32, idx i32, gates f64).

    With ``selection_only_bias`` (reading 8) the bias only shifts the
    selection key; the logits returned and the gates are unbiased.
    """
    if selection_only_bias and bias is not None:
        logits = router_logits(x, w_r, None)
        key = logits + np.asarray(bias, dtype=np.float32)[None, :]   # float32, one rounding
        idx = select_top_k(key, K)
        return logits, idx, renormalised_gates(logits, idx)
    logits = router_logits(x, w_r, bias)
    idx = select_top_k(logits, K)
    gates = renormalised_gates(logits, idx)
    return logits, idx, gates


# ---------------------------------------------------------------------------
# Dispatch: [TopK] capacity factor section (limit, drop); reading 5
# ---------------------------------------------------------------------------

def capacity_limit(capacity_factor: float, T: int, K: int, N: int,
                   explicit: Optional[int] = None) -> Optional[int]:
    """C = ceil(cf * T * K / N) in float64, or None when cf <= 0 (no limit).

    ``explicit`` (>= 0) is a limit given directly; it takes precedence.
    """
    if explicit is not None and explicit >= 0:
        return int(explicit)
    cf = float(np.float32(capacity_factor))
    if cf <= 0.0:
        return None
    return int(math.ceil(cf * T * K / N))


def dispatch(idx: np.ndarray, N: int, capacity: Optional[int]) -> Dict[str, np.ndarray]:
    """Per-expert token lists, in the order of reading 5.

    Walks tokens in ascending order; the rank of (t, k) in expert e is the
    number of earlier tokens routed to e.  Kept iff no limit or rank < C.
    Returns counts [N], offsets [N+1], row_token [R], slot_row [T,K] (-1 for a
    dropped assignment), raw_counts [N], rank [T,K], n_dropped.
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    seen = np.zeros(N, dtype=np.int64)
    rank = np.zeros((T, K), dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            rank[t, k] = seen[e]
            seen[e] += 1
    raw = seen.copy()
    counts = raw if capacity is None else np.minimum(raw, capacity)
    offsets = np.zeros(N + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    slot_row = np.full((T, K), -1, dtype=np.int64)
    row_token = np.full(int(offsets[-1]), -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if capacity is None or rank[t, k] < capacity:
                r = offsets[e] + rank[t, k]
                slot_row[t, k] = r
                row_token[r] = t
    n_dropped = int(raw.sum() - counts.sum())
    return {
        "counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
        "row_token": row_token.astype(np.int32), "slot_row": slot_row.astype(np.int32),
        "raw_counts": raw.astype(np.int32), "rank": rank.astype(np.int32),
        "n_dropped": n_dropped,
    }


def gather_rows(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """X_perm[r] = x[row_token[r]]."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


# ---------------------------------------------------------------------------
# FP8 dispatch: [DeepEP] "DeepEP とは？" item 5; reading 10
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every E4M3 code 0..255 (float64); NaN for the two NaN codes.

    Code = sign (bit 7), exponent field e (bits 6..3, bias 7), mantissa m
    (bits 2..0): e > 0 gives (1 + m/8) * 2^(e-7), e = 0 gives (m/8) * 2^-6;
    e = 15 with m = 7 is NaN.
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def round_e4m3(v) -> np.ndarray:
    """Codes (uint8) of the E4M3 values nearest to v (|v| <= 448), ties to the
    code with the even mantissa; the sign bit follows v's sign (-0 -> 0x80).

    Among the non-negative codes 0x00..0x7E the magnitudes ascend with the
    code, so the two candidates are found by a search on |v|; the mantissa's
    last bit is the code's last bit.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("round_e4m3 takes finite values within +-448")
    mags = e4m3_values()[:0x7F]                  # codes 0x00 .. 0x7E, ascending
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code[a == mags[hi]] = hi[a == mags[hi]]      # exact values
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def fp8_scale_exponent(row) -> int:
    """Smallest integer E with max|row| <= 448 * 2^E (0 for an all-zero row).

    With max|row| = m * 2^e, m in [0.5, 1), and 448 = 0.875 * 2^9:
    448 * 2^(e-9) >= max|row| exactly when m <= 0.875.
    """
    amax = float(np.max(np.abs(np.asarray(row, dtype=np.float64)))) if np.size(row) else 0.0
    if amax == 0.0:
        return 0
    m, e = math.frexp(amax)
    return e - 9 if m <= 0.875 else e - 8


def quantize_fp8_rows(x):
    """Per-token FP8 dispatch (reading 10): exponents E [T] (int32) and codes
    q [T, d] (uint8) with q[t] = round_e4m3(x[t] / 2^E[t])."""
    x = np.asarray(x, dtype=np.float64)
    E = np.array([fp8_scale_exponent(r) for r in x], dtype=np.int32)
    q = np.stack([round_e4m3(r / 2.0 ** int(e)) for r, e in zip(x, E)]) if len(x) else \
        np.zeros(x.shape, dtype=np.uint8)
    return E, q


def dequantize_fp8_rows(E, q) -> np.ndarray:
    """Dispatched rows x~[t, k] = 2^E[t] * value(q[t, k]) (float64, exact)."""
    vals = e4m3_values()
    return vals[np.asarray(q, dtype=np.int64)] * np.exp2(np.asarray(E, dtype=np.float64))[:, None]


# ---------------------------------------------------------------------------
# Experts: [DSMoE] reference layer (Linear - SiLU - Linear); reading 6
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(z, w1, b1, w2, b2, return_hidden: bool = False):
    """E(z) = W2 SiLU(W1 z + b1) + b2 for rows z [M, d], in float64."""
    z = np.asarray(z, dtype=np.float64)
    a = z @ np.asarray(w1, dtype=np.float64).T
    if b1 is not None:
        a = a + np.asarray(b1, dtype=np.float64)
    h = silu(a)
    y = h @ np.asarray(w2, dtype=np.float64).T
    if b2 is not None:
        y = y + np.asarray(b2, dtype=np.float64)
    return (y, h) if return_hidden else y


def grouped_ffn(x_rows, offsets, expert: Callable[[int], tuple], n_groups: int):
    """Each group g runs its own expert over rows offsets[g]..offsets[g+1]-1.

    Returns (H [R, f], Y [R, d]) in float64.
    """
    x_rows = np.asarray(x_rows)
    R = int(offsets[n_groups])
    d = x_rows.shape[1]
    H = None
    Y = np.zeros((R, d), dtype=np.float64)
    for g in range(n_groups):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        w1, b1, w2, b2 = expert(g)
        y, h = expert_ffn(x_rows[r0:r1], w1, b1, w2, b2, return_hidden=True)
        if H is None:
            H = np.zeros((R, h.shape[1]), dtype=np.float64)
        H[r0:r1] = h
        Y[r0:r1] = y
    return H, Y


# ---------------------------------------------------------------------------
# Combine: [DSMoE] output equation; [TopK] gate-weighted sum; reading 7
# ---------------------------------------------------------------------------

def combine(y_rows, slot_row, gates, shared_out=None) -> np.ndarray:
    """y[t] = sum_i S_i[t] + sum_{k kept} g[t,k] * Y[slot_row[t,k]]  (float64)."""
    slot_row = np.asarray(slot_row)
    T, K = slot_row.shape
    y_rows = np.asarray(y_rows, dtype=np.float64)
    # the width comes from the expert rows even when every slot was dropped
    # (an empty [0, d] array); a bare empty array leaves it to the shared outputs
    if y_rows.ndim == 2:
        d = y_rows.shape[1]
    else:
        d = shared_out.shape[2] if shared_out is not None else 0
    out = np.zeros((T, d), dtype=np.float64)
    if shared_out is not None:
        for i in range(shared_out.shape[0]):
            out += np.asarray(shared_out[i], dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    for k in range(K):
        r = slot_row[:, k]
        keep = r >= 0
        out[keep] += g[keep, k:k + 1] * y_rows[r[keep]]
    return out


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def layer_forward(x, w_r, bias, routed_expert: Callable[[int], tuple],
                  shared_expert: Optional[Callable[[int], tuple]], *, top_k: int,
                  n_shared: int, capacity_factor: float = 0.0,
                  capacity: Optional[int] = None,
                  tokens: Optional[Sequence[int]] = None,
                  selection_only_bias: bool = False,
                  dispatch_fp8: bool = False) -> Dict[str, np.ndarray]:
    """Routing for all tokens and y for ``tokens`` (default: all), float64.

    The routing (logits, selection, gates, dispatch) always covers every token,
    because a token's rank in an expert depends on the earlier tokens.  Only
    the experts that the requested tokens keep are evaluated, each on just
    those tokens, so a handful of tokens of a large layer stays cheap.
    With ``dispatch_fp8`` (reading 10) the routed experts take the dispatched
    FP8 rows x~; the router and the shared experts take x.
    """
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    N = np.asarray(w_r).shape[0]
    logits, idx, gates = route(x, w_r, bias, top_k, selection_only_bias)
    C = capacity_limit(capacity_factor, T, top_k, N, capacity)
    disp = dispatch(idx, N, C)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = x[toks].astype(np.float64)
    xr = xs
    fp8 = {}
    if dispatch_fp8:
        E, q = quantize_fp8_rows(x[toks])
        xr = dequantize_fp8_rows(E, q)
        fp8 = {"fp8_exp": E, "fp8_codes": q}
    y = np.zeros((len(toks), x.shape[1]), dtype=np.float64)
    for i in range(n_shared):
        w1, b1, w2, b2 = shared_expert(i)
        y += expert_ffn(xs, w1, b1, w2, b2)
    slot = disp["slot_row"][toks]
    sel = idx[toks]
    g = gates[toks]
    for e in np.unique(sel[slot >= 0]):
        w1, b1, w2, b2 = routed_expert(int(e))
        for k in range(top_k):
            m = (sel[:, k] == e) & (slot[:, k] >= 0)
            if m.any():
                y[m] += g[m, k:k + 1] * expert_ffn(xr[m], w1, b1, w2, b2)
    out = dict(disp)
    out.update({"logits": logits, "topk_idx": idx, "gates": gates, "capacity": C,
                "tokens": toks, "y": y})
    out.update(fp8)
    return out


def dense_masked_forward(x, w_r, bias, routed_expert, shared_expert, *, top_k: int,
                         n_shared: int, capacity_factor: float = 0.0,
                         capacity: Optional[int] = None,
                         selection_only_bias: bool = False,
                         dispatch_fp8: bool = False) -> np.ndarray:
    """Brute force in the shape of the pages' reference layer.

    Every routed expert is evaluated on every token; for each slot k and each
    expert e the output gains gate * mask(idx[:,k] == e, kept) * E_e(x).  It
    shares the routing with :func:`layer_forward` but none of its dispatch.
    With ``dispatch_fp8`` the routed experts see the dispatched rows x~.
    """
    x = np.asarray(x, dtype=np.float32)
    T, d = x.shape
    N = np.asarray(w_r).shape[0]
    logits, idx, gates = route(x, w_r, bias, top_k, selection_only_bias)
    C = capacity_limit(capacity_factor, T, top_k, N, capacity)
    # kept mask by brute force: count earlier tokens with the same expert
    kept = np.ones((T, top_k), dtype=bool)
    if C is not None:
        for t in range(T):
            for k in range(top_k):
                e = idx[t, k]
                earlier = int(np.sum(idx[:t] == e))
                kept[t, k] = earlier < C
    xs = x.astype(np.float64)
    xr = dequantize_fp8_rows(*quantize_fp8_rows(x)) if dispatch_fp8 else xs
    out = np.zeros((T, d), dtype=np.float64)
    for i in range(n_shared):
        out += expert_ffn(xs, *shared_expert(i))
    for e in range(N):
        ye = expert_ffn(xr, *routed_expert(e))
        for k in range(top_k):
            mask = ((idx[:, k] == e) & kept[:, k]).astype(np.float64)[:, None]
            out += gates[:, k:k + 1] * mask * ye
    return out


# ---------------------------------------------------------------------------
# Load statistics: [DSMoE] balance-loss equation
# ---------------------------------------------------------------------------

def balance_statistics(logits: np.ndarray, idx: np.ndarray, alpha: float = 0.01):
    """f_j (share of routed assignments), P_j (mean full softmax prob), loss (reading 9).

    f_j = (number of (t,k) with idx = j) / (T*K); P_j = mean_t softmax(logits_t)_j;
    L = alpha * N * sum_j f_j P_j.  float64.
    """
    l64 = np.asarray(logits, dtype=np.float64)
    T, N = l64.shape
    K = idx.shape[1]
    s = np.exp(l64 - l64.max(axis=1, keepdims=True))
    s /= s.sum(axis=1, keepdims=True)
    f = np.bincount(np.asarray(idx).ravel(), minlength=N).astype(np.float64) / (T * K)
    P = s.mean(axis=0)
    return f, P, float(alpha * N * np.sum(f * P))
