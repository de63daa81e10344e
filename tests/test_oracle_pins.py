"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: exact
rational arithmetic, brute force over all subsets, the pages' printed numbers,
a second formula printed on the pages, a library routine for a special case,
or an invariant.  None needs a GPU.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# exact float32 rounding of a rational number (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def round_to_f32(q: Fraction) -> np.float32:
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormal range shares the min exponent
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = sign * fl * ulp
    out = np.float32(float(v))
    assert Fraction(float(out)) == v, "value must be representable"
    return out


def F(v) -> Fraction:
    return Fraction(float(np.float32(v)))


# ---------------------------------------------------------------------------
# logits: fixed-order fused multiply-add chain
# ---------------------------------------------------------------------------

def test_round_to_f32_helper_on_known_values():
    assert round_to_f32(Fraction(1, 3)) == np.float32(1.0 / 3.0)
    # a halfway case: 1 + 2^-24 lies between 1 and 1 + 2^-23 -> ties to even (1)
    assert round_to_f32(1 + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert round_to_f32(1 + Fraction(3, 2 ** 24)) == np.float32(1 + 2 ** -22)


def test_fmaf_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))).astype(np.float32)
    b = (rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))).astype(np.float32)
    c = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    # crafted cases where a*b + c falls exactly halfway between two floats, or
    # where a separately rounded product would round differently
    h = np.float32(1 + 2 ** -12)
    extra = [(h, h, 0.0), (h, h, -1.0), (np.float32(1 + 2 ** -23), np.float32(1 - 2 ** -24), 0.0),
             (np.float32(3.0), np.float32(1 / 3), np.float32(-1.0)), (0.0, 5.0, -0.0)]
    for (p, q, r) in extra:
        a = np.append(a, np.float32(p)); b = np.append(b, np.float32(q)); c = np.append(c, np.float32(r))
    got = oracle.fmaf_array(a, b, c)
    for i in range(a.size):
        want = round_to_f32(F(a[i]) * F(b[i]) + F(c[i]))
        assert got[i] == want, (i, a[i], b[i], c[i], got[i], want)


def exact_chain_logits(x, w, bias):
    T, d = x.shape
    N = w.shape[0]
    out = np.zeros((T, N), dtype=np.float32)
    for t in range(T):
        for e in range(N):
            acc = np.float32(0.0)
            for k in range(d):
                acc = round_to_f32(F(x[t, k]) * F(w[e, k]) + F(acc))
            if bias is not None:
                acc = round_to_f32(F(acc) + F(bias[e]))
            out[t, e] = acc
    return out


@pytest.mark.parametrize("with_bias", [False, True])
def test_router_logits_equal_exact_fixed_order_chain(with_bias):
    rng = np.random.default_rng(2)
    T, N, d = 3, 5, 24
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((N, d)) / np.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    got = oracle.router_logits(x, w, bias)
    want = exact_chain_logits(x, w, bias)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_router_logits_fma_order_differs_from_separate_rounding():
    """The fixed order is observable: a mul-then-add chain gives other bits here."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    w = rng.standard_normal((8, 64)).astype(np.float32)
    got = oracle.router_logits(x, w)
    sep = np.zeros((16, 8), dtype=np.float32)
    for k in range(64):
        sep = (sep + (x[:, k:k + 1] * w[None, :, k]).astype(np.float32)).astype(np.float32)
    assert not np.array_equal(got, sep)


def test_router_logits_close_to_float64_product():
    wl = W.get_workload("tiny_fp32")
    x = wl.x().numpy()
    w = wl.w_router().numpy()
    got = oracle.router_logits(x, w).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_router_logits_one_hot_exact():
    rng = np.random.default_rng(4)
    N, d = 6, 10
    w = rng.standard_normal((N, d)).astype(np.float32)
    x = np.eye(d, dtype=np.float32)
    got = oracle.router_logits(x, w)
    assert np.array_equal(got, w.T)


# ---------------------------------------------------------------------------
# top-K selection
# ---------------------------------------------------------------------------

def dominates(li, i, lj, j):
    return li > lj or (li == lj and i < j)


def test_top_k_is_the_unique_dominating_subset_by_brute_force():
    wl = W.get_workload("tiny_fp32")
    logits = oracle.router_logits(wl.x().numpy(), wl.w_router().numpy())
    K, N = wl.top_k, wl.n_routed
    idx = oracle.select_top_k(logits, K)
    for t in range(logits.shape[0]):
        l = logits[t]
        winners = []
        best_mass, best_sets = -1.0, []
        for S in itertools.combinations(range(N), K):
            rest = [j for j in range(N) if j not in S]
            if all(dominates(l[i], i, l[j], j) for i in S for j in rest):
                winners.append(S)
            mass = sum(math.exp(float(l[i])) for i in S)       # sum of softmax numerators
            if mass > best_mass:
                best_mass, best_sets = mass, [S]
        assert len(winners) == 1
        assert tuple(sorted(idx[t])) == winners[0]
        assert tuple(sorted(idx[t])) in best_sets      # the kept set carries the most probability
        # slot order: key descending
        for k in range(K - 1):
            assert dominates(l[idx[t, k]], idx[t, k], l[idx[t, k + 1]], idx[t, k + 1])


def test_top_k_all_ties_take_lowest_ids_and_equal_gates():
    T, N, d, K = 5, 8, 16, 3
    x = np.random.default_rng(5).standard_normal((T, d)).astype(np.float32)
    w = np.zeros((N, d), dtype=np.float32)
    logits, idx, gates = oracle.route(x, w, None, K)
    assert np.all(logits == 0)
    assert np.array_equal(idx, np.tile(np.arange(K, dtype=np.int32), (T, 1)))
    assert np.allclose(gates, 1.0 / K, rtol=0, atol=1e-15)


@pytest.mark.parametrize("entry", range(2))
def test_every_subset_is_selectable_and_counts_match_pages(entry):
    """Each K-subset wins for some input, so the router spans C(N, K) choices."""
    g = golden()["combinations"][entry]
    N, K = g["n"], g["k"]
    w = np.eye(N, dtype=np.float32)               # logits equal the input
    seen = set()
    for S in itertools.combinations(range(N), K):
        x = np.zeros((1, N), dtype=np.float32)
        x[0, list(S)] = 1.0
        idx = oracle.select_top_k(oracle.router_logits(x, w), K)
        seen.add(tuple(sorted(idx[0])))
        assert tuple(sorted(idx[0])) == S
    assert len(seen) == g["value"]


def test_fine_grained_combination_count_matches_page():
    g = golden()
    fg = g["fine_grained_split"]
    N, K, m = fg["N"], fg["K"], fg["m"]
    vals = {(c["n"], c["k"]): c["value"] for c in g["combinations"]}
    assert math.comb(N, K) == vals[(N, K)]
    assert math.comb(m * N, m * K) == vals[(m * N, m * K)]


# ---------------------------------------------------------------------------
# renormalised gates: two formulas printed on the pages must agree
# ---------------------------------------------------------------------------

def full_softmax(l):
    l = np.asarray(l, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("name", ["tiny_fp32", "dsv3_decode"])
def test_gates_equal_ratio_form_and_masked_resoftmax_form(name):
    wl = W.get_workload(name)
    x = wl.x().float().numpy()
    b = wl.router_bias_values()
    logits, idx, gates = oracle.route(x, wl.w_router().numpy(), None if b is None else b.numpy(),
                                      wl.top_k)
    s = full_softmax(logits)
    # ratio form: g_j = s_j / sum_{k in TopK} s_k
    sk = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    ratio = sk / sk.sum(axis=1, keepdims=True)
    # masked form: probabilities outside the top K set to zero, then renormalised
    mask = np.zeros_like(s)
    np.put_along_axis(mask, idx.astype(np.int64), 1.0, axis=1)
    masked = s * mask
    masked = masked / masked.sum(axis=1, keepdims=True)
    masked_k = np.take_along_axis(masked, idx.astype(np.int64), axis=1)
    assert np.allclose(gates, ratio, rtol=0, atol=1e-12)
    assert np.allclose(gates, masked_k, rtol=0, atol=1e-12)
    assert np.allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # the literal "zeros then softmax" variant would give dropped experts weight
    lit = full_softmax(np.where(mask > 0, logits, 0.0))
    if wl.n_routed > wl.top_k:
        assert np.all(lit.sum(axis=1) - np.take_along_axis(lit, idx.astype(np.int64), 1).sum(1) > 0)


def test_gates_k1_are_one():
    wl = W.get_workload("tiny_fp32")
    _, idx, gates = oracle.route(wl.x().numpy(), wl.w_router().numpy(), None, 1)
    assert np.all(gates == 1.0)


# ---------------------------------------------------------------------------
# dispatch: counting walk vs a sort-based definition
# ---------------------------------------------------------------------------

def dispatch_by_sort(idx, N, C):
    T, K = idx.shape
    e = idx.ravel().astype(np.int64)
    t = np.repeat(np.arange(T), K)
    order = np.lexsort((t, e))                  # rows sorted by (expert, token)
    es, ts = e[order], t[order]
    first = np.searchsorted(es, np.arange(N))
    rank_sorted = np.arange(es.size) - first[es]
    keep = np.ones(es.size, bool) if C is None else rank_sorted < C
    counts = np.bincount(es[keep], minlength=N)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    row = offsets[es] + rank_sorted
    slot = np.full(T * K, -1)
    slot[order[keep]] = row[keep]
    row_token = np.empty(int(offsets[-1]), dtype=np.int64)
    row_token[row[keep]] = ts[keep]
    return counts, offsets, row_token, slot.reshape(T, K)


@pytest.mark.parametrize("C", [None, 0, 1, 3, 7, 10 ** 6])
def test_dispatch_matches_sort_definition_and_invariants(C):
    rng = np.random.default_rng(6)
    T, N, K = 97, 11, 3
    idx = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(idx, N, C)
    counts, offsets, row_token, slot = dispatch_by_sort(idx, N, C)
    assert np.array_equal(d["counts"], counts)
    assert np.array_equal(d["offsets"], offsets)
    assert np.array_equal(d["row_token"], row_token)
    assert np.array_equal(d["slot_row"], slot)
    assert d["counts"].sum() == T * K - d["n_dropped"]
    if C is not None:
        assert d["counts"].max() <= C
        assert d["n_dropped"] == int(np.maximum(d["raw_counts"] - C, 0).sum())
    # row_token / slot_row are inverse bijections onto [0, offsets[N])
    kept = d["slot_row"] >= 0
    rows = d["slot_row"][kept]
    assert np.array_equal(np.sort(rows), np.arange(d["offsets"][-1]))
    tt = np.nonzero(kept)[0]
    assert np.array_equal(d["row_token"][rows], tt)
    if C is not None and C >= T * K:
        assert d["n_dropped"] == 0


def test_capacity_formula_at_decode_shape():
    wl = W.get_workload("dsv3_decode")
    assert oracle.capacity_limit(wl.capacity_factor, wl.T, wl.top_k, wl.n_routed) == 5
    assert oracle.capacity_limit(0.0, 128, 8, 256) is None
    assert oracle.capacity_limit(1.0, 10, 2, 3) == 7          # ceil(20/3)


# ---------------------------------------------------------------------------
# expert FFN and whole layer
# ---------------------------------------------------------------------------

def test_expert_ffn_matches_torch_modules():
    wl = W.get_workload("tiny_fp32")
    w1, b1, w2, b2 = (t.double() for t in wl.routed_expert(0))
    x = wl.x().double()
    mod = torch.nn.Sequential(torch.nn.Linear(wl.d_model, wl.d_ff), torch.nn.SiLU(),
                              torch.nn.Linear(wl.d_ff, wl.d_model)).double()
    with torch.no_grad():
        mod[0].weight.copy_(w1); mod[0].bias.copy_(b1)
        mod[2].weight.copy_(w2); mod[2].bias.copy_(b2)
        ref = mod(x).numpy()
    got = oracle.expert_ffn(x.numpy(), w1.numpy(), b1.numpy(), w2.numpy(), b2.numpy())
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def providers(wl):
    cache = {}

    def routed(e):
        if ("r", e) not in cache:
            cache[("r", e)] = tuple(None if t is None else t.float().numpy() for t in wl.routed_expert(e))
        return cache[("r", e)]

    def shared(i):
        if ("s", i) not in cache:
            cache[("s", i)] = tuple(None if t is None else t.float().numpy() for t in wl.shared_expert(i))
        return cache[("s", i)]
    return routed, shared


SMALL = [
    W.get_workload("tiny_fp32"),
    W.custom_workload("small_shared_cap", T=40, d_model=32, n_routed=6, top_k=2, n_shared=2,
                      d_ff=48, dtype="f32", expert_bias=True, capacity_factor=1.0),
    W.custom_workload("small_bias", T=33, d_model=16, n_routed=5, top_k=3, n_shared=1,
                      d_ff=24, dtype="bf16", router_bias="gauss", router_bias_var=0.5),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_layer_equals_dense_masked_brute_force(wl):
    routed, shared = providers(wl)
    x = wl.x().float().numpy()
    b = wl.router_bias_values()
    b = None if b is None else b.numpy()
    kw = dict(top_k=wl.top_k, n_shared=wl.n_shared, capacity_factor=wl.capacity_factor)
    got = oracle.layer_forward(x, wl.w_router().numpy(), b, routed, shared, **kw)
    ref = oracle.dense_masked_forward(x, wl.w_router().numpy(), b, routed, shared, **kw)
    assert np.allclose(got["y"], ref, rtol=1e-12, atol=1e-12)


def test_layer_entry_point_composition_equals_layer():
    """dispatch -> gather -> grouped FFN -> combine reproduces layer_forward."""
    wl = SMALL[1]
    routed, shared = providers(wl)
    x = wl.x().numpy()
    lay = oracle.layer_forward(x, wl.w_router().numpy(), None, routed, shared, top_k=wl.top_k,
                               n_shared=wl.n_shared, capacity_factor=wl.capacity_factor)
    xp = oracle.gather_rows(x, lay["row_token"])
    _, Y = oracle.grouped_ffn(xp, lay["offsets"], routed, wl.n_routed)
    S = np.stack([oracle.expert_ffn(x, *shared(i)) for i in range(wl.n_shared)])
    y = oracle.combine(Y, lay["slot_row"], lay["gates"], S)
    assert np.allclose(y, lay["y"], rtol=1e-12, atol=1e-12)


def test_identical_experts_reduce_to_one_ffn():
    wl = W.custom_workload("ident", T=20, d_model=16, n_routed=7, top_k=3, n_shared=1, d_ff=32,
                           dtype="f32", expert_bias=True)
    e0 = tuple(t.numpy() for t in wl.routed_expert(0))
    s0 = tuple(t.numpy() for t in wl.shared_expert(0))
    x = wl.x().numpy()
    out = oracle.layer_forward(x, wl.w_router().numpy(), None, lambda e: e0, lambda i: s0,
                               top_k=3, n_shared=1)
    ref = oracle.expert_ffn(x, *e0) + oracle.expert_ffn(x, *s0)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_k_equals_n_is_the_dense_softmax_mixture():
    wl = W.custom_workload("dense", T=12, d_model=16, n_routed=4, top_k=4, n_shared=0, d_ff=8,
                           dtype="f32", expert_bias=True)
    routed, _ = providers(wl)
    x = wl.x().numpy()
    out = oracle.layer_forward(x, wl.w_router().numpy(), None, routed, None, top_k=4, n_shared=0)
    s = full_softmax(out["logits"])
    ref = sum(s[:, e:e + 1] * oracle.expert_ffn(x, *routed(e)) for e in range(4))
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_zero_capacity_leaves_only_shared_experts():
    wl = SMALL[1]
    routed, shared = providers(wl)
    x = wl.x().numpy()
    out = oracle.layer_forward(x, wl.w_router().numpy(), None, routed, shared, top_k=wl.top_k,
                               n_shared=wl.n_shared, capacity=0)
    ref = sum(oracle.expert_ffn(x, *shared(i)) for i in range(wl.n_shared))
    assert out["n_dropped"] == wl.T * wl.top_k
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_combine_with_every_slot_dropped_and_no_shared_expert_is_zero():
    # a token whose K slots are all dropped gets only the shared sum, here
    # empty: y = 0 at the rows' width, also when no routed row was kept
    T, K, d = 5, 3, 7
    slot_row = np.full((T, K), -1, dtype=np.int32)
    y = oracle.combine(np.zeros((0, d)), slot_row, np.full((T, K), 1.0 / K))
    assert y.shape == (T, d) and not y.any()
    S = np.arange(2 * T * d, dtype=np.float64).reshape(2, T, d)
    y = oracle.combine(np.zeros((0, d)), slot_row, np.full((T, K), 1.0 / K), S)
    assert np.array_equal(y, S[0] + S[1])


def test_capacity_that_drops_nothing_equals_unlimited():
    wl = SMALL[1]
    routed, shared = providers(wl)
    x = wl.x().numpy()
    a = oracle.layer_forward(x, wl.w_router().numpy(), None, routed, shared, top_k=wl.top_k,
                             n_shared=wl.n_shared)
    big = int(a["raw_counts"].max())
    b = oracle.layer_forward(x, wl.w_router().numpy(), None, routed, shared, top_k=wl.top_k,
                             n_shared=wl.n_shared, capacity=big)
    assert b["n_dropped"] == 0
    assert np.array_equal(a["y"], b["y"])


def test_active_parameters_are_k_over_n():
    """Evaluated routed experts per token equal K, so the active share is K/N."""
    g = golden()["active_fraction"][0]
    wl = W.custom_workload("act", T=64, d_model=16, n_routed=g["n"], top_k=g["k"], n_shared=0,
                           d_ff=8, dtype="f32")
    routed, _ = providers(wl)
    rows = {"n": 0}
    import oracle.moe_oracle as mo
    orig = mo.expert_ffn

    def spy(z, *a, **k):
        rows["n"] += np.asarray(z).shape[0]
        return orig(z, *a, **k)
    mo.expert_ffn = spy
    try:
        oracle.layer_forward(wl.x().numpy(), wl.w_router().numpy(), None, routed, None,
                             top_k=wl.top_k, n_shared=0)
    finally:
        mo.expert_ffn = orig
    per_expert = 2 * wl.d_model * wl.d_ff
    active = rows["n"] * per_expert / wl.T
    total = wl.n_routed * per_expert
    assert active / total == pytest.approx(g["percent"] / 100.0, abs=0)


def test_fine_grained_workload_is_the_pages_split():
    """64 experts, top-8, width 1408 is the m=4 split of 16 experts, top-2, width 5632."""
    fg = golden()["fine_grained_split"]
    wl = W.get_workload("deepseekmoe_fine")
    assert wl.n_routed == fg["m"] * fg["N"] and wl.top_k == fg["m"] * fg["K"]
    d_ff_coarse = wl.d_ff * fg["m"]
    # active routed width per token is unchanged by the split
    assert wl.top_k * wl.d_ff == fg["K"] * d_ff_coarse


# ---------------------------------------------------------------------------
# balance statistics ([DSMoE] balance-loss equation, reading 9)
# ---------------------------------------------------------------------------

def test_balance_statistics_hand_examples():
    ln3 = math.log(3.0)
    # softmax rows (1/4, 3/4) and (3/4, 1/4): P = (1/2, 1/2); one token per
    # expert: f = (1/2, 1/2); L = alpha * 2 * (1/4 + 1/4) = alpha
    f, P, L = oracle.balance_statistics(np.array([[0.0, ln3], [ln3, 0.0]]), np.array([[1], [0]]), 0.01)
    assert np.allclose(P, [0.5, 0.5], atol=1e-15) and np.allclose(f, [0.5, 0.5])
    assert abs(L - 0.01) < 1e-15
    # both tokens pick expert 1 with probability 3/4: L = alpha * 2 * 3/4
    f, P, L = oracle.balance_statistics(np.array([[0.0, ln3], [0.0, ln3]]), np.array([[1], [1]]), 0.01)
    assert np.allclose(P, [0.25, 0.75], atol=1e-15) and np.allclose(f, [0.0, 1.0])
    assert abs(L - 0.015) < 1e-15


def test_balance_statistics_invariants_and_even_routing():
    rng = np.random.default_rng(5)
    T, N, K = 96, 16, 4
    logits = rng.standard_normal((T, N)).astype(np.float32)
    idx = oracle.select_top_k(logits, K)
    f, P, L = oracle.balance_statistics(logits, idx, 0.01)
    assert abs(f.sum() - 1.0) < 1e-12 and abs(P.sum() - 1.0) < 1e-12
    # brute-force definition, token by token
    Pb = np.zeros(N)
    for t in range(T):
        e = np.exp(logits[t].astype(np.float64))
        Pb += e / e.sum()
    assert np.allclose(P, Pb / T, rtol=1e-12)
    assert np.allclose(f * T * K, [np.sum(idx == j) for j in range(N)])
    # equal logits and a perfectly even routing give L = alpha
    even = np.array([[(t * K + k) % N for k in range(K)] for t in range(T)])
    f, P, L = oracle.balance_statistics(np.zeros((T, N)), even, 0.01)
    assert np.allclose(P, 1.0 / N) and np.allclose(f, 1.0 / N) and abs(L - 0.01) < 1e-14


# ---------------------------------------------------------------------------
# selection-only bias (reading 8)
# ---------------------------------------------------------------------------

def _tiny_router(seed, T=24, d=32, N=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    return x, w, b


def test_selection_only_bias_of_zero_is_the_plain_router():
    x, w, _ = _tiny_router(1)
    z = np.zeros(w.shape[0], dtype=np.float32)
    l0, i0, g0 = oracle.route(x, w, None, 3)
    l1, i1, g1 = oracle.route(x, w, z, 3, selection_only_bias=True)
    assert np.array_equal(l0, l1) and np.array_equal(i0, i1) and np.array_equal(g0, g1)


def test_selection_only_bias_steers_selection_not_gates():
    x, w, _ = _tiny_router(2)
    N = w.shape[0]
    b = np.zeros(N, dtype=np.float32)
    b[5] = 1.0e4                      # expert 5 always wins the selection
    logits, idx, gates = oracle.route(x, w, b, 2, selection_only_bias=True)
    assert np.all(idx[:, 0] == 5)
    plain = x @ w.T                   # the returned logits carry no bias
    assert np.allclose(logits, plain, atol=1e-5)
    # gate of expert 5 from the unbiased logits of the two kept experts
    for t in range(x.shape[0]):
        l5, lo = float(logits[t, 5]), float(logits[t, idx[t, 1]])
        assert abs(gates[t, 0] - 1.0 / (1.0 + math.exp(lo - l5))) < 1e-12


def test_selection_only_bias_brute_force():
    x, w, b = _tiny_router(3, N=6)
    K = 3
    logits, idx, gates = oracle.route(x, w, b, K, selection_only_bias=True)
    key = logits + b[None, :]
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(w.shape[0]), K),
                   key=lambda s: (sum(float(key[t, j]) for j in s), [-j for j in s]))
        assert sorted(best) == sorted(idx[t].tolist())
        kept = np.exp(logits[t, idx[t]].astype(np.float64))
        assert np.allclose(gates[t], kept / kept.sum(), rtol=1e-12)
