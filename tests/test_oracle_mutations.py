"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one oracle function (on the CPU, inside this process only)
with a plausible error and checks that the pin written for that step fails.
"""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as mo
import test_oracle_pins as pins


def patch(monkeypatch, name, fn):
    """Replace one oracle function everywhere it can be reached from."""
    monkeypatch.setattr(mo, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def expect_failure(fn):
    with pytest.raises(AssertionError):
        fn()


def test_unrenormalised_gates_are_caught(monkeypatch):
    def bad(logits, idx):
        l = np.asarray(logits, np.float64)
        s = np.exp(l - l.max(1, keepdims=True)); s /= s.sum(1, keepdims=True)
        return np.take_along_axis(s, idx.astype(np.int64), 1)      # missing renormalisation
    patch(monkeypatch, "renormalised_gates", bad)
    expect_failure(lambda: pins.test_gates_equal_ratio_form_and_masked_resoftmax_form("tiny_fp32"))


def test_wrong_tie_rule_is_caught(monkeypatch):
    def bad(logits, K):
        l = np.asarray(logits, np.float32)[:, ::-1]
        o = np.argsort(-l, axis=1, kind="stable")[:, :K]
        return (l.shape[1] - 1 - o).astype(np.int32)               # ties to the higher id
    patch(monkeypatch, "select_top_k", bad)
    expect_failure(pins.test_top_k_all_ties_take_lowest_ids_and_equal_gates)


def test_ascending_selection_is_caught(monkeypatch):
    def bad(logits, K):
        return np.argsort(np.asarray(logits, np.float32), axis=1, kind="stable")[:, :K].astype(np.int32)
    patch(monkeypatch, "select_top_k", bad)
    expect_failure(pins.test_top_k_is_the_unique_dominating_subset_by_brute_force)


def test_dropping_the_first_tokens_instead_of_the_last_is_caught(monkeypatch):
    orig = mo.dispatch

    def bad(idx, N, C):
        if C is None:
            return orig(idx, N, C)
        rev = orig(np.asarray(idx)[::-1], N, C)                   # keeps the last C tokens
        T = idx.shape[0]
        out = dict(rev)
        out["slot_row"] = rev["slot_row"][::-1].copy()
        out["row_token"] = (T - 1 - rev["row_token"]).astype(np.int32)
        return out
    patch(monkeypatch, "dispatch", bad)
    expect_failure(lambda: pins.test_dispatch_matches_sort_definition_and_invariants(3))


def test_sign_error_in_silu_is_caught(monkeypatch):
    patch(monkeypatch, "silu", lambda z: z / (1.0 + np.exp(z)))
    expect_failure(pins.test_expert_ffn_matches_torch_modules)


def test_transposed_second_linear_is_caught(monkeypatch):
    orig = mo.expert_ffn

    def bad(z, w1, b1, w2, b2, return_hidden=False):
        w2 = np.asarray(w2)
        if w2.shape[0] == w2.shape[1]:
            w2 = w2.T
        return orig(z, w1, b1, w2, b2, return_hidden)
    patch(monkeypatch, "expert_ffn", bad)
    wl = pins.W.custom_workload("sq", T=6, d_model=8, n_routed=3, top_k=2, n_shared=0, d_ff=8,
                                dtype="f32", expert_bias=True)
    routed, _ = pins.providers(wl)
    x = wl.x().numpy()
    import torch
    w1, b1, w2, b2 = (torch.from_numpy(np.asarray(t, np.float64)) for t in routed(0))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(
        torch.nn.functional.linear(torch.from_numpy(x).double(), w1, b1)), w2, b2).numpy()
    got = mo.expert_ffn(x, *routed(0))
    assert not np.allclose(got, ref)


def test_dropped_shared_experts_are_caught(monkeypatch):
    orig = mo.layer_forward

    def bad(*a, **k):
        k["n_shared"] = 0
        return orig(*a, **k)
    patch(monkeypatch, "layer_forward", bad)
    expect_failure(lambda: pins.test_layer_equals_dense_masked_brute_force(pins.SMALL[1]))


def test_biased_gates_in_selection_only_mode_are_caught(monkeypatch):
    orig = oracle.renormalised_gates
    real_route = mo.route

    def bad(x, w_r, bias, K, selection_only_bias=False):
        if selection_only_bias and bias is not None:
            logits = mo.router_logits(x, w_r, bias)      # bias leaks into the gates
            idx = mo.select_top_k(logits, K)
            return mo.router_logits(x, w_r, None), idx, orig(logits, idx)
        return real_route(x, w_r, bias, K, selection_only_bias)
    patch(monkeypatch, "route", bad)
    with pytest.raises(AssertionError):
        pins.test_selection_only_bias_steers_selection_not_gates()


def test_assignment_share_over_tokens_instead_of_assignments_is_caught(monkeypatch):
    def bad(logits, idx, alpha=0.01):
        l64 = np.asarray(logits, dtype=np.float64)
        T, N = l64.shape
        s = np.exp(l64 - l64.max(axis=1, keepdims=True))
        s /= s.sum(axis=1, keepdims=True)
        f = np.bincount(np.asarray(idx).ravel(), minlength=N) / T      # share of tokens
        P = s.mean(axis=0)
        return f, P, float(alpha * N * np.sum(f * P))
    patch(monkeypatch, "balance_statistics", bad)
    expect_failure(pins.test_balance_statistics_invariants_and_even_routing)


# ---------------------------------------------------------------------------
# FP8 dispatch (reading 10)
# ---------------------------------------------------------------------------
import test_oracle_fp8 as fp8pins  # noqa: E402


def test_e4m3_ties_away_from_zero_are_caught(monkeypatch):
    orig = mo.round_e4m3

    def bad(v):
        v = np.asarray(v, dtype=np.float64)
        c = orig(v)
        vals = mo.e4m3_values()
        up = np.minimum((c & 0x7F).astype(np.int64) + 1, 0x7E)
        mid = (np.abs(vals[(c & 0x7F).astype(np.int64)]) + vals[up]) / 2
        tie_down = np.abs(v) == mid                        # a tie rounded to the even code below
        return np.where(tie_down, (up | (c & 0x80)).astype(np.uint8), c)
    patch(monkeypatch, "round_e4m3", bad)
    expect_failure(fp8pins.test_hand_rounded_codes)
    expect_failure(fp8pins.test_rounding_matches_torch_cast)


def test_e4m3_truncation_is_caught(monkeypatch):
    def bad(v):
        v = np.asarray(v, dtype=np.float64)
        mags = mo.e4m3_values()[:0x7F]
        code = np.clip(np.searchsorted(mags, np.abs(v), side="right") - 1, 0, 0x7E).astype(np.uint8)
        return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    patch(monkeypatch, "round_e4m3", bad)
    expect_failure(fp8pins.test_hand_rounded_codes)


def test_scale_exponent_off_by_one_is_caught(monkeypatch):
    orig = mo.fp8_scale_exponent
    patch(monkeypatch, "fp8_scale_exponent", lambda row: orig(row) + 1)
    expect_failure(fp8pins.test_scale_exponent_is_the_smallest_that_fits)
    expect_failure(fp8pins.test_quantisation_error_bound)


def test_dequantisation_without_the_scale_is_caught(monkeypatch):
    def bad(E, q):
        return mo.e4m3_values()[np.asarray(q, dtype=np.int64)]
    patch(monkeypatch, "dequantize_fp8_rows", bad)
    expect_failure(fp8pins.test_quantisation_error_bound)
    expect_failure(fp8pins.test_fp8_dispatch_of_representable_rows_changes_nothing)
