"""Pins of the oracle's FP8 dispatch (reading 10: OCP E4M3 codes with one
power-of-two scale per token row; DeepEP page, section "DeepEP とは？" item 5
and section "DeepEP の性能", FP8 dispatch with BF16 combine).

What fixes it, independently of the oracle's own code:
* hand-rounded codes from the format's definition (tests/golden);
* every finite code maps to itself, and the codes' values are the format's;
* torch's float8_e4m3fn cast (an independent implementation of the same
  format and rounding) on random values, on every midpoint between two
  neighbouring values (the ties) and just off them;
* the scale rule by brute force over exponents, and the closed-form bound on
  the rounding error (half a step of a 3-bit mantissa, 2^-4 relative, or
  2^-10 * 2^E below the normal range);
* a layer whose token rows are already E4M3 values times their own scale is
  unchanged by FP8 dispatch; the FP8 layer equals the dense masked brute
  force evaluated on the dispatched rows.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_rounded.json")


def torch_e4m3_codes(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_hand_rounded_codes():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 15
    for c in cases:
        assert int(oracle.round_e4m3([c["value"]])[0]) == c["code"], c


def test_code_values_follow_the_format():
    v = oracle.e4m3_values()
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = np.isfinite(v)
    assert finite.sum() == 254
    assert v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    # non-negative codes ascend strictly in value; the sign bit negates
    assert np.all(np.diff(v[:0x7F]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])
    # the same values as torch's format
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(tv), np.isnan(v))
    assert np.array_equal(tv[finite], v[finite].astype(np.float32))


def test_every_code_rounds_to_itself():
    v = oracle.e4m3_values()
    codes = np.array([c for c in range(256) if np.isfinite(v[c])])
    vals = v[codes].copy()
    vals[codes == 0x80] = -0.0
    assert np.array_equal(oracle.round_e4m3(vals), codes.astype(np.uint8))


def test_rounding_matches_torch_cast():
    rng = np.random.default_rng(7)
    v = oracle.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2                    # every tie
    near = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    rand = np.concatenate([rng.uniform(-448, 448, 20000),
                           rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 6, 20000)])
    rand = np.clip(rand, -448, 448)
    for arr in (mids, -mids, near, rand):
        arr32 = arr.astype(np.float32)              # the cast's input, exactly
        assert np.array_equal(oracle.round_e4m3(arr32.astype(np.float64)), torch_e4m3_codes(arr32))


def test_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(3)
    for _ in range(2000):
        amax = float(np.float32(rng.standard_normal() * 2.0 ** rng.integers(-60, 60)))
        amax = abs(amax) or 1.0
        E = oracle.fp8_scale_exponent([amax, -amax / 3])
        brute = min(e for e in range(-300, 300) if amax <= 448.0 * 2.0 ** e)
        assert E == brute
    for amax, E in ((448.0, 0), (449.0, 1), (224.0, -1), (224.5, 0), (1.0, -8), (1.75, -8),
                    (1.76, -7)):
        assert oracle.fp8_scale_exponent([amax]) == E
    assert oracle.fp8_scale_exponent([0.0, -0.0]) == 0


def test_quantisation_error_bound():
    wl = W.custom_workload("fp8pin", T=300, d_model=512, n_routed=4, top_k=2, dtype="bf16")
    x = wl.x().float().numpy().astype(np.float64)
    x[5] *= 2.0 ** -40                              # a tiny row
    x[6] = 0.0                                      # an all-zero row
    E, q = oracle.quantize_fp8_rows(x)
    xt = oracle.dequantize_fp8_rows(E, q)
    scaled = np.abs(x) / np.exp2(E)[:, None]
    # the scale: max |x| / 2^E in (224, 448] for every non-zero row
    amax = scaled.max(axis=1)
    nz = np.abs(x).max(axis=1) > 0
    assert np.all(amax[nz] <= 448) and np.all(amax[nz] > 224)
    assert E[6] == 0 and np.all(q[6] & 0x7F == 0)
    err = np.abs(xt - x)
    normal = scaled >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]))
    bound_sub = (2.0 ** -10 * np.exp2(E))[:, None] * np.ones_like(x)
    assert np.all(err[~normal] <= bound_sub[~normal])
    # the rounding bound is attained within a factor of 2 (it is not loose)
    assert np.max(err[normal] / np.abs(x[normal])) > 2.0 ** -5


def _layer(wl):
    return (wl.x().float().numpy(), wl.w_router().numpy(),
            None if wl.router_bias_values() is None else wl.router_bias_values().numpy(),
            lambda e: tuple(None if t is None else t.float().numpy() for t in wl.routed_expert(e)),
            lambda i: tuple(None if t is None else t.float().numpy() for t in wl.shared_expert(i)))


def test_fp8_layer_equals_dense_masked_on_dispatched_rows():
    wl = W.custom_workload("fp8dense", T=48, d_model=64, n_routed=6, top_k=2, n_shared=1,
                           d_ff=96, dtype="bf16", capacity_factor=1.0, router_bias="gauss",
                           router_bias_var=0.5)
    x, wr, rb, routed, shared = _layer(wl)
    ref = oracle.layer_forward(x, wr, rb, routed, shared, top_k=2, n_shared=1,
                               capacity_factor=1.0, dispatch_fp8=True)
    dense = oracle.dense_masked_forward(x, wr, rb, routed, shared, top_k=2, n_shared=1,
                                        capacity_factor=1.0, dispatch_fp8=True)
    assert np.abs(ref["y"] - dense).max() <= 1e-12 * np.abs(dense).max()
    # and it differs from the bf16 dispatch (the mode is not a no-op)
    plain = oracle.layer_forward(x, wr, rb, routed, shared, top_k=2, n_shared=1,
                                 capacity_factor=1.0)
    assert np.array_equal(plain["topk_idx"], ref["topk_idx"])    # routing uses x itself
    rel = np.linalg.norm(ref["y"] - plain["y"]) / np.linalg.norm(plain["y"])
    assert 1e-4 < rel < 2.0 ** -4


def test_fp8_dispatch_of_representable_rows_changes_nothing():
    # token rows that are already E4M3 values times a power of two whose
    # largest element is 448 * 2^E: the dispatched rows are the rows
    rng = np.random.default_rng(11)
    wl = W.custom_workload("fp8exact", T=40, d_model=64, n_routed=4, top_k=2, n_shared=0,
                           d_ff=64, dtype="bf16")
    _, wr, rb, routed, shared = _layer(wl)
    v = oracle.e4m3_values()[:0x7F]
    E = rng.integers(-14, -6, 40)
    x = v[rng.integers(0, 0x7F, (40, 64))] * rng.choice([-1.0, 1.0], (40, 64))
    x[:, 0] = 448.0
    x = (x * np.exp2(E)[:, None]).astype(np.float32)
    Eq, q = oracle.quantize_fp8_rows(x)
    assert np.array_equal(Eq, E)
    assert np.array_equal(oracle.dequantize_fp8_rows(Eq, q), x.astype(np.float64))
    a = oracle.layer_forward(x, wr, rb, routed, shared, top_k=2, n_shared=0, dispatch_fp8=True)
    b = oracle.layer_forward(x, wr, rb, routed, shared, top_k=2, n_shared=0)
    assert np.array_equal(a["y"], b["y"])
