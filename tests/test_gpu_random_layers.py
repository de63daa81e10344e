"""Seeded random small layers through moe_layer_forward against the oracle.

Shapes, dtypes, capacity factors, router biases (in the logit or for the
selection only), expert biases and the FP8 dispatch are drawn from a fixed
generator, inside the interface limits: T from one token to a few tiles with a
ragged tail, N from 1 to 300 experts, any top-K up to min(N, 64), widths that
are multiples of 64 (bf16) or 16 (fp32), up to two shared experts.  Every
layer gets the checks of the hand-picked cases: routing outputs bit exact
(ids, counts, and from the workspace the logits, offsets, row_token, slot_row
and n_dropped; the FP8 codes, exponents and widened rows), gates within 1e-6,
y within the global and the per-row tolerance of the oracle's layer
(DeepSeekMoE explainer page, section 共有エキスパート機構, output equation)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import workloads.device  # noqa: F401

from test_gpu_parity import (ROW_TOL, TOL, bias_np, check_layer, host, providers_host, rel_l2,
                             row_rel_l2_max)
from test_gpu_fp8 import check_fp8_layer

pytestmark = pytest.mark.gpu


def random_layers(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        q = 64 if dtype == "bf16" else 16
        N = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 100, 256, 300]))
        K = int(rng.integers(1, min(N, 64) + 1))
        T = int(rng.choice([1, 7, 64, 129, 300, 777, 1500]))
        d = q * int(rng.integers(1, 512 // q + 1))
        f = q * int(rng.integers(1, 512 // q + 1))
        Ks = int(rng.integers(0, 3))
        cf = float(rng.choice([0.0, 0.0, 0.5, 1.0, 1.25, 2.0]))
        rb = str(rng.choice(["none", "gauss", "zipf"]))
        sel = rb != "none" and rng.random() < 0.3
        fp8 = dtype == "bf16" and rng.random() < 0.25
        eb = bool(rng.random() < 0.3)
        out.append(W.custom_workload(f"rnd{i}", T=T, d_model=d, n_routed=N, top_k=K, n_shared=Ks,
                                     d_ff=f, dtype=dtype, capacity_factor=cf, router_bias=rb,
                                     router_bias_var=0.5, zipf_s=1.1, selection_only_bias=sel,
                                     dispatch_fp8=fp8, expert_bias=eb,
                                     seed=int(rng.integers(0, 1000))))
    return out


LAYERS = random_layers(40, 2024)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_renormalised_amd import binding
    binding.lib()
    yield


@pytest.mark.parametrize("wl", LAYERS, ids=lambda w: w.name)
def test_random_layer_matches_oracle(wl):
    print(f"[random] {wl}", flush=True)
    dl = W.device.DeviceLayer(wl)
    dl.forward()
    torch.cuda.synchronize()
    if wl.dispatch_fp8:
        check_fp8_layer(dl, wl.name)
        return
    routed, shared = providers_host(wl)
    ref = oracle.layer_forward(host(dl.x), wl.w_router().numpy(), bias_np(wl), routed, shared,
                               top_k=wl.top_k, n_shared=wl.n_shared,
                               capacity_factor=wl.capacity_factor,
                               selection_only_bias=wl.selection_only_bias)
    if not wl.selection_only_bias:
        check_layer(dl, ref, wl)
        return
    # with the bias in the selection key only, the stored logits are the
    # unbiased ones; everything else as in check_layer
    assert np.array_equal(dl.topk_idx.cpu().numpy(), ref["topk_idx"])
    assert np.array_equal(dl.counts.cpu().numpy(), ref["counts"])
    assert np.abs(dl.topk_gate.cpu().numpy() - ref["gates"]).max() <= 1e-6
    r = dl.routing_from_workspace()
    assert np.array_equal(r["offsets"], ref["offsets"])
    assert np.array_equal(r["row_token"], ref["row_token"])
    assert np.array_equal(r["slot_row"], ref["slot_row"])
    assert r["n_dropped"] == ref["n_dropped"]
    y = host(dl.y)
    assert rel_l2(y, ref["y"]) <= TOL[wl.dtype]
    assert row_rel_l2_max(y, ref["y"]) <= ROW_TOL[wl.dtype]


def test_random_layers_cover_the_options():
    # the drawn set exercises every option at least once
    assert {w.dtype for w in LAYERS} == {"bf16", "f32"}
    assert any(w.dispatch_fp8 for w in LAYERS)
    assert any(w.selection_only_bias for w in LAYERS)
    assert any(w.capacity_factor > 0 for w in LAYERS)
    assert any(w.n_shared == 2 for w in LAYERS)
    assert any(w.T == 1 for w in LAYERS) and any(w.top_k > 32 for w in LAYERS)
