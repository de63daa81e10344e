"""FP8 dispatch (MOE_DISPATCH_FP8) of the HIP library against the oracle's
reading of it (DeepEP page, section "DeepEP とは？" item 5, and section
"DeepEP の性能": FP8 dispatch, BF16 combine): E4M3 codes, per-row
exponents and the rows widened back to bf16 bit exact, routing bit exact, y within the bf16 tolerance of the
oracle's layer on the dispatched rows (all of [T, d] and every row), on small
layers, on rows that use every code, and on the four large workloads at full
size.  The FP8 layer's distance from the bf16 dispatch is bounded by the
format's half step (2^-4 relative)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import workloads.device  # noqa: F401

from test_gpu_parity import ROW_TOL, TOL, host, rel_l2, row_rel_l2_max

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_renormalised_amd import binding
    binding.lib()
    yield


def expert64(dl, e, shared=False):
    src = (dl.ws1, dl.bs1, dl.ws2, dl.bs2) if shared else (dl.w1, dl.b1, dl.w2, dl.b2)
    return tuple(None if t is None else t[e].double().cpu().numpy() for t in src)


def check_fp8_layer(dl, label):
    wl = dl.wl
    ref = oracle.layer_forward(host(dl.x), host(dl.w_router),
                               None if dl.router_bias is None else host(dl.router_bias),
                               lambda e: expert64(dl, e), lambda i: expert64(dl, i, True),
                               top_k=wl.top_k, n_shared=wl.n_shared,
                               capacity_factor=wl.capacity_factor,
                               selection_only_bias=wl.selection_only_bias, dispatch_fp8=True)
    r = dl.routing_from_workspace()
    assert np.array_equal(r["fp8_exp"], ref["fp8_exp"]), label
    assert np.array_equal(r["fp8_codes"], ref["fp8_codes"]), label
    # the rows the first Linear reads: every code widened to 2^E times its
    # value, which bf16 holds exactly, so they compare bit for bit
    wide = torch.from_numpy(oracle.dequantize_fp8_rows(ref["fp8_exp"], ref["fp8_codes"]))
    assert np.array_equal(r["fp8_wide"], wide.to(torch.bfloat16).view(torch.int16).numpy()), label
    assert np.array_equal(dl.topk_idx.cpu().numpy(), ref["topk_idx"]), label
    assert np.array_equal(dl.counts.cpu().numpy(), ref["counts"]), label
    assert np.array_equal(r["slot_row"], ref["slot_row"]), label
    y = host(dl.y)
    err, row = rel_l2(y, ref["y"]), row_rel_l2_max(y, ref["y"])
    print(f"[fp8] {label}: rel_l2={err:.3e} max_row_rel_l2={row:.3e}", flush=True)
    assert err <= TOL["bf16"] and row <= ROW_TOL["bf16"], label
    return ref


SMALL = [
    W.custom_workload("fp8_small", T=333, d_model=128, n_routed=16, top_k=4, n_shared=1,
                      d_ff=256, dtype="bf16", router_bias="gauss", router_bias_var=0.5,
                      dispatch_fp8=True),
    # decode-sized groups (the weight-streaming kernel, with capacity drops)
    W.custom_workload("fp8_decode_like", T=64, d_model=512, n_routed=64, top_k=6, n_shared=1,
                      d_ff=192, dtype="bf16", router_bias="zipf", zipf_s=1.1,
                      capacity_factor=1.25, dispatch_fp8=True),
    # groups of more than 128 rows (the 256x256 kernel), ragged, two shared experts
    W.custom_workload("fp8_big_groups", T=700, d_model=256, n_routed=4, top_k=2, n_shared=2,
                      d_ff=320, dtype="bf16", expert_bias=True, dispatch_fp8=True),
    W.custom_workload("fp8_T1", T=1, d_model=128, n_routed=8, top_k=2, n_shared=0, d_ff=128,
                      dtype="bf16", dispatch_fp8=True),
    # capacity drops and a selection-only bias: the codes of every token are
    # produced, only kept slots are computed
    W.custom_workload("fp8_sel_only_cap", T=256, d_model=256, n_routed=32, top_k=4, n_shared=1,
                      d_ff=128, dtype="bf16", router_bias="gauss", router_bias_var=0.5,
                      selection_only_bias=True, capacity_factor=1.0, dispatch_fp8=True),
    W.custom_workload("fp8_N1024_K64", T=150, d_model=64, n_routed=1024, top_k=64, n_shared=1,
                      d_ff=64, dtype="bf16", capacity_factor=1.5, dispatch_fp8=True),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_fp8_small_layers(wl):
    dl = W.device.DeviceLayer(wl)
    dl.forward()
    torch.cuda.synchronize()
    check_fp8_layer(dl, wl.name)


def test_fp8_rows_using_every_code():
    # token rows made of every finite E4M3 value (both signs, subnormals,
    # zeros) times a per-row power of two, largest element 448 * 2^E: the
    # codes must come back exactly, and the layer must match the oracle
    wl = W.custom_workload("fp8_codes", T=96, d_model=256, n_routed=8, top_k=2, n_shared=1,
                           d_ff=128, dtype="bf16", dispatch_fp8=True)
    dl = W.device.DeviceLayer(wl)
    vals = oracle.e4m3_values()
    finite = np.array([c for c in range(256) if np.isfinite(vals[c])])
    rng = np.random.default_rng(5)
    x = np.empty((96, 256))
    E = rng.integers(-14, -4, 96)
    for t in range(96):
        row = vals[np.resize(np.roll(finite, 3 * t), 256)].copy()
        row[np.resize(np.roll(finite, 3 * t), 256) == 0x80] = -0.0
        row[0] = 448.0
        x[t] = row * 2.0 ** E[t]
    dl.x.copy_(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    assert torch.equal(dl.x.double().cpu(), torch.from_numpy(x))     # exact in bf16
    dl.forward()
    torch.cuda.synchronize()
    ref = check_fp8_layer(dl, "every code")
    assert np.array_equal(ref["fp8_exp"], E)
    assert len(np.unique(ref["fp8_codes"])) == len(finite)


@pytest.mark.parametrize("name", ["mixtral_shape", "deepseekmoe_fine", "dsv3_prefill",
                                  "dsv3_decode"])
def test_fp8_full_size(name):
    wl = W.get_workload(name).with_(dispatch_fp8=True)
    print(f"[fp8] full-size {name}", flush=True)
    dl = W.device.DeviceLayer(wl)
    dl.forward()
    torch.cuda.synchronize()
    check_fp8_layer(dl, f"full-size {name}")
    # against the bf16 dispatch of the same layer: the format's half step
    y8 = dl.y.clone()
    dl.cfg.dispatch = 0
    dl.forward()
    torch.cuda.synchronize()
    d = rel_l2(host(y8), host(dl.y))
    print(f"[fp8] {name}: rel_l2 to the bf16 dispatch {d:.3e}", flush=True)
    assert 1e-3 < d <= 2.0 ** -4
