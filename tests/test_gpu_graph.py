"""The layer under HIP graph capture: moe_layer_forward (caller workspace) and
moe_layer_forward_noalloc (the library's static array) captured once and
replayed three times, with eager layer calls and synchronisations between the
replays; every replay's outputs must equal the eager call's bit for bit (the
layer is deterministic: fixed-order routing, fixed reduction orders).  The
library records no memset and allocates nothing during a call, so a captured
call holds kernel launches only."""
import pytest
import torch

import workloads as W
import workloads.device  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_renormalised_amd import binding
    binding.lib()
    yield


CASES = [
    W.get_workload("dsv3_decode"),
    W.custom_workload("graph_bf16", T=300, d_model=256, n_routed=16, top_k=4, n_shared=1,
                      d_ff=320, dtype="bf16", router_bias="gauss", router_bias_var=0.5,
                      capacity_factor=1.25),
    W.custom_workload("graph_fp8", T=200, d_model=256, n_routed=16, top_k=4, n_shared=1,
                      d_ff=256, dtype="bf16", dispatch_fp8=True),
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_captured_layer_replays_equal_the_eager_call(wl, noalloc):
    from sparse_mixture_experts_renormalised_amd import binding as B
    print(f"[graph] {wl.name} noalloc={noalloc}", flush=True)
    dl = W.device.DeviceLayer(wl)

    def call(stream=None):
        if noalloc:
            B.layer_forward_noalloc(dl.cfg, dl.weights, dl.x, dl.y, dl.topk_idx, dl.topk_gate,
                                    dl.counts, stream)
        else:
            dl.forward(stream)

    call()          # eager (and, for noalloc, the array's address looked up first)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dl.y, dl.topk_idx, dl.topk_gate, dl.counts)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(3):
        dl.y.fill_(float("nan"))
        dl.topk_idx.fill_(-1)
        dl.topk_gate.fill_(float("nan"))
        dl.counts.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (dl.y, dl.topk_idx, dl.topk_gate, dl.counts)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {r}"
        call()      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(dl.y, ref[0])
    del g
