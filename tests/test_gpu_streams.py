"""Two layers on two streams at once.  The library keeps no state between
calls and each call works only in the workspace it is given, so layers
launched concurrently on different streams, each with its own workspace, must
give exactly what each gives alone on one stream (the layer is deterministic:
fixed-order routing and fixed reduction orders).  Streams keep the default
priority."""
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


PAIRS = [
    # a weight-streaming decode layer beside a 256x256-tile layer
    (W.get_workload("dsv3_decode"),
     W.custom_workload("streams_big", T=2048, d_model=1024, n_routed=8, top_k=2, n_shared=1,
                       d_ff=2048, dtype="bf16", router_bias="gauss", router_bias_var=0.5)),
    # two small layers of different kinds (capacity drops, FP8 dispatch, fp32)
    (W.custom_workload("streams_cap", T=700, d_model=256, n_routed=32, top_k=4, n_shared=1,
                       d_ff=320, dtype="bf16", capacity_factor=1.0, dispatch_fp8=True),
     W.custom_workload("streams_f32", T=300, d_model=128, n_routed=16, top_k=3, n_shared=2,
                       d_ff=96, dtype="f32", expert_bias=True)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0].name}+{p[1].name}")
def test_concurrent_layers_on_two_streams_equal_their_single_runs(pair):
    print(f"[streams] {pair[0].name} + {pair[1].name}", flush=True)
    a, b = (W.device.DeviceLayer(wl) for wl in pair)
    outs = []
    for dl in (a, b):
        dl.forward()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (dl.y, dl.topk_idx, dl.topk_gate, dl.counts)])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(3):
        for dl in (a, b):
            dl.y.fill_(float("nan"))
            dl.topk_idx.fill_(-1)
        torch.cuda.synchronize()
        # both layers in flight together: each stream gets its own layer, and
        # each layer is issued several times so that the two overlap
        for _ in range(3):
            a.forward(s1)
            b.forward(s2)
        torch.cuda.synchronize()
        for dl, ref in ((a, outs[0]), (b, outs[1])):
            got = (dl.y, dl.topk_idx, dl.topk_gate, dl.counts)
            assert all(torch.equal(g, e) for g, e in zip(got, ref)), f"round {r}"
