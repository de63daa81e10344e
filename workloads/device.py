"""Device-resident instance of a workload for the HIP library.

Fills every input tensor on the GPU with the seeded generator (same bits as
the host), allocates the outputs and the library workspace, and calls the
library through its binding.  Plumbing only: no layer arithmetic here.
"""
from __future__ import annotations

from typing import Optional

import torch

from sparse_mixture_experts_renormalised_amd import binding as B

from . import Workload


class DeviceLayer:
    def __init__(self, wl: Workload, device="cuda", with_stages: bool = False):
        self.wl = wl
        self.dev = torch.device(device)
        dev = self.dev
        self.act = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.cfg = B.config(wl.T, wl.d_model, wl.n_routed, wl.top_k, wl.n_shared, wl.d_ff,
                            wl.dtype, wl.capacity_factor,
                            selection_only_bias=wl.selection_only_bias,
                            dispatch_fp8=wl.dispatch_fp8)
        self.x = wl.x(dev)
        self.w_router = wl.w_router(dev)
        self.router_bias = wl.router_bias_values(dev)
        self.w1, self.b1, self.w2, self.b2 = wl.stacked(False, dev)
        if wl.n_shared > 0:
            self.ws1, self.bs1, self.ws2, self.bs2 = wl.stacked(True, dev)
        else:
            self.ws1 = self.bs1 = self.ws2 = self.bs2 = None
        self.weights = B.weights(self.w_router, self.router_bias, self.w1, self.b1, self.w2,
                                 self.b2, self.ws1, self.bs1, self.ws2, self.bs2)
        T, K, N, d = wl.T, wl.top_k, wl.n_routed, wl.d_model
        self.y = torch.zeros((T, d), dtype=self.act, device=dev)
        self.topk_idx = torch.zeros((T, K), dtype=torch.int32, device=dev)
        self.topk_gate = torch.zeros((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.zeros((N,), dtype=torch.int32, device=dev)
        self.ws = torch.empty((max(1, B.workspace_size(self.cfg)),), dtype=torch.uint8,
                              device=dev)

    def forward(self, stream=None):
        B.layer_forward(self.cfg, self.weights, self.x, self.y, self.topk_idx, self.topk_gate,
                        self.counts, self.ws, stream)
        return self.y

    def forward_events(self, events, stream=None):
        B.layer_forward_events(self.cfg, self.weights, self.x, self.y, events, self.topk_idx,
                               self.topk_gate, self.counts, self.ws, stream)
        return self.y

    def routing_from_workspace(self):
        """The layer's own routing arrays, read back from its workspace (the
        regions moe_workspace_layout names), as host numpy arrays."""
        wl = self.wl
        T, K, N = wl.T, wl.top_k, wl.n_routed
        lay = B.workspace_layout(self.cfg)

        def region(off, n, dtype):
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return self.ws[off:off + nbytes].view(dtype).cpu().numpy()

        offsets = region(lay.offsets, N + 1, torch.int32)
        R = int(offsets[-1])
        out = {}
        if lay.x_fp8:
            out["fp8_codes"] = region(lay.x_fp8, T * wl.d_model, torch.uint8).reshape(T, wl.d_model)
            out["fp8_exp"] = region(lay.x_fp8_exp, T, torch.int32)
            out["fp8_wide"] = region(lay.x_fp8_wide, T * wl.d_model,
                                     torch.int16).reshape(T, wl.d_model)
        return out | {
            "logits": region(lay.logits, T * N, torch.float32).reshape(T, N),
            "offsets": offsets,
            "n_dropped": int(region(lay.n_dropped, 1, torch.int32)[0]),
            "row_token": region(lay.row_token, T * K, torch.int32)[:R],
            "slot_row": region(lay.slot_row, T * K, torch.int32).reshape(T, K),
        }

    def expert_host(self, e: int, shared: bool = False):
        """One expert's tensors copied to the host as float32 numpy (None for absent bias)."""
        src = (self.ws1, self.bs1, self.ws2, self.bs2) if shared else (self.w1, self.b1, self.w2, self.b2)
        return tuple(None if t is None else t[e].float().cpu().numpy() for t in src)


def stage_tensors(wl: Workload, device="cuda"):
    """Output buffers for calling the entry points one at a time."""
    dev = torch.device(device)
    act = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    T, K, N, d, f = wl.T, wl.top_k, wl.n_routed, wl.d_model, wl.d_ff
    R = T * K
    return {
        "logits": torch.zeros((T, N), dtype=torch.float32, device=dev),
        "topk_idx": torch.zeros((T, K), dtype=torch.int32, device=dev),
        "topk_gate": torch.zeros((T, K), dtype=torch.float32, device=dev),
        "counts": torch.zeros((N,), dtype=torch.int32, device=dev),
        "offsets": torch.zeros((N + 1,), dtype=torch.int32, device=dev),
        "row_token": torch.full((max(R, 1),), -7, dtype=torch.int32, device=dev),
        "slot_row": torch.full((max(R, 1),), -7, dtype=torch.int32, device=dev),
        "n_dropped": torch.zeros((1,), dtype=torch.int32, device=dev),
        "x_perm": torch.zeros((max(R, 1), d), dtype=act, device=dev),
        "h": torch.zeros((max(R, 1), f), dtype=act, device=dev),
        "y_rows": torch.zeros((max(R, 1), d), dtype=act, device=dev),
        "y": torch.zeros((T, d), dtype=act, device=dev),
    }
