"""Seeded synthetic inputs for the sparse top-K MoE FFN layer.

This module is shared by the CPU oracle's callers (tests, the CPU baseline) and
by the GPU harness.  It holds shapes, value distributions and one counter-based
generator, and nothing of the layer's own arithmetic: no routing, no capacity,
no expert evaluation.

Generator
---------
Every tensor is a pure function of (seed, tensor id, expert id, element index):

* a 32-bit key pair is derived from (seed, tensor id, expert id) with the
  integer mixer below;
* element ``i`` (flat index into the tensor's own slab, ``i < 2**32``) is hashed
  twice with that key pair, and the top 16 bits pick one of 65,536
  equiprobable quantiles of the standard normal, ``z_j = Phi^-1((j + 1/2)/65536)``;
* the quantile is scaled by the tensor's standard deviation in float64 and
  rounded once to float32 (round to nearest even), then, for bfloat16 tensors,
  to bfloat16 (round to nearest even).

The mixer is the two-round multiply/xor-shift 32-bit integer hash with the
odd multiplier 0x45D9F3B (Thomas Mueller's widely published "hash32"), run on
int64 containers so that every intermediate stays below 2**63.  Because only
integer operations and a table gather are involved, the same code gives the
same bits on the CPU and on the GPU (torch int64 arithmetic is exact on both),
so the GPU harness can fill multi-gigabyte expert stacks on the device while the
oracle regenerates the few experts it needs on the host.

The discretised normal has |z| <= 4.325 and exact mean zero; it stands in for
the Gaussian draws the workloads call for.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from statistics import NormalDist
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "custom_workload",
    "fill_normal", "quantile_table", "stream_keys", "mix32",
    "TENSOR_IDS", "bf16_bits_to_f32", "f32_to_bf16_bits",
]

M32 = 0xFFFFFFFF
_MULT = 0x45D9F3B

TENSOR_IDS = {
    "x": 1, "w_router": 2, "router_bias": 3,
    "w1": 4, "b1": 5, "w2": 6, "b2": 7,
    "ws1": 8, "bs1": 9, "ws2": 10, "bs2": 11,
}


def mix32(v):
    """32-bit integer mixer; works on Python ints and on int64 torch tensors.

    Inputs must lie in [0, 2**32); the output does too.  Each step is a
    bijection on 32-bit words (xor-shift, multiply by an odd constant).
    """
    v = v ^ (v >> 16)
    v = (v * _MULT) & M32
    v = v ^ (v >> 16)
    v = (v * _MULT) & M32
    v = v ^ (v >> 16)
    return v


def _mix32_(v: torch.Tensor) -> torch.Tensor:
    """In-place form of :func:`mix32` on an int64 tensor (same bits)."""
    v ^= v >> 16
    v.mul_(_MULT).bitwise_and_(M32)
    v ^= v >> 16
    v.mul_(_MULT).bitwise_and_(M32)
    v ^= v >> 16
    return v


def stream_keys(seed: int, tensor_id: int, expert_id: int = 0) -> tuple[int, int]:
    """Key pair of one tensor slab (Python ints in [0, 2**32))."""
    a = mix32((seed + 0x632BE5AB) & M32)
    a = mix32(a ^ (tensor_id & M32))
    a = mix32(a ^ ((expert_id + 1) & M32))
    b = mix32(a ^ 0x2545F491)
    return a, b


_Z64: Optional[np.ndarray] = None


def _normal_quantiles() -> np.ndarray:
    global _Z64
    if _Z64 is None:
        nd = NormalDist()
        _Z64 = np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)],
                        dtype=np.float64)
    return _Z64


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values (finite) to bfloat16, nearest even; returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_TABLES: dict = {}


def quantile_table(std: float, dtype: str) -> np.ndarray:
    """65,536 scaled quantiles: float32 values, or uint16 bfloat16 bit patterns."""
    key = (float(std), dtype)
    t = _TABLES.get(key)
    if t is None:
        v32 = (_normal_quantiles() * float(std)).astype(np.float32)
        if dtype == "f32":
            t = v32
        elif dtype == "bf16":
            t = f32_to_bf16_bits(v32)
        else:
            raise ValueError(dtype)
        _TABLES[key] = t
    return t


def fill_normal(shape, std: float, dtype: str, seed: int, tensor_id: int,
                expert_id: int = 0, device="cpu") -> torch.Tensor:
    """One seeded slab; identical bits on every device.

    Returns float32, or bfloat16 when ``dtype == "bf16"``.
    """
    n = 1
    for s in shape:
        n *= int(s)
    if n >= (1 << 32):
        raise ValueError("slab too large for a 32-bit element counter")
    ka, kb = stream_keys(seed, tensor_id, expert_id)
    dev = torch.device(device)
    table = quantile_table(std, dtype)
    if dtype == "bf16":
        ttab = torch.from_numpy(table.view(np.int16).copy()).to(dev)
    else:
        ttab = torch.from_numpy(table.copy()).to(dev)
    out = torch.empty(n, dtype=ttab.dtype, device=dev)
    chunk = 1 << 25
    for s0 in range(0, n, chunk):
        s1 = min(n, s0 + chunk)
        h = torch.arange(s0, s1, dtype=torch.int64, device=dev)
        h ^= ka
        _mix32_(h)
        h ^= kb
        _mix32_(h)
        h >>= 16
        out[s0:s1] = ttab[h]
        del h
    out = out.view(*shape)
    if dtype == "bf16":
        out = out.view(torch.bfloat16)
    return out


# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """Shapes and input distributions of one MoE layer instance.

    ``dtype`` is the activation / expert-weight type ("f32" or "bf16"); the
    router weight and router bias are always float32.  Variances follow the
    fan-in rule: W1, b1 use 1/d_model, W2, b2 use 1/d_ff, W_r uses 1/d_model.
    ``router_bias`` is "none", "gauss" (variance ``router_bias_var``) or
    "zipf" (deterministic, bias[e] = -s*ln(e+1)).
    ``capacity_factor <= 0`` means no per-expert limit.
    ``selection_only_bias`` marks a router bias that enters the selection key
    only (the gates then use the unbiased logits).  ``dispatch_fp8`` sends
    the routed experts' token rows as FP8 (E4M3 with a per-row scale).
    """
    name: str
    T: int
    d_model: int
    n_routed: int
    top_k: int
    n_shared: int
    d_ff: int
    dtype: str
    capacity_factor: float = 0.0
    expert_bias: bool = False
    router_bias: str = "none"
    router_bias_var: float = 0.0
    zipf_s: float = 0.0
    selection_only_bias: bool = False
    dispatch_fp8: bool = False
    seed: int = 0
    description: str = field(default="", compare=False)

    # ---- tensors -------------------------------------------------------
    def x(self, device="cpu") -> torch.Tensor:
        return fill_normal((self.T, self.d_model), 1.0, self.dtype, self.seed,
                           TENSOR_IDS["x"], 0, device)

    def w_router(self, device="cpu") -> torch.Tensor:
        return fill_normal((self.n_routed, self.d_model), math.sqrt(1.0 / self.d_model),
                           "f32", self.seed, TENSOR_IDS["w_router"], 0, device)

    def router_bias_values(self, device="cpu") -> Optional[torch.Tensor]:
        if self.router_bias == "none":
            return None
        if self.router_bias == "gauss":
            return fill_normal((self.n_routed,), math.sqrt(self.router_bias_var), "f32",
                               self.seed, TENSOR_IDS["router_bias"], 0, device)
        if self.router_bias == "zipf":
            e = np.arange(self.n_routed, dtype=np.float64)
            b = (-self.zipf_s * np.log(e + 1.0)).astype(np.float32)
            return torch.from_numpy(b).to(device)
        raise ValueError(self.router_bias)

    def _expert(self, e: int, shared: bool, device="cpu"):
        d, f = self.d_model, self.d_ff
        t1, tb1, t2, tb2 = (("ws1", "bs1", "ws2", "bs2") if shared else ("w1", "b1", "w2", "b2"))
        w1 = fill_normal((f, d), math.sqrt(1.0 / d), self.dtype, self.seed, TENSOR_IDS[t1], e, device)
        w2 = fill_normal((d, f), math.sqrt(1.0 / f), self.dtype, self.seed, TENSOR_IDS[t2], e, device)
        if self.expert_bias:
            b1 = fill_normal((f,), math.sqrt(1.0 / d), self.dtype, self.seed, TENSOR_IDS[tb1], e, device)
            b2 = fill_normal((d,), math.sqrt(1.0 / f), self.dtype, self.seed, TENSOR_IDS[tb2], e, device)
        else:
            b1 = b2 = None
        return w1, b1, w2, b2

    def routed_expert(self, e: int, device="cpu"):
        """(w1 [f,d], b1 [f] or None, w2 [d,f], b2 [d] or None) of routed expert e."""
        return self._expert(e, False, device)

    def shared_expert(self, i: int, device="cpu"):
        return self._expert(i, True, device)

    def stacked(self, shared: bool, device="cpu"):
        """All routed (or shared) experts stacked: w1 [G,f,d], b1 [G,f]|None, w2 [G,d,f], b2 [G,d]|None."""
        G = self.n_shared if shared else self.n_routed
        d, f = self.d_model, self.d_ff
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        w1 = torch.empty((G, f, d), dtype=tdt, device=device)
        w2 = torch.empty((G, d, f), dtype=tdt, device=device)
        b1 = torch.empty((G, f), dtype=tdt, device=device) if self.expert_bias else None
        b2 = torch.empty((G, d), dtype=tdt, device=device) if self.expert_bias else None
        for g in range(G):
            a1, c1, a2, c2 = self._expert(g, shared, device)
            w1[g].copy_(a1)
            w2[g].copy_(a2)
            if b1 is not None:
                b1[g].copy_(c1)
                b2[g].copy_(c2)
            del a1, a2, c1, c2
        return w1, b1, w2, b2

    # ---- bookkeeping ---------------------------------------------------
    @property
    def act_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", T=64, d_model=128, n_routed=8, top_k=2, n_shared=0, d_ff=256,
                 dtype="f32", expert_bias=True,
                 description="tiny layer, fp32, biased expert Linears, no capacity limit"),
        Workload("mixtral_shape", T=4096, d_model=4096, n_routed=8, top_k=2, n_shared=0,
                 d_ff=14336, dtype="bf16",
                 description="Mixtral-8x7B-shaped layer, bf16, 4096 tokens"),
        Workload("deepseekmoe_fine", T=4096, d_model=2048, n_routed=64, top_k=8, n_shared=2,
                 d_ff=1408, dtype="bf16",
                 description="DeepSeekMoE fine-grained layer (m=4 split of 16 experts), 2 shared"),
        Workload("dsv3_prefill", T=4096, d_model=7168, n_routed=256, top_k=8, n_shared=1,
                 d_ff=2048, dtype="bf16", router_bias="gauss", router_bias_var=0.5,
                 description="DeepSeek-V3-shaped prefill, 256 experts resident, imbalanced bias"),
        Workload("dsv3_decode", T=128, d_model=7168, n_routed=256, top_k=8, n_shared=1,
                 d_ff=2048, dtype="bf16", router_bias="zipf", zipf_s=1.1, capacity_factor=1.25,
                 description="DeepSeek-V3-shaped decode, Zipf-skewed bias, capacity factor 1.25"),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def custom_workload(name="custom", **kw) -> Workload:
    base = dict(T=64, d_model=128, n_routed=8, top_k=2, n_shared=0, d_ff=256, dtype="f32")
    base.update(kw)
    return Workload(name=name, **base)
