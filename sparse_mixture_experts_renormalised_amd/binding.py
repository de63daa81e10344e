"""ctypes binding of libmoe_mi355x.so (argument marshalling only).

The functions keep the C names without the ``moe_`` prefix and take torch
tensors that already live on the GPU; every step of the layer runs in the
library's HIP kernels.  Each call enqueues work on the current torch stream
(or the stream given) and returns after the launches, like the C calls.  A
non-zero status raises :class:`MoeError`.  When the library has not been
built, loading fails loudly; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB names another build of the same library (for example a
# second build kept for side-by-side timing); the default is the in-tree one.
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(HERE, "_lib", "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported size", -3: "workspace", -4: "HIP error"}

# Symbols declared in include/moe_mi355x.h.
EXPORTS = ("moe_route", "moe_permute", "moe_permute_workspace_size", "moe_grouped_ffn",
           "moe_grouped_ffn_workspace_size", "moe_combine", "moe_balance_stats",
           "moe_balance_stats_workspace_size", "moe_layer_forward", "moe_layer_forward_events",
           "moe_layer_forward_noalloc", "moe_workspace_size", "moe_workspace_layout",
           "moe_capacity", "moe_status_string", "moe_version")
STAGES = ("router", "topk", "dispatch", "up", "down", "combine")
# moe_version() of the interface these ctypes declarations mirror (the structs
# below must match the header's field for field)
INTERFACE_VERSION = 0x000200


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


class Config(ctypes.Structure):
    """Mirror of moe_config."""
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("capacity", ctypes.c_int32), ("bias_mode", ctypes.c_int32),
                ("dispatch", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    """Mirror of moe_ws_layout (byte offsets into the layer workspace)."""
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("logits", "topk_idx", "topk_gate", "counts", "offsets", "n_dropped", "row_token",
                 "slot_row", "x_fp8", "x_fp8_exp", "x_fp8_wide", "total")]


class Weights(ctypes.Structure):
    """Mirror of moe_weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "router_bias", "w1", "b1", "w2", "b2", "ws1", "bs1", "ws2", "bs2")]


_LIB = None


def lib():
    """Load the library once; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
        C = ctypes.POINTER(Config)
        sig = {
            "moe_route": (I, [C, P, P, P, P, P, P, P]),
            "moe_permute": (I, [C, P, P, P, P, P, P, P, P, P, Z, P]),
            "moe_permute_workspace_size": (Z, [C]),
            "moe_grouped_ffn": (I, [C, ctypes.c_int32, P, P, I64, P, P, P, P, P, P, P, Z, P]),
            "moe_grouped_ffn_workspace_size": (Z, [C, ctypes.c_int32, I64]),
            "moe_balance_stats": (I, [C, P, P, ctypes.c_float, P, P, P, P, Z, P]),
            "moe_balance_stats_workspace_size": (Z, [C]),
            "moe_combine": (I, [C, P, P, P, P, P, P]),
            "moe_layer_forward": (I, [C, ctypes.POINTER(Weights), P, P, P, P, P, P, Z, P]),
            "moe_layer_forward_events": (I, [C, ctypes.POINTER(Weights), P, P, P, P, P, P, Z,
                                             ctypes.POINTER(ctypes.c_void_p), P]),
            "moe_layer_forward_noalloc": (I, [C, ctypes.POINTER(Weights), P, P, P, P, P, P]),
            "moe_workspace_size": (Z, [C]),
            "moe_workspace_layout": (I, [C, ctypes.POINTER(WsLayout)]),
            "moe_capacity": (I64, [C]),
            "moe_status_string": (ctypes.c_char_p, [I]),
            "moe_version": (I, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        if L.moe_version() != INTERFACE_VERSION:
            raise RuntimeError(f"{LIB_PATH} implements interface {L.moe_version():#08x}, this "
                               f"binding {INTERFACE_VERSION:#08x}: rebuild the library")
        _LIB = L
    return _LIB


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn: str, st: int):
    if st != 0:
        raise MoeError(fn, st)


MOE_BIAS_IN_LOGIT, MOE_BIAS_SELECTION_ONLY = 0, 1
MOE_DISPATCH_BF16, MOE_DISPATCH_FP8 = 0, 1


def config(T, d_model, n_routed, top_k, n_shared, d_ff, dtype, capacity_factor=0.0,
           capacity=-1, selection_only_bias=False, dispatch_fp8=False) -> Config:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, MOE_F32: MOE_F32, MOE_BF16: MOE_BF16}[dtype]
    return Config(int(T), int(d_model), int(n_routed), int(top_k), int(n_shared), int(d_ff),
                  dt, float(capacity_factor), int(capacity),
                  MOE_BIAS_SELECTION_ONLY if selection_only_bias else MOE_BIAS_IN_LOGIT,
                  MOE_DISPATCH_FP8 if dispatch_fp8 else MOE_DISPATCH_BF16)


def capacity(cfg: Config) -> int:
    return int(lib().moe_capacity(ctypes.byref(cfg)))


def route(cfg: Config, x, w_router, router_bias, logits, topk_idx, topk_gate, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router),
                                        _ptr(router_bias), _ptr(logits), _ptr(topk_idx),
                                        _ptr(topk_gate), _stream(stream)))


def permute_workspace_size(cfg: Config) -> int:
    return int(lib().moe_permute_workspace_size(ctypes.byref(cfg)))


def permute(cfg: Config, topk_idx, x, counts, offsets, row_token, slot_row, n_dropped,
            x_perm, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_permute", lib().moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(x),
                                            _ptr(counts), _ptr(offsets), _ptr(row_token),
                                            _ptr(slot_row), _ptr(n_dropped), _ptr(x_perm),
                                            _ptr(ws), nbytes, _stream(stream)))


def grouped_ffn_workspace_size(cfg: Config, n_groups, max_rows) -> int:
    return int(lib().moe_grouped_ffn_workspace_size(ctypes.byref(cfg), int(n_groups), int(max_rows)))


def grouped_ffn(cfg: Config, n_groups, x_rows, offsets, max_rows, w1, b1, w2, b2, h, y_rows,
                ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(ctypes.byref(cfg), int(n_groups), _ptr(x_rows),
                                                    _ptr(offsets), int(max_rows), _ptr(w1),
                                                    _ptr(b1), _ptr(w2), _ptr(b2), _ptr(h),
                                                    _ptr(y_rows), _ptr(ws), nbytes,
                                                    _stream(stream)))


def balance_stats_workspace_size(cfg: Config) -> int:
    return int(lib().moe_balance_stats_workspace_size(ctypes.byref(cfg)))


def balance_stats(cfg: Config, logits, topk_idx, alpha, f, P, loss, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_balance_stats", lib().moe_balance_stats(ctypes.byref(cfg), _ptr(logits),
                                                        _ptr(topk_idx), float(alpha), _ptr(f),
                                                        _ptr(P), _ptr(loss), _ptr(ws), nbytes,
                                                        _stream(stream)))


def combine(cfg: Config, y_rows, slot_row, topk_gate, shared_out, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _ptr(y_rows), _ptr(slot_row),
                                            _ptr(topk_gate), _ptr(shared_out), _ptr(y),
                                            _stream(stream)))


def workspace_size(cfg: Config) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(cfg)))


def workspace_layout(cfg: Config) -> WsLayout:
    out = WsLayout()
    _check("moe_workspace_layout", lib().moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def weights(w_router, router_bias, w1, b1, w2, b2, ws1=None, bs1=None, ws2=None,
            bs2=None) -> Weights:
    return Weights(*[_ptr(t) for t in (w_router, router_bias, w1, b1, w2, b2, ws1, bs1, ws2, bs2)])


def layer_forward(cfg: Config, w: Weights, x, y, topk_idx=None, topk_gate=None, counts=None,
                  ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_layer_forward", lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w),
                                                        _ptr(x), _ptr(y), _ptr(topk_idx),
                                                        _ptr(topk_gate), _ptr(counts), _ptr(ws),
                                                        nbytes, _stream(stream)))


def layer_forward_noalloc(cfg: Config, w: Weights, x, y, topk_idx=None, topk_gate=None,
                          counts=None, stream=None):
    """layer_forward with the library's own static device scratch (no workspace)."""
    _check("moe_layer_forward_noalloc",
           lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(y),
                                           _ptr(topk_idx), _ptr(topk_gate), _ptr(counts),
                                           _stream(stream)))


def layer_forward_events(cfg: Config, w: Weights, x, y, events, topk_idx=None, topk_gate=None,
                         counts=None, ws=None, stream=None):
    """layer_forward recording ``events`` (len(STAGES)+1 hipEvent_t handles) per stage."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    arr = (ctypes.c_void_p * len(events))(*events)
    _check("moe_layer_forward_events",
           lib().moe_layer_forward_events(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(y),
                                          _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _ptr(ws),
                                          nbytes, arr, _stream(stream)))


class HipEvents:
    """Raw HIP events (created through the HIP runtime torch already loaded)."""

    def __init__(self, n: int):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self.rt.hipEventDestroy(h)
        self.handles = []
