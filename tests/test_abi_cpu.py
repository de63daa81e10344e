"""The C library loads, exports every declared entry point, and rejects bad
arguments on the host (no GPU needed: validation happens before any launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def B():
    from sparse_mixture_experts_renormalised_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    binding.lib()
    return binding


def test_every_declared_symbol_is_exported(B):
    names = declared_functions()
    assert "moe_layer_forward" in names and "moe_route" in names
    for n in names:
        assert hasattr(B.lib(), n), n
    assert set(names) == set(B.EXPORTS)


def test_version_and_status_strings(B):
    assert B.lib().moe_version() == B.INTERFACE_VERSION == 0x000200
    assert B.lib().moe_status_string(0) == b"ok"
    assert B.lib().moe_status_string(-3).startswith(b"workspace")


def test_capacity_rule(B):
    assert B.capacity(B.config(128, 7168, 256, 8, 1, 2048, "bf16", 1.25)) == 5
    assert B.capacity(B.config(10, 64, 3, 2, 0, 64, "bf16", 1.0)) == 7
    assert B.capacity(B.config(10, 64, 3, 2, 0, 64, "bf16", 0.0)) == -1
    assert B.capacity(B.config(10, 64, 3, 2, 0, 64, "bf16", 1.0, 0)) == 0


def call_status(fn, *args):
    try:
        fn(*args)
    except Exception as e:     # MoeError carries the status
        return getattr(e, "status", None)
    return 0


def test_invalid_arguments_are_rejected_before_launch(B):
    L = B.lib()
    P = ctypes.c_void_p
    good = B.config(64, 128, 8, 2, 0, 256, "bf16")
    # K > N, K = 0, N too large, bad dtype, unaligned widths
    for cfg, want in [(B.config(64, 128, 4, 5, 0, 256, "bf16"), -1),
                      (B.config(64, 128, 4, 0, 0, 256, "bf16"), -1),
                      (B.config(64, 128, 2048, 2, 0, 256, "bf16"), -2),
                      (B.config(64, 100, 8, 2, 0, 256, "bf16"), -2),
                      (B.config(64, 128, 8, 2, 0, 96, "bf16"), -2),
                      (B.config(64, 128, 8, 2, 65, 256, "bf16"), -2),
                      (B.config(-1, 128, 8, 2, 0, 256, "bf16"), -1)]:
        assert L.moe_layer_forward(ctypes.byref(cfg), None, None, None, None, None, None, None,
                                   0, None) == want
    bad = B.config(64, 128, 8, 2, 0, 256, "bf16")
    bad.dtype = 7
    assert L.moe_route(ctypes.byref(bad), None, None, None, None, None, None, None) == -1
    # NULL pointers and missing workspace
    assert L.moe_route(ctypes.byref(good), None, None, None, None, None, None, None) == -1
    assert L.moe_permute(ctypes.byref(good), P(16), None, P(16), P(16), P(16), P(16), P(16),
                         None, None, 0, None) == -3
    w = B.Weights()
    assert L.moe_layer_forward(ctypes.byref(good), ctypes.byref(w), P(16), P(16), None, None,
                               None, None, 0, None) == -1
    w.w_router = w.w1 = w.w2 = 4096
    assert L.moe_layer_forward(ctypes.byref(good), ctypes.byref(w), P(4096), P(4096), None, None,
                               None, None, 0, None) == -3
    # misaligned device pointer
    assert L.moe_layer_forward(ctypes.byref(good), ctypes.byref(w), P(4100), P(4096), None, None,
                               None, None, 1 << 30, P(4096)) == -1
    # misaligned shared-expert weights and biases (every device pointer is
    # 16-byte aligned; the epilogues read biases as 8-byte pairs)
    sh = B.config(64, 128, 8, 2, 1, 256, "bf16")
    for field in ("ws1", "ws2", "b1", "b2", "bs1", "bs2", "router_bias"):
        w2 = B.Weights(w_router=4096, w1=4096, w2=4096, ws1=4096, ws2=4096)
        setattr(w2, field, 4104)
        assert L.moe_layer_forward(ctypes.byref(sh), ctypes.byref(w2), P(4096), P(4096), None,
                                   None, None, P(4096), 1 << 30, None) == -1, field
    # optional routing outputs too
    w3 = B.Weights(w_router=4096, w1=4096, w2=4096, ws1=4096, ws2=4096)
    assert L.moe_layer_forward(ctypes.byref(sh), ctypes.byref(w3), P(4096), P(4096), P(4100),
                               None, None, P(4096), 1 << 30, None) == -1
    # grouped FFN argument checks
    assert L.moe_grouped_ffn(ctypes.byref(good), 0, None, None, 10, None, None, None, None, None,
                             None, None, 0, None) == -1
    assert L.moe_grouped_ffn(ctypes.byref(good), 3, None, None, 10, None, None, None, None, None,
                             None, None, 0, None) == -1
    # misaligned bias of the grouped FFN
    for b1, b2 in ((P(4100), None), (None, P(4104))):
        assert L.moe_grouped_ffn(ctypes.byref(good), 3, P(4096), P(4096), 10, P(4096), b1,
                                 P(4096), b2, P(4096), P(4096), None, 0, None) == -1
    # combine needs shared outputs when shared experts exist
    sh = B.config(64, 128, 8, 2, 2, 256, "bf16")
    assert L.moe_combine(ctypes.byref(sh), P(16), P(16), P(16), None, P(16), None) == -1


def test_top_k_limit(B):
    # top_k <= 64: slot k of a token lives in lane k of one wave
    L = B.lib()
    w = B.Weights()
    assert L.moe_layer_forward(ctypes.byref(B.config(64, 128, 100, 65, 0, 256, "bf16")),
                               ctypes.byref(w), None, None, None, None, None, None, 0, None) == -2
    assert L.moe_route(ctypes.byref(B.config(64, 128, 100, 65, 0, 256, "bf16")), None, None, None,
                       None, None, None, None) == -2
    assert B.workspace_size(B.config(64, 128, 100, 65, 0, 256, "bf16")) == 0
    assert B.workspace_size(B.config(64, 128, 100, 64, 0, 256, "bf16")) > 0


def test_workspace_layout(B):
    cfg = B.config(333, 128, 16, 4, 1, 256, "bf16")
    lay = B.workspace_layout(cfg)
    assert lay.total == B.workspace_size(cfg)
    T, N, K = 333, 16, 4
    regions = sorted([(lay.logits, T * N * 4), (lay.topk_idx, T * K * 4), (lay.topk_gate, T * K * 4),
                      (lay.counts, N * 4), (lay.offsets, (N + 1) * 4), (lay.n_dropped, 4),
                      (lay.row_token, T * K * 4), (lay.slot_row, T * K * 4)])
    # 256-aligned, disjoint, inside the workspace
    for (o, n), (o2, _) in zip(regions, regions[1:] + [(lay.total, 0)]):
        assert o % 256 == 0 and o + n <= o2
    assert lay.x_fp8 == lay.x_fp8_exp == lay.x_fp8_wide == 0   # bf16 dispatch
    with pytest.raises(B.MoeError):
        B.workspace_layout(B.config(64, 128, 4, 5, 0, 256, "bf16"))


def test_workspace_layout_fp8_dispatch(B):
    T, d, N, K = 333, 128, 16, 4
    cfg = B.config(T, d, N, K, 1, 256, "bf16", dispatch_fp8=True)
    lay = B.workspace_layout(cfg)
    assert lay.total == B.workspace_size(cfg)
    assert lay.total > B.workspace_size(B.config(T, d, N, K, 1, 256, "bf16"))
    regions = sorted([(lay.logits, T * N * 4), (lay.topk_idx, T * K * 4), (lay.topk_gate, T * K * 4),
                      (lay.counts, N * 4), (lay.offsets, (N + 1) * 4), (lay.n_dropped, 4),
                      (lay.row_token, T * K * 4), (lay.slot_row, T * K * 4),
                      (lay.x_fp8, T * d), (lay.x_fp8_exp, T * 4), (lay.x_fp8_wide, T * d * 2)])
    for (o, n), (o2, _) in zip(regions, regions[1:] + [(lay.total, 0)]):
        assert o % 256 == 0 and o + n <= o2


def test_empty_batch_is_a_no_op(B):
    L = B.lib()
    cfg = B.config(0, 128, 8, 2, 0, 256, "bf16")
    w = B.Weights()
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), None, None, None, None, None,
                               None, 0, None) == 0
    assert L.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None) == 0


def test_workspace_sizes_grow_with_the_layer(B):
    small = B.workspace_size(B.config(64, 128, 8, 2, 0, 256, "f32"))
    big = B.workspace_size(B.config(4096, 7168, 256, 8, 1, 2048, "bf16"))
    assert 0 < small < big
    # hidden + expert outputs of every assignment dominate: T*K*(d+f) act elements
    assert big >= 4096 * 8 * (7168 + 2048) * 2
    assert B.workspace_size(B.config(64, 128, 8, 9, 0, 256, "f32")) == 0


def test_grouped_ffn_split_workspace_size(B):
    bf = B.config(128, 7168, 256, 8, 1, 2048, "bf16")
    n = B.grouped_ffn_workspace_size(bf, 256, 1024)
    # one int, the last-round piece tiles (256 workgroups x 128 x 256 float32),
    # then up to 8 float32 partial sums of every row x max(d, f)
    assert n == 256 + 256 * 128 * 256 * 4 + 4 * 8 * 1024 * 7168
    # large products only split the last round of 256x256 tiles: one float32
    # tile per workgroup of up to 256
    assert B.grouped_ffn_workspace_size(bf, 256, 1 << 20) == 256 * 256 * 256 * 4
    f32 = B.config(64, 128, 8, 2, 0, 256, "f32")
    assert B.grouped_ffn_workspace_size(f32, 8, 128) == 0
    assert B.grouped_ffn_workspace_size(bf, 0, 1024) == 0


def test_bias_mode_is_validated(B):
    L = B.lib()
    bad = B.config(64, 128, 8, 2, 0, 256, "f32")
    bad.bias_mode = 2
    assert L.moe_route(ctypes.byref(bad), None, None, None, None, None, None, None) == -1
    ok = B.config(64, 128, 8, 2, 0, 256, "f32", selection_only_bias=True)
    assert ok.bias_mode == 1
    # balance statistics: missing pointers and workspace
    assert L.moe_balance_stats(ctypes.byref(ok), None, None, 0.01, None, None, None, None, 0,
                               None) == -1
    P = ctypes.c_void_p
    assert L.moe_balance_stats(ctypes.byref(ok), P(16), P(16), 0.01, P(16), P(16), P(16), None, 0,
                               None) == -3
    assert B.balance_stats_workspace_size(ok) == 4 * 8   # one 64-token block x N floats


def test_missing_library_fails_loudly(tmp_path):
    # the product path has no fallback: without the built library, loading raises
    import subprocess
    import sys
    code = ("from sparse_mixture_experts_renormalised_amd import binding\n"
            "try:\n"
            "    binding.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, MOE_MI355X_LIB=str(tmp_path / "absent.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("raised:"), out.stdout


def test_package_never_imports_the_oracle():
    # the oracle is test infrastructure: no module of the package may reach it
    import re
    pkg = os.path.join(ROOT, "sparse_mixture_experts_renormalised_amd")
    pat = re.compile(r"^\s*(import\s+oracle\b|from\s+oracle\b|from\s+\.\.\s*import\s+oracle)", re.M)
    hits = []
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                path = os.path.join(dirpath, f)
                with open(path) as fh:
                    if pat.search(fh.read()):
                        hits.append(path)
    assert not hits, hits
