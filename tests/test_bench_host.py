"""Host-side checks of bench.py: the one-GPU guard, the algorithmic work
figures the roofline is computed from, and the staleness rule of the
committed traffic counters.  No GPU needed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stage_work_mixtral_shape_closed_forms():
    # Mixtral-shaped layer: T = 4096 tokens, top-2 of 8 experts, no capacity
    # limit, so R = 8192 kept assignments and all 8 experts are touched.
    wl = W.get_workload("mixtral_shape")
    T, d, N, K, f = wl.T, wl.d_model, wl.n_routed, wl.top_k, wl.d_ff
    R = T * K
    work = bench.stage_work(wl, kept_rows=R, touched=N)
    # each expert Linear is 2·R·d·f flops; the two together are the 4·R·d·f of
    # the routed FFN (1,924,145,348,608 for this shape)
    assert work["up"]["flops"] == work["down"]["flops"] == 2 * R * d * f
    assert work["up"]["flops"] + work["down"]["flops"] == 1_924_145_348_608
    # weights read once per touched expert (bf16), plus rows in and out
    w_bytes = N * f * d * 2
    assert w_bytes == 939_524_096                 # one Linear of all 8 experts (1.879 GB for both)
    assert work["up"]["bytes"] == w_bytes + R * (d + f) * 2 + R * 4
    assert work["down"]["bytes"] == w_bytes + R * (d + f) * 2
    assert work["router"]["flops"] == 2 * T * d * N == 268_435_456


def test_stage_work_counts_only_touched_experts():
    wl = W.get_workload("dsv3_decode")
    few = bench.stage_work(wl, kept_rows=200, touched=60)
    more = bench.stage_work(wl, kept_rows=200, touched=61)
    per_expert = wl.d_model * wl.d_ff * 2
    assert more["up"]["bytes"] - few["up"]["bytes"] == per_expert
    assert more["down"]["bytes"] - few["down"]["bytes"] == per_expert
    # the shared expert runs on all T tokens and its weights are always read
    assert few["up"]["flops"] == 2 * (200 + wl.n_shared * wl.T) * wl.d_model * wl.d_ff


def test_traffic_is_null_unless_taken_on_this_source(tmp_path, monkeypatch):
    sha = bench.source_sha()
    good = {"mixtral_shape": {"up": {"fetch_bytes": 10.0, "write_bytes": 2.0, "source_sha": sha}},
            "dsv3_decode": {"up": {"fetch_bytes": 10.0, "write_bytes": 2.0,
                                   "source_sha": "0" * 16}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("mixtral_shape", "up") == 12.0
    assert bench.measured_traffic("mixtral_shape", "down") is None
    assert bench.measured_traffic("dsv3_decode", "up") is None      # other source
    assert bench.measured_traffic("deepseekmoe_fine", "up") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("mixtral_shape", "up") is None


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_every_workload_has_a_cpu_sample(name):
    assert bench.CPU_SAMPLE[name] >= 1


def test_roofline_reports_both_roofs():
    # an HBM-bound stage (prefill-shaped: 128 mean rows per expert, below the
    # 312.5 flop/byte ridge) also gets its MFMA share, and an MFMA-bound one
    # (Mixtral-shaped) its HBM share, from the same work and time
    for name, kept, touched, bound in (("dsv3_prefill", 32768, 241, "hbm"),
                                       ("mixtral_shape", 8192, 8, "mfma")):
        wl = W.get_workload(name)
        work = bench.stage_work(wl, kept, touched)
        ms = {"up": 2.0, "down": 1.0}
        roof = bench.roofline(wl, work, ms)
        assert roof["bound"] == bound and roof["kernel"].endswith("(up)")
        t = 2.0e-3
        flops_frac = work["up"]["flops"] / t / 1e12 / bench.PEAK_BF16_TFLOPS
        bytes_frac = work["up"]["bytes"] / t / 1e9 / bench.PEAK_HBM_GBS
        main, other = (bytes_frac, flops_frac) if bound == "hbm" else (flops_frac, bytes_frac)
        assert roof["frac"] == pytest.approx(main, rel=1e-12)
        assert roof["other_roof"]["frac"] == pytest.approx(other, rel=1e-12)
        assert roof["other_roof"]["unit"] == ("TFLOP/s" if bound == "hbm" else "GB/s")
