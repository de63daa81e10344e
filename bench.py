"""Benchmark of the MoE FFN layer forward on one MI355X.

One step = one full pass of the layer (router, top-K gates, dispatch, routed
and shared expert FFNs, combine) over one batch of seeded synthetic tokens
already resident in HBM, through the library's C interface.

Prints one JSON line with whole-job tokens/s, the per-stage times (HIP events
recorded by the library on the stream it launches on), the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; grouped-GEMM % MFMA peak; decode HBM GB/s (1 MI355X)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
DEFAULT_WORKLOAD = "mixtral_shape"
CPU_SAMPLE = {"tiny_fp32": 64, "mixtral_shape": 4096, "deepseekmoe_fine": 512,
              "dsv3_prefill": 64, "dsv3_decode": 128}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only copy 1 GiB device-to-device three times (counter calibration)")
    return p.parse_args()


GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_renormalised_amd", "csrc", "grouped_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_sha() -> str:
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of the stage's kernel, from committed counter runs.

    None when no measurement exists for this workload and stage, or when the
    GEMM source changed since the counters were taken.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(stage)
    if not e or e.get("source_sha") != source_sha():
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def stage_work(wl, kept_rows: int, touched: int):
    """Algorithmic flops and HBM bytes of each stage of one forward.

    Bytes count what the method must move once: activations in and out,
    the weights of experts that receive at least one token (untouched experts
    cost nothing), index arrays; not cache re-reads or padding rows.
    """
    T, d, f, N, K, Ks = wl.T, wl.d_model, wl.d_ff, wl.n_routed, wl.top_k, wl.n_shared
    a = wl.act_bytes
    R = kept_rows
    w1_bytes = (touched + Ks) * f * d * a + ((touched + Ks) * f * a if wl.expert_bias else 0)
    w2_bytes = (touched + Ks) * d * f * a + ((touched + Ks) * d * a if wl.expert_bias else 0)
    return {
        "router": {"flops": 2 * T * d * N, "bytes": T * d * a + N * d * 4 + T * N * 4},
        "topk": {"flops": 0, "bytes": T * N * 4 + T * K * 8},
        "dispatch": {"flops": 0, "bytes": T * K * 4 * 3 + R * 4},
        "up": {"flops": 2 * (R + Ks * T) * d * f,
               "bytes": w1_bytes + (R + Ks * T) * (d + f) * a + R * 4},
        "down": {"flops": 2 * (R + Ks * T) * d * f,
                 "bytes": w2_bytes + (R + Ks * T) * (d + f) * a},
        "combine": {"flops": 0, "bytes": (R + Ks * T + T) * d * a + T * K * 8},
    }


def cpu_baseline(dl, wl, n_sample: int):
    """The oracle as it stands, on n_sample tokens (routing over all T)."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(wl.T, size=min(n_sample, wl.T), replace=False))
    x = dl.x.float().cpu().numpy()
    wr = dl.w_router.cpu().numpy()
    rb = None if dl.router_bias is None else dl.router_bias.cpu().numpy()
    # inputs the oracle will need, staged on the host before timing
    idx = dl.topk_idx.cpu().numpy()
    need = sorted(set(int(e) for e in idx[toks].ravel()))
    experts = {e: dl.expert_host(e) for e in need}
    shared = {i: dl.expert_host(i, shared=True) for i in range(wl.n_shared)}
    t0 = time.perf_counter()
    oracle.layer_forward(x, wr, rb, lambda e: experts[e], lambda i: shared[i], top_k=wl.top_k,
                         n_shared=wl.n_shared, capacity_factor=wl.capacity_factor, tokens=toks)
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = 1
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of {wl.T} tokens of {wl.name} (routing over all {wl.T}; "
                      f"float64 expert FFNs), {dt:.2f} s; host has "
                      f"{len(os.sched_getaffinity(0))} usable cores"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return

    import workloads as W
    from sparse_mixture_experts_renormalised_amd import binding as B
    from workloads.device import DeviceLayer

    wl = W.get_workload(args.workload)
    print(f"[bench] workload {wl.name}: T={wl.T} d={wl.d_model} N={wl.n_routed} K={wl.top_k} "
          f"Ks={wl.n_shared} f={wl.d_ff} {wl.dtype}", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    dl = DeviceLayer(wl, "cuda:0")
    stream = torch.cuda.current_stream()
    nst = len(B.STAGES)
    ev_warm = B.HipEvents(nst + 1)
    for _ in range(args.warmup):
        dl.forward(stream)
    dl.forward_events(ev_warm.handles, stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Per-stage breakdown first: K steps with an event recorded between stages
    # (each record adds a few microseconds between kernels).  Then the timed
    # steps: K plain layer calls, as a user makes them.
    evs = [B.HipEvents(nst + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        dl.forward_events(evs[k].handles, stream)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ms_events = (t3 - t2) * 1e3 / args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dl.forward(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    stage_ms = {s: float(np.mean([e.elapsed_ms(i, i + 1) for e in evs]))
                for i, s in enumerate(B.STAGES)}
    for e in evs + [ev_warm]:
        e.close()
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step "
          f"({ms_events:.4f} with stage events); stages "
          + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()), file=sys.stderr, flush=True)

    counts = dl.counts.cpu().numpy()
    kept = int(counts.sum())
    touched = int((counts > 0).sum())
    work = stage_work(wl, kept, touched)
    dom = max(("up", "down"), key=lambda s: stage_ms[s])
    t_dom = stage_ms[dom] * 1e-3
    flops, nbytes = work[dom]["flops"], work[dom]["bytes"]
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes >= ridge:
        roof = {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": flops / t_dom / 1e12,
                "peak": peak_flops, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / t_dom / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name, dom)
    roof["kernel"] = f"grouped_gemm_bf16 ({dom})" if wl.dtype == "bf16" else f"grouped_gemm_valu ({dom})"
    roof["work_per_launch"] = {"flops": flops, "bytes": nbytes}

    out = {
        "metric": METRIC,
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded counter-based generator, discretised normal)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d_model,
                   "n_routed": wl.n_routed, "top_k": wl.top_k, "n_shared": wl.n_shared,
                   "d_ff": wl.d_ff, "capacity_factor": wl.capacity_factor,
                   "kept_rows": kept, "experts_touched": touched},
        "stage_ms": stage_ms,
        "ms_per_step_with_stage_events": ms_events,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(dl, wl, CPU_SAMPLE.get(wl.name, 64))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
