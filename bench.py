"""Benchmark of the MoE FFN layer forward on one MI355X.

One step = one full pass of the layer (router, top-K gates, dispatch, routed
and shared expert FFNs, combine) over one batch of seeded synthetic tokens
already resident in HBM, through the library's C interface.

Prints one JSON line with whole-job tokens/s, the per-stage times (HIP events
recorded by the library on the stream it launches on), the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--only]

The headline value is the Mixtral-shaped layer (the configuration whose
expert GEMMs have the matrix-core target); ``per_config`` carries the same figures
for every other workload of the metric, among them the DeepSeek-V3-shaped
decode layer's HBM rate.
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
    p.add_argument("--dispatch", choices=("bf16", "fp8"), default="bf16",
                   help="precision of the routed experts' token rows (the FP8 dispatch mode)")
    p.add_argument("--only", action="store_true",
                   help="time only --workload (no per-config lines for the other workloads)")
    p.add_argument("--vs-hipblaslt", action="store_true",
                   help="also time torch.matmul (hipBLASLt) on the same expert products: one "
                        "product per touched expert and shared expert, rows and weights of "
                        "this layer, no gather, SiLU or bias (reported as vendor_gemm)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only copy 1 GiB device-to-device three times (counter calibration)")
    p.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                       "COPY_WRITE_CSV"),
                   help="no GPU: turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of a "
                        "run of this command (and of --calibrate-copy) into the workload's "
                        "entry of profiles/traffic.json; --steps gives the timed passes")
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


def _read_counter_csv(path: str):
    """(kernel name, value) per dispatch, in dispatch order, from a rocprofv3
    counter_collection.csv holding one counter."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            did = int(r.get("Dispatch_Id") or r.get("Dispatch_ID"))
            name = r.get("Kernel_Name") or r.get("Kernel-Name")
            rows.setdefault(did, [name, 0.0])[1] += float(r["Counter_Value"])
    return [tuple(rows[k]) for k in sorted(rows)]


def _short(name: str) -> str:
    """Kernel name without namespaces and arguments: 'grouped_gemm_bf16_rs_kernel<1, 4, false, true>'."""
    head = name.replace("(anonymous namespace)", "").replace("void ", "")
    head = head.split("(")[0]
    return head.split("::")[-1].strip()


def _epi_of(short: str):
    """The epilogue template argument of an expert-GEMM kernel (1: bias + SiLU,
    the first Linear; 0: bias), or None for other kernels."""
    base, _, args = short.partition("<")
    args = [a.strip() for a in args.rstrip(">").split(",")] if args else []
    pos = {"grouped_gemm_bf16_rs_kernel": 0, "rs_fixup_kernel": 0,
           "grouped_gemm_bf16_stream_kernel": 4, "stream_finish_kernel": 3,
           "grouped_gemm_valu_kernel": 1}.get(base)
    if pos is None or pos >= len(args):
        return None
    return 1 if args[pos] in ("1", "kEpiBiasSilu") else 0


def stage_traffic(fetch_csv: str, write_csv: str, passes: int, fetch_scale: float,
                  write_scale: float):
    """HBM bytes of the two expert-GEMM stages per layer pass, averaged over the
    last `passes` passes.  A pass starts at its router kernel; the first
    Linear's stage runs from the kernel after the dispatch through the last
    kernel with the SiLU epilogue (the FP8 quantisation pass included), the
    second Linear's stage from there up to the combine."""
    out = {}
    for which, path, scale in (("fetch", fetch_csv, fetch_scale), ("write", write_csv, write_scale)):
        disp = [(_short(n), v) for n, v in _read_counter_csv(path)]
        starts = [i for i, (n, _) in enumerate(disp) if n.startswith("router_logits")]
        if len(starts) < passes:
            raise ValueError(f"{path}: {len(starts)} layer passes, {passes} asked for")
        bounds = starts + [len(disp)]
        acc = {"up": 0.0, "down": 0.0}
        kern = {"up": [], "down": []}
        for p in range(len(starts) - passes, len(starts)):
            seq = disp[bounds[p]:bounds[p + 1]]
            names = [n for n, _ in seq]
            first = next(i for i, n in enumerate(names) if n.startswith("dispatch")) + 1
            while first < len(names) and names[first].startswith("dispatch"):
                first += 1
            end = next(i for i, n in enumerate(names) if n.startswith("combine"))
            last_up = max(i for i in range(first, end)
                          if _epi_of(names[i]) == 1 or names[i].startswith("quantize"))
            for i in range(first, end):
                st = "up" if i <= last_up else "down"
                acc[st] += seq[i][1] * 1024.0 * scale     # KiB per dispatch
                if names[i] not in kern[st]:
                    kern[st].append(names[i])
        for st in acc:
            out.setdefault(st, {"kernels": kern[st]})[f"{which}_bytes"] = acc[st] / passes
    return out


def copy_scales(fetch_csv: str, write_csv: str, copy_bytes: int = 1 << 30):
    """Bytes per counter unit of FETCH_SIZE and WRITE_SIZE, from the device
    copies of --calibrate-copy (the largest dispatches of those runs)."""
    f = max(v for _, v in _read_counter_csv(fetch_csv)) * 1024.0
    w = max(v for _, v in _read_counter_csv(write_csv)) * 1024.0
    return copy_bytes / f, copy_bytes / w


def stage_work(wl, kept_rows: int, touched: int):
    """Algorithmic flops and HBM bytes of each stage of one forward.

    Bytes count what the method must move once: activations in and out,
    the weights of experts that receive at least one token (untouched experts
    cost nothing), index arrays; not cache re-reads or padding rows.
    """
    T, d, f, N, K, Ks = wl.T, wl.d_model, wl.d_ff, wl.n_routed, wl.top_k, wl.n_shared
    a = wl.act_bytes
    R = kept_rows
    fp8 = getattr(wl, "dispatch_fp8", False)
    w1_bytes = (touched + Ks) * f * d * a + ((touched + Ks) * f * a if wl.expert_bias else 0)
    w2_bytes = (touched + Ks) * d * f * a + ((touched + Ks) * d * a if wl.expert_bias else 0)
    return {
        "router": {"flops": 2 * T * d * N, "bytes": T * d * a + N * d * 4 + T * N * 4},
        "topk": {"flops": 0, "bytes": T * N * 4 + T * K * 8},
        "dispatch": {"flops": 0, "bytes": T * K * 4 * 3 + R * 4},
        # with FP8 dispatch one pass reads x and writes the codes (one byte per
        # element), the per-row exponents and the rows widened back to bf16,
        # which the first Linear then reads like x
        "up": {"flops": 2 * (R + Ks * T) * d * f,
               "bytes": w1_bytes + (R + Ks * T) * (d + f) * a + R * 4
                        + ((T * d * a + T * d + T * 4 + T * d * a) if fp8 else 0)},
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


def roofline(wl, work, stage_ms):
    """Roofline of the dominant stage (the slower expert GEMM)."""
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
    roof["traffic"] = measured_traffic(wl.name + ("+fp8" if wl.dispatch_fp8 else ""), dom)
    roof["kernel"] = f"grouped_gemm_bf16 ({dom})" if wl.dtype == "bf16" else f"grouped_gemm_valu ({dom})"
    roof["work_per_launch"] = {"flops": flops, "bytes": nbytes}
    # the other expert GEMM, in the same units, for reference
    other = "down" if dom == "up" else "up"
    t_o = stage_ms[other] * 1e-3
    roof["other_stage"] = {"stage": other,
                           "achieved": (work[other]["flops"] / t_o / 1e12 if roof["unit"] == "TFLOP/s"
                                        else work[other]["bytes"] / t_o / 1e9)}
    roof["other_stage"]["frac"] = roof["other_stage"]["achieved"] / roof["peak"]
    # the same stage against the other roof (an HBM-bound stage's share of the
    # matrix-core peak, an MFMA-bound stage's share of HBM bandwidth)
    if roof["unit"] == "GB/s":
        a = flops / t_dom / 1e12
        roof["other_roof"] = {"unit": "TFLOP/s", "achieved": a, "peak": peak_flops,
                              "frac": a / peak_flops}
    else:
        a = nbytes / t_dom / 1e9
        roof["other_roof"] = {"unit": "GB/s", "achieved": a, "peak": PEAK_HBM_GBS,
                              "frac": a / PEAK_HBM_GBS}
    return roof


def vendor_gemms(dl, wl, steps: int, warmup: int):
    """torch.matmul (hipBLASLt for bf16) on this layer's expert products: for
    each expert with rows, its gathered token rows times W1_e^T, then the
    hidden rows times W2_e^T; the shared experts on all T tokens.  Operands
    are laid out contiguously beforehand (weights pre-transposed), so only the
    products are timed; no gather, SiLU, bias or combine.  Stage times from
    events over `steps` repetitions."""
    import torch
    r = dl.routing_from_workspace()
    offs, row_token = r["offsets"], r["row_token"]
    x = dl.x
    ups, downs = [], []
    for e in range(wl.n_routed):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi <= lo:
            continue
        a = x[torch.from_numpy(row_token[lo:hi]).long().cuda()].contiguous()
        w1t = dl.w1[e].t().contiguous()
        w2t = dl.w2[e].t().contiguous()
        h = torch.empty((hi - lo, wl.d_ff), dtype=x.dtype, device=x.device)
        y = torch.empty((hi - lo, wl.d_model), dtype=x.dtype, device=x.device)
        ups.append((a, w1t, h))
        downs.append((h, w2t, y))
    for i in range(wl.n_shared):
        w1t = dl.ws1[i].t().contiguous()
        w2t = dl.ws2[i].t().contiguous()
        h = torch.empty((wl.T, wl.d_ff), dtype=x.dtype, device=x.device)
        y = torch.empty((wl.T, wl.d_model), dtype=x.dtype, device=x.device)
        ups.append((x, w1t, h))
        downs.append((h, w2t, y))

    def stage(prods):
        for a, w, o in prods:
            torch.matmul(a, w, out=o)

    out = {"library": "torch.matmul (hipBLASLt), one product per expert with rows and per "
                      "shared expert; no gather, SiLU, bias or combine"}
    for name, prods in (("up", ups), ("down", downs)):
        for _ in range(warmup):
            stage(prods)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            stage(prods)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flops = sum(2.0 * a.shape[0] * a.shape[1] * w.shape[1] for a, w, _ in prods)
        out[f"{name}_ms"] = ms
        out[f"{name}_tflops"] = flops / (ms * 1e-3) / 1e12
        out[f"{name}_frac"] = out[f"{name}_tflops"] / PEAK_BF16_TFLOPS
    del ups, downs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure(wl, steps: int, warmup: int, keep_layer: bool = False, vendor: bool = False):
    """Times one workload: warmup passes, a pass set with stage events, then
    the timed plain layer calls.  Returns the figures and (optionally) the
    device layer."""
    import numpy as np
    import torch
    from sparse_mixture_experts_renormalised_amd import binding as B
    from workloads.device import DeviceLayer

    print(f"[bench] workload {wl.name}: T={wl.T} d={wl.d_model} N={wl.n_routed} K={wl.top_k} "
          f"Ks={wl.n_shared} f={wl.d_ff} {wl.dtype}", file=sys.stderr, flush=True)
    dl = DeviceLayer(wl, "cuda:0")
    stream = torch.cuda.current_stream()
    nst = len(B.STAGES)
    ev_warm = B.HipEvents(nst + 1)
    for _ in range(warmup):
        dl.forward(stream)
    dl.forward_events(ev_warm.handles, stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({warmup} steps)", file=sys.stderr, flush=True)

    # Per-stage breakdown first: K steps with an event recorded between stages
    # (each record adds a few microseconds between kernels).  Then the timed
    # steps: K plain layer calls, as a user makes them.
    evs = [B.HipEvents(nst + 1) for _ in range(steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(steps):
        dl.forward_events(evs[k].handles, stream)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ms_events = (t3 - t2) * 1e3 / steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dl.forward(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    stage_ms = {s: float(np.mean([e.elapsed_ms(i, i + 1) for e in evs]))
                for i, s in enumerate(B.STAGES)}
    for e in evs + [ev_warm]:
        e.close()
    print(f"[bench] {wl.name}: timed {steps} steps: {ms_per_step:.4f} ms/step "
          f"({ms_events:.4f} with stage events); stages "
          + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()), file=sys.stderr, flush=True)

    counts = dl.counts.cpu().numpy()
    kept = int(counts.sum())
    touched = int((counts > 0).sum())
    work = stage_work(wl, kept, touched)
    res = {
        "ms_per_step": ms_per_step,
        "tokens_per_s": wl.T / (ms_per_step * 1e-3),
        "ms_per_step_with_stage_events": ms_events,
        "stage_ms": stage_ms,
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d_model,
                   "n_routed": wl.n_routed, "top_k": wl.top_k, "n_shared": wl.n_shared,
                   "d_ff": wl.d_ff, "capacity_factor": wl.capacity_factor,
                   "dispatch": "fp8" if wl.dispatch_fp8 else "bf16",
                   "kept_rows": kept, "experts_touched": touched},
        "roofline": roofline(wl, work, stage_ms),
        # algorithmic bytes of the whole layer over its wall time per step
        "layer_hbm_gbs": sum(w["bytes"] for w in work.values()) / (ms_per_step * 1e-3) / 1e9,
    }
    if vendor and wl.dtype == "bf16":
        print(f"[bench] {wl.name}: torch.matmul on the same expert products ...",
              file=sys.stderr, flush=True)
        res["vendor_gemm"] = vendor_gemms(dl, wl, steps, warmup)
    if keep_layer:
        return res, dl
    del dl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, None


def record_traffic(args):
    fetch_csv, write_csv, cf, cw = args.traffic_from
    fs, ws = copy_scales(cf, cw)
    st = stage_traffic(fetch_csv, write_csv, args.steps, fs, ws)
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t["_copy_calibration"] = {"fetch_scale": fs, "write_scale": ws,
                              "note": "1 GiB device copy; counters in KiB per dispatch"}
    key = args.workload + ("" if args.dispatch == "bf16" else "+fp8")
    t[key] = {k: dict(v, source_sha=source_sha()) for k, v in st.items()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps({key: t[key]}, indent=1))


def main():
    args = parse()
    if args.traffic_from:
        record_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
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

    torch.cuda.set_device(0)
    wl = W.get_workload(args.workload)
    if args.dispatch == "fp8":
        wl = wl.with_(dispatch_fp8=True)
    head, dl = measure(wl, args.steps, args.warmup, keep_layer=not args.no_cpu_baseline,
                       vendor=args.vs_hipblaslt)
    cpu = None
    if dl is not None:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(dl, wl, CPU_SAMPLE.get(wl.name, 64))
        del dl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    # the other workloads of the metric, each timed the same way (not the
    # headline value): their own expert-GEMM rooflines, and decode's HBM rate
    per_config = {}
    if not args.only:
        for name in W.WORKLOADS:
            # the tiny float32 layer is a parity case (launch-bound), not a bench line
            if name == wl.name or name == "tiny_fp32":
                continue
            w = W.get_workload(name)
            r, _ = measure(w.with_(dispatch_fp8=True) if args.dispatch == "fp8" else w,
                           args.steps, args.warmup, vendor=args.vs_hipblaslt)
            per_config[name] = r

    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded counter-based generator, discretised normal)",
        "config": head["config"],
        "stage_ms": head["stage_ms"],
        "ms_per_step_with_stage_events": head["ms_per_step_with_stage_events"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "per_config": per_config,
    }
    if "vendor_gemm" in head:
        out["vendor_gemm"] = head["vendor_gemm"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
