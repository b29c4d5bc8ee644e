#!/usr/bin/env python3
"""Throughput of one compressed-expert MoE FFN layer forward on one MI355X.

A step is one moe_forward over one batch of T synthetic tokens already
resident in HBM (router, token lists, the grouped GEMMs, combine).  The
default workload is the largest layer that fits one GPU: the flat top-2 of
8 bf16 SwiGLU layer (T = 4096, d = 4096, f = 14336, 8 experts);
``--workload N`` selects another of the five shapes.  The decode-shaped
layer is timed cold: steps alternate between two copies of its weights
whose total exceeds the 256 MB last-level cache, so every step streams
its weights from HBM.

Prints one JSON line: routed tokens/s (T per forward), the roofline of the
dominant kernel (algorithmic work per launch over its average duration,
timed with HIP events on the launch stream inside the timed region), and
the CPU oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer fwd on 1 MI355X; % MFMA peak or % HBM BW"
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
STAGES = ("router", "scatter", "ugemm", "gemm1", "vreduce", "gemm2", "combine")


def resid_bytes_per_entry(w) -> float:
    return {"int4_g32": 0.5 + 2.0 / 32, "f16": 2.0, "f32": 4.0, "none": 0.0}[w.resid]


def kernel_work(w, T, touched_groups, touched_experts) -> dict:
    """Algorithmic FLOPs and bytes per launch of each kernel (the method's
    own work: base projections once per (token, chosen group), residual
    only for selected experts; bytes = weights of touched groups and
    experts plus the layer's input and output, workspace excluded)."""
    d, f, r, k, kg, K, G, Pin = w.d, w.f, w.r, w.k, w.top_groups, w.K, w.G, w.P_in
    xb = 4 if w.x_dtype == "f32" else 2
    bb = 4 if w.base_dtype == "f32" else 2
    rb = resid_bytes_per_entry(w)
    tg, te = touched_groups, touched_experts
    flops = dict(
        router=2 * T * d * (G + (kg * K if K > 1 else 0)),
        scatter=0,
        ugemm=2 * T * k * r * Pin * d,
        gemm1=2 * T * kg * Pin * d * f + 2 * T * k * r * Pin * f + 2 * T * k * r * f + 2 * T * k * f,
        vreduce=0,
        gemm2=2 * T * kg * f * d + 2 * T * k * r * d,
        combine=T * (kg - 1) * d,
    )
    nbytes = dict(
        router=T * d * xb + d * G * 4 + (tg * d * K * 4 if K > 1 else 0),
        scatter=T * k * 4 * 3,
        ugemm=T * d * xb + te * Pin * d * r * rb,
        gemm1=T * d * xb + tg * Pin * d * f * bb + te * (Pin * f * r + f * r) * rb,
        vreduce=T * k * 16 * 4 * 2,
        gemm2=tg * f * d * bb + te * d * r * rb + T * d * xb,
        combine=T * kg * d * 4 + T * d * xb,
    )
    return dict(flops=flops, bytes=nbytes)


def traffic_for(workload_name: str, kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the record
    under profiles/ was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[workload_name][kernel]
    except (KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "compressed_expert_ffn_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    return rec.get("bytes_per_launch") if rec.get("src_sha") == sha else None


KERNEL_STAGE = (("route_fused", "router"), ("logits_kernel", "router"), ("select_kernel", "router"),
                ("scatter", "scatter"), ("group_sort", "scatter"), ("cvt_bf16", "ugemm"), ("ugemm", "ugemm"), ("gemm1", "gemm1"),
                ("vreduce", "vreduce"), ("gemm2", "gemm2"), ("tailfix", "tailfix"), ("combine", "combine"),
                ("zero_kernel", "zero"))


def stage_of(kernel_name: str):
    for key, stage in KERNEL_STAGE:
        if key in kernel_name:
            return stage
    return None


def pmc_means(csv_path: str, counter: str) -> dict:
    """Mean value of one counter per dispatch, by stage and for the copy."""
    import csv
    acc = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            name = row["Kernel_Name"]
            key = stage_of(name) or ("copy" if "copy" in name.lower() else None)
            if key is None:
                continue
            acc.setdefault(key, []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_pmc(args) -> None:
    """Turn two rocprofv3 counter runs of the benchmark (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) and the same two counters on a plain device
    copy of --copy-mib MiB into HBM bytes per launch per kernel, scaled so the
    copy reads and writes exactly its size; written to profiles/pmc_traffic.json
    keyed by workload and stamped with the kernel source it was taken on."""
    fetch = pmc_means(args.fetch_csv, "FETCH_SIZE")
    write = pmc_means(args.write_csv, "WRITE_SIZE")
    cf = pmc_means(args.copy_fetch_csv, "FETCH_SIZE")["copy"]
    cw = pmc_means(args.copy_write_csv, "WRITE_SIZE")["copy"]
    kib = args.copy_mib * 1024.0
    f_scale, w_scale = kib / cf, kib / cw
    src = os.path.join(ROOT, "compressed_expert_ffn_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    from compressed_expert_ffn_amd.workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    rec = {}
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        rec[k] = dict(fetch_kib=round(fetch[k], 1), write_kib=round(write[k], 1),
                      bytes_per_launch=int((fetch[k] * f_scale + write[k] * w_scale) * 1024),
                      src_sha=sha)
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    allrec = json.load(open(path)) if os.path.exists(path) else {}
    allrec[w.name] = dict(rec, _calibration=dict(copy_mib=args.copy_mib, copy_fetch_kib=round(cf, 1),
                                                 copy_write_kib=round(cw, 1), fetch_scale=round(f_scale, 4),
                                                 write_scale=round(w_scale, 4)))
    json.dump(allrec, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps(allrec[w.name], indent=1))


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of a known size, for counter scaling."""
    import torch
    a = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x5", flush=True)


def blas_reference(w) -> None:
    """The layer's two base GEMMs as plain batched library GEMMs (torch.matmul,
    hipBLASLt on ROCm), rows split evenly over the groups: a reference point
    for the main loop, not part of the layer."""
    import torch
    torch.manual_seed(0)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.base_dtype]
    G, rows = w.G, w.T * w.top_groups
    m = rows // G
    x = torch.randn(G, m, w.d, device="cuda", dtype=dt)
    w1 = torch.randn(G, w.d, w.P_in * w.f, device="cuda", dtype=dt) / w.d ** 0.5
    hh = torch.randn(G, m, w.f, device="cuda", dtype=dt)
    w2 = torch.randn(G, w.f, w.d, device="cuda", dtype=dt) / w.f ** 0.5
    out = {}
    for name, a, b in (("gemm1", x, w1), ("gemm2", hh, w2)):
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            torch.matmul(a, b)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 10
        fl = 2.0 * G * m * a.shape[2] * b.shape[2]
        out[name] = {"shape": [G, m, a.shape[2], b.shape[2]], "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}
    print(json.dumps({"blas_reference": w.name, **out}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, inputs, budget_s: float) -> dict:
    """The CPU oracle as it stands, on the same workload (the sample is the
    whole batch, repeated while the time budget lasts)."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    fields = dict(G=w.G, K=w.K, top_groups=w.top_groups, top_experts=w.top_experts, r=w.r,
                  d=w.d, f=w.f, act=w.act, x_dtype=w.x_dtype, base_dtype=w.base_dtype,
                  resid=w.resid)
    layer = O.layer_from(fields, inputs)
    T = inputs["X"].shape[0]
    # bound the sample for the large layers: route everything, FFN on a prefix
    n_tok = T if w.index in (0, 1, 4) else min(T, 256)
    toks = list(range(n_tok))
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.forward(layer, tokens=toks)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 3:
            break
    times.sort()
    med = times[len(times) // 2]
    return dict(value=n_tok / med, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{n_tok} of {T} tokens of the {w.name} layer, float64 NumPy oracle, "
                       f"median of {len(times)} run(s) of {med:.2f} s",
                cpu_model=cpu_model(), nproc=os.cpu_count())


def side_modes(args, w, inputs) -> None:
    """The backward pass, or the forward pass with offloaded groups: one
    JSON line with the time per call (HIP events around the timed calls on
    the launch stream) and the work rate."""
    import numpy as np
    import torch
    from compressed_expert_ffn_amd import _lib as L
    from compressed_expert_ffn_amd import synth
    lay = L.Layer(L.config_from_workload(w), inputs)
    Xh = inputs["X"]
    if w.x_dtype == "bf16":
        X = torch.from_numpy(Xh.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        X = torch.from_numpy(Xh).cuda()
    out = dict(metric=args.mode, workload=w.name, T=w.T, steps=args.steps, warmup=args.warmup)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.mode == "backward":
        dY32 = np.random.default_rng(17).standard_normal((w.T, w.d)).astype(np.float32)
        dYs = synth.to_storage(dY32, w.x_dtype)
        dY = (torch.from_numpy(dYs.view(np.int16)).cuda().view(torch.bfloat16) if w.x_dtype == "bf16"
              else torch.from_numpy(dYs).cuda())
        for _ in range(max(1, args.warmup)):
            lay.backward(X, dY)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(args.steps):
            lay.backward(X, dY)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        flops = 2 * w.algorithmic_flops()["total"]
        out.update(ms_per_call=round(ms, 4), tokens_per_s=round(w.T / (ms * 1e-3), 1),
                   algorithmic_tflops=round(flops / (ms * 1e-3) / 1e12, 2),
                   note="algorithmic work counted as twice the forward pass's; the recomputed forward "
                        "intermediates are overhead")
    else:
        slots = args.slots or max(1, w.G // 2)
        lay.offload_enable(slots)
        Y = torch.empty_like(X)
        rng_batches = [X] + [(torch.from_numpy(synth.draw_x(w, seed=500 + i).view(np.int16)).cuda()
                              .view(torch.bfloat16) if w.x_dtype == "bf16"
                              else torch.from_numpy(synth.draw_x(w, seed=500 + i)).cuda()) for i in range(3)]
        for i in range(max(1, args.warmup)):
            lay.forward_offload(rng_batches[i % 4], Y)
        torch.cuda.synchronize()
        s0 = lay.offload_stats()
        t0 = time.perf_counter()
        for i in range(args.steps):
            lay.forward_offload(rng_batches[i % 4], Y)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        s1 = lay.offload_stats()
        d = {k: s1[k] - s0[k] for k in s1}
        out.update(slots=slots, groups=w.G, ms_per_call=round(ms, 4), tokens_per_s=round(w.T / (ms * 1e-3), 1),
                   h2d_gb_per_s=round(d["bytes_h2d"] / (ms * 1e-3 * args.steps) / 1e9, 2),
                   loads_per_call=round(d["group_loads"] / args.steps, 2),
                   hits_per_call=round(d["group_hits"] / args.steps, 2),
                   prefetched_per_call=round(d["prefetched"] / args.steps, 2),
                   passes_per_call=round(d["passes"] / args.steps, 2),
                   note="batches rotate over 4 seeded token sets; host wall clock per call (the call "
                        "synchronises once to read the touched groups)")
    lay.close()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--copies", type=int, default=0,
                    help="weight copies rotated between steps (0: 2 for the decode layer, else 1)")
    ap.add_argument("--no-graph", action="store_true", help="plain stream launches only")
    ap.add_argument("--mode", choices=("forward", "backward", "offload"), default="forward",
                    help="backward: time moe_backward; offload: moe_forward_offload with --slots device slots")
    ap.add_argument("--slots", type=int, default=0, help="offload mode: device group slots (0: G/2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of --copy-mib MiB (counter scaling)")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--blas-reference", action="store_true",
                    help="only time the workload's base GEMM shapes as plain library GEMMs")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/pmc_traffic.json from rocprofv3 counter CSVs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        args.fetch_csv, args.write_csv, args.copy_fetch_csv, args.copy_write_csv = args.summarize_pmc
        summarize_pmc(args)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_mib)
        return
    if args.blas_reference:
        from compressed_expert_ffn_amd.workloads import WORKLOADS
        blas_reference(WORKLOADS[args.workload])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this layer is built and measured on one GPU only; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from compressed_expert_ffn_amd import _lib as L
    from compressed_expert_ffn_amd import synth
    from compressed_expert_ffn_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    inputs = synth.make_layer(w)
    if args.mode != "forward":
        side_modes(args, w, inputs)
        return
    copies = args.copies or (2 if w.index == 4 else 1)
    lays = [L.Layer(L.config_from_workload(w), inputs) for _ in range(copies)]
    lay = lays[0]
    weight_mb = lay.stats()["stored_bytes"] / 1e6
    xt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.x_dtype]
    Xh = inputs["X"]
    if w.x_dtype == "bf16":
        X = torch.from_numpy(Xh.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        X = torch.from_numpy(Xh).cuda()
    Y = torch.empty((w.T, w.d), dtype=xt, device="cuda")

    # routing statistics of this batch (untimed)
    rb = lay.route(X)
    counts = rb["counts"].cpu().numpy()
    gcounts = rb["gcounts"].cpu().numpy()
    tg, te = int((gcounts > 0).sum()), int((counts > 0).sum())
    work = kernel_work(w, w.T, tg, te)

    def step(i):
        lays[i % copies].forward(X, Y)

    # warm-up, with every stage timed to find the dominant kernel (the first
    # call of each copy loads code objects and is left out)
    for i in range(copies):
        step(i)
    torch.cuda.synchronize()
    nw = max(copies, args.warmup)
    for lw in lays:
        lw.profile_begin(nw)
    for i in range(nw):
        step(i)
    warm = [lw.profile_end() for lw in lays]
    calls = max(1, sum(x["calls"] for x in warm))
    stage_ms = {s: sum(x["stage_ms"].get(s, 0.0) for x in warm) / calls for s in STAGES}
    dominant = max(STAGES, key=lambda s: stage_ms[s])

    # timed region: plain stream launches, HIP events around the dominant kernel
    torch.cuda.synchronize()
    for lw in lays:
        lw.profile_begin(args.steps, stages=[dominant])
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    profs = [lw.profile_end() for lw in lays]
    ms_stream = (t1 - t0) * 1e3 / args.steps
    dom_ms = sum(p["stage_ms"][dominant] for p in profs) / max(1, sum(p["calls"] for p in profs))

    # the same steps replayed from captured HIP graphs (one per weight copy)
    ms_graph = None
    if not args.no_graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(copies):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        ms_graph = (time.perf_counter() - t0) * 1e3 / args.steps

    ms = ms_stream if ms_graph is None else min(ms_stream, ms_graph)
    launch = "stream" if ms_graph is None or ms_stream <= ms_graph else "hipgraph"

    # per-step latency distribution: the same launch form, each step
    # bracketed by HIP events on the launch stream
    nlat = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nlat)]
    for i in range(nlat):
        evs[i][0].record()
        if launch == "hipgraph":
            graphs[i % copies].replay()
        else:
            step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    lat = np.sort(np.array([a.elapsed_time(b) for a, b in evs]))
    step_lat = dict(n=nlat, p10=round(float(np.percentile(lat, 10)), 5), p50=round(float(np.percentile(lat, 50)), 5),
                    p90=round(float(np.percentile(lat, 90)), 5))
    value = w.T / (ms * 1e-3)

    hbm_bound = w.index == 4
    if hbm_bound:
        achieved = work["bytes"][dominant] / (dom_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_for(w.name, dominant),
                    kernel=dominant, kernel_ms=round(dom_ms, 5),
                    work_per_launch=work["bytes"][dominant])
    else:
        peak = MFMA_PEAK_TFLOPS[w.base_dtype]
        achieved = work["flops"][dominant] / (dom_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=traffic_for(w.name, dominant),
                    kernel=dominant, kernel_ms=round(dom_ms, 5),
                    work_per_launch=work["flops"][dominant])

    total_flops = w.algorithmic_flops()["total"]
    out = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype=w.base_dtype, data="synthetic",
        config=dict(workload=w.name, T=w.T, d=w.d, f=w.f, G=w.G, K=w.K,
                    top_groups=w.top_groups, top_experts=w.top_experts, r=w.r,
                    residual=w.resid, act=w.act, x_dtype=w.x_dtype, launch=launch,
                    weight_copies=copies, weight_mb_per_copy=round(weight_mb, 1),
                    cache="cold" if copies * weight_mb > 256 else "warm"),
        roofline=roof,
        assignments_per_s=round(w.T * w.k / (ms * 1e-3), 1),
        layer_tflops=round(total_flops / (ms * 1e-3) / 1e12, 2),
        ms_stream=round(ms_stream, 5), ms_graph=None if ms_graph is None else round(ms_graph, 5),
        step_ms_events=step_lat,
        stage_ms={k: round(v, 5) for k, v in stage_ms.items() if v > 0},
        touched_groups=tg, touched_experts=te,
        expert_load_max_over_avg=round(float(counts.max() / max(counts.mean(), 1e-9)), 3),
        expert_load_var=round(float(counts.var()), 2),
    )
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    for lw in lays:
        lw.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
