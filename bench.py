#!/usr/bin/env python3
"""Benchmark of the pre-gated fused multi-adapter projection step on one MI355X.

A step is the whole hot path once over one batch (AdaFuse technical summary
§2.A-§2.B): router pre-gating, segmentation and every projection group in
dependency order (q|k|v, then o, and for the MLP workloads gate|up, then down)
through rp_sgmm_step, which computes the routing inside its first launch.  Weights and inputs are seeded
synthetic data already resident in HBM; weight copies are rotated so repeated
steps stream from HBM rather than the on-chip caches.  A round of steps, one
on each weight copy in turn, is captured in one HIP graph and replayed (as a
decode loop captures its steps); single-step graphs make up the rest of K.

Prints one JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "fused adapter-projection tokens/s + achieved HBM GB/s (% peak), 4096-d decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "rank_pregate_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the current kernels.

    The summary is a text file of `key: value` lines; it names the kernel sources it was measured on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    d = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                d[key.strip()] = val.strip()
    if d.get("kernel_src_sha") != kernel_source_hash():
        log(f"traffic counters in {path} predate the current kernels; reporting null")
        return None
    return int(d["bytes_per_launch"]) if "bytes_per_launch" in d else None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def graph_kernel_nodes(graph) -> int:
    """Kernel nodes of a captured torch CUDAGraph (hipGraphGetNodes / hipGraphNodeGetType), or -1."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        g = ctypes.c_void_p(graph.raw_cuda_graph())
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(g, None, ctypes.byref(n)) != 0:
            return -1
        nodes = (ctypes.c_void_p * n.value)()
        if hip.hipGraphGetNodes(g, nodes, ctypes.byref(n)) != 0:
            return -1
        kernels = 0
        for i in range(n.value):
            t = ctypes.c_int(-1)
            if hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) != 0:
                return -1
            kernels += t.value == 0  # hipGraphNodeTypeKernel
        return kernels
    except (OSError, AttributeError, RuntimeError, TypeError):
        return -1


def percentile(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def cpu_baseline(wl, seconds: float):
    """The CPU oracle on the same workload, timed on this host (a reported baseline only)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from rank_pregate_amd import datagen

    # inputs drawn outside the timed region (bf16 bit patterns, as uploaded)
    xr, Wg = datagen.router_input(wl), datagen.router_weight(wl)
    groups = []
    for g in wl.groups:
        xg = datagen.layer_input(wl, 0, g.x_name)
        groups.append((xg, [datagen.proj_weights(wl, 0, g, p) for p in g.projs]))
    reps = 0
    t0 = time.perf_counter()
    while True:
        idx, gate, _ = oracle.pregate(oracle.widen(xr, wl.dtype), oracle.widen(Wg, wl.dtype), wl.k)
        oracle.segment(idx, wl.E)
        for xg, ws in groups:
            x64 = oracle.widen(xg, wl.dtype)
            for w in ws:
                oracle.sgmm(x64, oracle.widen(w.W0, wl.dtype), oracle.widen(w.A, wl.dtype),
                            oracle.widen(w.B, wl.dtype), idx, gate)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": wl.T * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full {wl.name} step(s) of the fp64 NumPy oracle (T={wl.T}, layer 0, all groups), "
                      f"{el:.1f} s, widening of bf16 inputs included, input generation excluded; "
                      f"host {cpu_model()}, "
                      f"{len(os.sched_getaffinity(0))} cores available"}


def stream_read_ceiling(dev, nbytes: int = 1 << 30) -> float:
    """GB/s of rp_util_stream_read over a fresh `nbytes` buffer (past the Infinity Cache), mean of 5."""
    import torch

    import rank_pregate_amd as rp
    big = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1024, dtype=torch.float32, device=dev)
    for _ in range(2):
        rp.stream_read(big, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        rp.stream_read(big, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 5
    del big
    return nbytes / (us * 1e-6) / 1e9


def calibrate():
    """Known-traffic kernels: a 1 GiB copy (reads 1 GiB, writes 1 GiB) for scaling the
    FETCH_SIZE / WRITE_SIZE counters, and a 4 GiB stream read for the achievable read bandwidth."""
    import torch

    import rank_pregate_amd as rp
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    big = torch.ones(1 << 30, dtype=torch.float32, device=dev)  # 4 GiB
    sink = torch.empty(1024, dtype=torch.float32, device=dev)
    out = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: rp.copy(dst, src), 2 << 30),
                             ("stream_read_4GiB", lambda: rp.stream_read(big, sink), 4 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        n = 10
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        out[name] = {"avg_us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log(f"[calibrate] {name}: {us:.1f} us, {nbytes / (us * 1e-6) / 1e9:,.0f} GB/s")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_qkvo")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated per step (0: auto)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--separate-route", action="store_true",
                    help="run rp_pregate and rp_segment as launches of their own instead of inside the first group")
    ap.add_argument("--ablation", default="auto",
                    help="comma list of baselines timed next to the fused step on the same kernels: unfused "
                         "(a base launch and one launch per adapter), per_layer_routing (the router re-run at "
                         "every layer); 'auto': unfused, plus per_layer_routing for multi-layer workloads; "
                         "'none' to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate", action="store_true",
                    help="instead of the step: time the plain copy and stream-read kernels (known traffic) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_pregate_amd as rp
    from rank_pregate_amd import datagen
    from rank_pregate_amd.workload import DeviceWorkload

    rp.lib()  # fail loudly if the HIP library is missing
    if args.calibrate:
        calibrate()
        return
    wl = datagen.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    copies = args.copies
    if copies <= 0:
        # keep the rotated weight set well above the 256 MB last-level cache
        per_copy = sum(g.d_in * g.d_out * len(g.projs) for g in wl.groups) * wl.layers * (2 if wl.dtype == "bf16" else 4)
        copies = max(1, min(16, -(-1_200_000_000 // per_copy)))
    log(f"[bench] workload {wl.name}: {wl.description}; weight copies {copies}")
    t_gen = time.perf_counter()
    if args.ablation == "auto":
        variants = [] if wl.assignment != "router" else (
            ["unfused"] + (["per_layer_routing"] if wl.layers > 1 else []) + ["token_fused", "token_merge_unmerge"]
            + (["chained_layers", "chained_layers_dependent"]
               if [g.name for g in wl.groups] == ["qkv", "o", "gate_up", "down"] else []))
    elif args.ablation == "none":
        variants = []
    else:
        variants = [v for v in args.ablation.split(",") if v]
    dw = DeviceWorkload(wl, dev, copies=copies, per_layer_router="per_layer_routing" in variants)
    log(f"[bench] data generated and uploaded in {time.perf_counter() - t_gen:.1f} s")

    stream = torch.cuda.Stream(device=dev)  # default priority
    with torch.cuda.stream(stream):
        for _ in range(3):
            dw.step()
        stream.synchronize()
        n_touched = int((torch.diff(dw.seg_offsets) > 0).sum().item())

        fused = not args.separate_route and dw.can_fuse_route()
        if args.no_graph:
            def run(i):
                dw.run(i % copies, fused=fused)
        else:
            # one graph per weight copy (single steps) and one graph of a round
            # of steps, one on each copy in turn, as a decode loop captures its
            # steps; K steps = K // copies rounds + K % copies single steps
            graphs = []
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    dw.run(c, fused=fused)
                graphs.append(g)
            round_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(round_graph, stream=stream):
                for c in range(copies):
                    dw.run(c, fused=fused)

            def run(i):
                graphs[i % copies].replay()

        def run_steps(n, marks=None):
            """n steps; with `marks`, an event after every round of `copies` steps (per-step samples)."""
            if args.no_graph:
                for i in range(n):
                    run(i)
                    if marks is not None and (i + 1) % copies == 0:
                        marks.append(torch.cuda.Event(enable_timing=True))
                        marks[-1].record(stream)
                return
            for _ in range(n // copies):
                round_graph.replay()
                if marks is not None:
                    marks.append(torch.cuda.Event(enable_timing=True))
                    marks[-1].record(stream)
            for i in range(n % copies):
                run(i)

        run_steps(args.warmup)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = [ev0]
        ev0.record(stream)
        run_steps(args.steps, marks)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = ev0.elapsed_time(ev1) / args.steps
        step_samples = [marks[i].elapsed_time(marks[i + 1]) / copies for i in range(len(marks) - 1)]
        if not step_samples:
            step_samples = [ms_per_step]

        # kernel launches of one step, counted in a captured graph of it
        cg = torch.cuda.CUDAGraph(keep_graph=True)
        with torch.cuda.graph(cg, stream=stream):
            dw.run(0, fused=fused)
        launches = graph_kernel_nodes(cg)
        del cg

        # the dominant launch: the step's first multi-group launch (routing
        # inside when fused, then up to eight projection groups), alone, one
        # graph of it on each weight copy in turn, replayed; events on the
        # stream it is launched on bracket the replays
        n_dom = min(8, len(dw.step_groups(0)))

        def dominant(c):
            dw.run(c, fused=fused, n_groups=n_dom)

        reps = max(2, args.steps // copies)
        if args.no_graph:
            for c in range(copies):
                dominant(c)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps * copies):
                dominant(i % copies)
            b.record(stream)
        else:
            dg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(dg, stream=stream):
                for c in range(copies):
                    dominant(c)
            dg.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                dg.replay()
            b.record(stream)
        torch.cuda.synchronize()
        dom_ms = a.elapsed_time(b) / (reps * copies)

        # base-only (k = 0) step for the adapter overhead: the same projection
        # groups without routing or adapters, a round of them per graph
        nb = max(2, args.steps // copies)
        if args.no_graph:
            for i in range(copies):
                dw.project(i, k=0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(nb * copies):
                dw.project(i % copies, k=0)
            e1.record(stream)
        else:
            bg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(bg, stream=stream):
                for c in range(copies):
                    dw.project(c, k=0)
            bg.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(nb):
                bg.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        base_ms = e0.elapsed_time(e1) / (nb * copies)

        # baselines on the same kernels: a round of steps per graph, rotating copies
        ablation = {}
        drift_ref = None
        if "token_merge_unmerge" in variants:
            # copy 0's layer-0 backbone weights before any merge, for the unmerge drift
            drift_ref = {key: v.W0.clone() for key, v in dw.weights[0].items() if key[0] == dw.layers[0]}
        for variant in variants:
            if variant.startswith("chained_layers"):
                dw.prepare_chain()  # uploads and allocates: not inside a graph
            if args.no_graph:
                for c in range(copies):
                    dw.run_variant(variant, c)
                torch.cuda.synchronize()
                va, vb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                va.record(stream)
                for i in range(nb * copies):
                    dw.run_variant(variant, i % copies)
                vb.record(stream)
            else:
                vg = torch.cuda.CUDAGraph()
                with torch.cuda.graph(vg, stream=stream):
                    for c in range(copies):
                        dw.run_variant(variant, c)
                vg.replay()
                torch.cuda.synchronize()
                va, vb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                va.record(stream)
                for _ in range(nb):
                    vg.replay()
                vb.record(stream)
            torch.cuda.synchronize()
            v_ms = va.elapsed_time(vb) / (nb * copies)
            lg = torch.cuda.CUDAGraph(keep_graph=True)
            with torch.cuda.graph(lg, stream=stream):
                dw.run_variant(variant, 0)
            v_launches = graph_kernel_nodes(lg)
            del lg
            if not args.no_graph:
                del vg
            if variant.startswith("token_"):
                ablation[variant] = {"ms_per_token": round(v_ms, 5), "launches_per_token": v_launches}
                log(f"[bench] one token, {variant}: {v_ms * 1e3:.1f} us, {v_launches} launches")
                continue
            ablation[variant] = {"ms_per_step": round(v_ms, 5), "vs_fused": round(v_ms / ms_per_step, 3),
                                 "vs_base_only": round(v_ms / base_ms, 3), "launches_per_step": v_launches}
            log(f"[bench] baseline {variant}: {v_ms * 1e3:.1f} us per step ({v_ms / ms_per_step:.2f}x the fused step, "
                f"{v_ms / base_ms:.2f}x base-only), {v_launches} launches")
        if "token_fused" in ablation and "token_merge_unmerge" in ablation:
            tf, tm = ablation["token_fused"]["ms_per_token"], ablation["token_merge_unmerge"]["ms_per_token"]
            w0_bytes = sum(v.W0.numel() * v.W0.element_size() for v in dw.weights[0].values())
            ablation["token_merge_unmerge"]["vs_token_fused"] = round(tm / tf, 3)
            # merge and unmerge each read and write every W0, the backbone reads it once more
            ablation["token_merge_unmerge"]["w0_bytes_moved"] = 5 * w0_bytes
            ablation["token_fused"]["w0_bytes_moved"] = w0_bytes
        if drift_ref is not None:
            torch.cuda.synchronize()
            changed = total = 0
            max_abs = max_w = 0.0
            for key, ref in drift_ref.items():
                now = dw.weights[0][key].W0
                diff = (now.float() - ref.float()).abs()
                changed += int((diff > 0).sum().item())
                total += now.numel()
                max_abs = max(max_abs, float(diff.max().item()))
                max_w = max(max_w, float(ref.float().abs().max().item()))
            cycles = nb + 1
            ablation["token_merge_unmerge"]["unmerge_drift"] = {
                "merge_unmerge_cycles": cycles, "elements_changed_frac": round(changed / total, 6),
                "max_abs_change": max_abs, "max_abs_change_over_max_w0": max_abs / max_w,
                "scope": f"layer {dw.layers[0]} backbone weights of weight copy 0"}
            log(f"[bench] unmerge drift after {cycles} merge/unmerge cycles: {100 * changed / total:.3f}% of "
                f"layer-{dw.layers[0]} W0 elements changed, max |change| {max_abs:.2e} ({max_abs / max_w:.2e} of max|W0|)")

        # every wait inside the launches ended and no index was out of range
        wait_overflow, bad_idx = rp.workspace_status(dw.ws, stream=stream)

    step_bytes = dw.algorithmic_bytes(n_touched)
    step_flops = dw.algorithmic_flops()
    base_bytes = dw.algorithmic_bytes(n_touched, k=0) - dw.routing_bytes()
    base_flops = dw.algorithmic_flops(k=0) - 2 * wl.T * wl.d * wl.E
    med, p10, p90 = (percentile(step_samples, q) for q in (50, 10, 90))
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = wl.T / (ms_per_step * 1e-3)
    dom_bytes = sum(dw.group_bytes(i, n_touched) for i in range(n_dom))
    if fused:  # the launch also reads the router weight and writes the routing arrays
        dom_bytes += dw.routing_bytes() - wl.T * wl.d * (2 if wl.dtype == "bf16" else 4)
    names = [f"{g.name}" for g in wl.groups]
    dom_groups = [names[i % len(names)] for i in range(n_dom)]
    dom_name = f"rp_sgmm_step({'route, ' if fused else ''}{', '.join(dom_groups)})"
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    dom_flops = sum(dw.group_flops(i) for i in range(n_dom)) + (2 * wl.T * wl.d * wl.E if fused else 0)
    dom_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    mfma_bound = wl.name == "prefill_mlp"  # ~1425 FLOP per byte: past the bf16 MFMA ridge (~312)
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, {tokens_per_s:,.0f} tokens/s, algorithmic {step_bytes / 1e6:.1f} MB "
        f"-> {gbs:,.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s); {step_flops / (ms_per_step * 1e-3) / 1e12:.1f} "
        f"TFLOP/s; touched adapters {n_touched}/{wl.E}")
    log(f"[bench] dominant call {dom_name}: {dom_ms * 1e3:.1f} us for {dom_bytes / 1e6:.1f} MB "
        f"-> {dom_gbs:,.0f} GB/s")
    log(f"[bench] base-only (k=0) projections {base_ms * 1e3:.1f} us per step; adapter overhead "
        f"{100 * (ms_per_step / base_ms - 1):.1f}%; {launches} kernel launches per step; "
        f"median {med * 1e3:.1f} us (p10 {p10 * 1e3:.1f}, p90 {p90 * 1e3:.1f})")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "r": wl.r, "k": wl.k,
                   "layers": wl.layers, "groups": [g.name for g in wl.groups], "weight_copies": copies,
                   "graph": not args.no_graph, "route_fused": fused, "achieved_GBps": round(gbs, 1),
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "algorithmic_bytes_per_step": step_bytes, "touched_adapters": n_touched},
        "roofline": ({"bound": "mfma", "achieved": round(dom_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(dom_tflops / BF16_PEAK_TFLOPS, 4)}
                     if mfma_bound else
                     {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(dom_gbs / HBM_PEAK_GBS, 4)}),
    }
    line["roofline"].update({"traffic": measured_traffic("step", wl.name), "kernel": dom_name,
                             "avg_launch_us": round(dom_ms * 1e3, 2), "bytes_per_launch": dom_bytes,
                             "flops_per_launch": dom_flops, "achieved_GBps": round(dom_gbs, 1),
                             "achieved_TFLOPs": round(dom_tflops, 1)})
    if not mfma_bound:
        # the achievable read rate on this GPU, measured after the timed work: the
        # dominant call's algorithmic GB/s against it as well as against the peak
        sr = stream_read_ceiling(dev)
        line["roofline"].update({"stream_read_GBps": round(sr, 1), "frac_of_stream_read": round(dom_gbs / sr, 4)})
        log(f"[bench] stream-read ceiling {sr:,.0f} GB/s; dominant call at {100 * dom_gbs / sr:.1f}% of it")
    line["timing"] = {"median_ms": round(med, 5), "p10_ms": round(p10, 5), "p90_ms": round(p90, 5),
                      "samples": len(step_samples), "sample": f"mean step time of each round of {copies} steps",
                      "launches_per_step": launches, "base_only_ms": round(base_ms, 5),
                      "adapter_overhead_pct": round(100 * (ms_per_step / base_ms - 1), 2),
                      "adapter_byte_frac": round(1 - base_bytes / step_bytes, 4),
                      "adapter_flop_frac": round(1 - base_flops / step_flops, 4),
                      "device_status": {"wait_overflow": wait_overflow, "bad_indices": bad_idx}}
    if ablation:
        line["ablation"] = ablation
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
