"""Benchmark: Llama-3-8B-shaped W4 decode step on one MI355X.

One step = the 224 decode GEMVs of a 32-layer Llama-3-8B-shaped decoder in
layer order (q, k, v, o, gate, up, down per layer; K x N = 4096x4096,
4096x1024, 4096x1024, 4096x4096, 4096x14336, 4096x14336, 14336x4096), M = 1,
symmetric INT4 with group size 128, fp16 scales U[0.002, 0.01], fp16
activations N(0,1) (one distinct input vector per GEMV), fp16 outputs.  Every
weight is distinct, 3.49 GB of packed codes and 0.11 GB of scales, so the step
streams 3,603,955,712 algorithmic bytes from HBM and no cache can hold it.
The step is captured once as a HIP graph and replayed.

Printed: one JSON line with the effective HBM GB/s of the step (the metric),
tokens/s (= steps/s at M = 1), the dominant kernel's roofline entry and the
CPU oracle's rate on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-layers L]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "W4 decode GEMV effective HBM GB/s (% of peak) and tokens/s at 8B shapes"
HBM_PEAK_GBPS = 8000.0
LAYERS = 32
G = 128
WORKLOAD_ID = 1


def algorithmic_bytes(K, N, M=1, G=128):
    """Bytes a W4 GEMV must move at least once: codes (0.5 B/weight), fp16
    scales (2/G B/weight), the fp16 input and output vectors."""
    return N * K // 2 + N * (K // G) * 2 + M * K * 2 + M * N * 2


def build_step(lb, synth, torch):
    """Pack every weight of the 32-layer step on the GPU; return the launch list."""
    fmt = lb.LOWBIT_W4_SYM
    launches = []
    for layer in range(LAYERS):
        for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS):
            w = synth.w4_weights(N, K, G, scale_range=(0.002, 0.01), workload_id=WORKLOAD_ID, layer=layer, part=pid)
            nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
            packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
            codes = torch.from_numpy(w["qweight"]).cuda()
            scales = torch.from_numpy(w["scales"].view(np.uint16)).cuda()
            lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, codes, scales, None, packed, nb))
            x = torch.from_numpy(synth.activations_f16(1, K, workload_id=WORKLOAD_ID, layer=layer, part=pid)).cuda()
            y = torch.empty((1, N), dtype=torch.float16, device="cuda")
            wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV, fmt, 1, N, K, G)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
            launches.append(dict(name=name, K=K, N=N, packed=packed, x=x, y=y, ws=ws, wsb=wsb,
                                 bytes=algorithmic_bytes(K, N)))
            del codes, scales
    torch.cuda.synchronize()
    return fmt, launches


def run_step(lb, fmt, launches, stream):
    for L in launches:
        st = lb.lowbit_gemv(fmt, 1, L["N"], L["K"], G, L["packed"], L["x"], L["y"], L["ws"], L["wsb"], stream)
        if st != 0:
            raise lb.LowbitError(st)


def cpu_baseline(synth, layers):
    """The CPU oracle on the first `layers` layers of the same step (single thread)."""
    import oracle
    t_total = 0.0
    nbytes = 0
    for layer in range(layers):
        for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS):
            w = synth.w4_weights(N, K, G, scale_range=(0.002, 0.01), workload_id=WORKLOAD_ID, layer=layer, part=pid)
            x = synth.activations_f16(1, K, workload_id=WORKLOAD_ID, layer=layer, part=pid)
            t0 = time.perf_counter()
            oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], None, G, "f16")
            t_total += time.perf_counter() - t0
            nbytes += algorithmic_bytes(K, N)
    return dict(value=round(nbytes / t_total / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample="layers 0..%d of the 32-layer step (%d GEMVs, %.1f MB), one thread, %.1f s"
                       % (layers - 1, 7 * layers, nbytes / 1e6, t_total),
                tokens_per_s=round(layers / LAYERS / t_total, 6))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-layers", type=int, default=2, help="layers of the step the CPU oracle runs (0 = skip)")
    ap.add_argument("--kernel-reps", type=int, default=5, help="event-timed passes over the step's launches")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs the decode step on a single MI355X "
              "(--gpus %d requested); multi-GPU sharding is described, not run." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_pack_amd as lb
    from bit_weight_only_pack_amd import synth

    torch.cuda.set_device(0)
    fmt, launches = build_step(lb, synth, torch)
    step_bytes = sum(L["bytes"] for L in launches)

    # ---- capture the step once as a HIP graph
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run_step(lb, fmt, launches, stream.cuda_stream)        # eager warm-up
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run_step(lb, fmt, launches, stream.cuda_stream)
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` replays, synchronized on both sides
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    # ---- dominant kernel: every launch of the step is the W4 GEMV kernel.
    # Each launch is bracketed by its own HIP event pair on the launch stream,
    # queued behind a busy stream so no host gap falls inside a pair.
    per = []
    with torch.cuda.stream(stream):
        for _ in range(args.kernel_reps):
            pairs = []
            torch.cuda._sleep(50_000_000)                       # bounded spin: keeps the GPU busy while we enqueue
            for L in launches:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                st = lb.lowbit_gemv(fmt, 1, L["N"], L["K"], G, L["packed"], L["x"], L["y"], L["ws"], L["wsb"],
                                    stream.cuda_stream)
                b.record(stream)
                if st != 0:
                    raise lb.LowbitError(st)
                pairs.append((a, b, L))
            torch.cuda.synchronize()
            per.append([(a.elapsed_time(b) * 1e3, L) for a, b, L in pairs])
    kern_us = np.array([[t for t, _ in rep] for rep in per])          # [reps][224]
    avg_launch_us = float(np.median(kern_us, axis=0).mean())
    bytes_per_launch = step_bytes / len(launches)
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    by_proj = {}
    med = np.median(kern_us, axis=0)
    for (t, L), m in zip(per[0], med):
        by_proj.setdefault(L["name"], []).append((m, L["bytes"]))
    proj_stats = {k: dict(us=round(float(np.mean([a for a, _ in v])), 3),
                          GBps=round(float(np.mean([b / (a * 1e-6) / 1e9 for a, b in v])), 1))
                  for k, v in by_proj.items()}

    profile_txt = os.path.join(ROOT, "profiles", "w4_gemv_decode_step_traffic.txt")
    traffic = None
    if os.path.exists(profile_txt):
        for line in open(profile_txt):
            if line.startswith("traffic_bytes_per_launch:"):
                traffic = float(line.split(":")[1])

    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; random INT4 codes, U[0.002,0.01] fp16 scales, N(0,1) fp16 inputs)",
        "config": {"workload": "llama3-8b-w4-decode-step", "layers": LAYERS, "gemvs_per_step": len(launches),
                   "M": 1, "group_size": G, "format": "int4 symmetric, fp16 scales", "bytes_per_step": step_bytes},
        "tokens_per_s": round(1e3 / ms_per_step, 2),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "kernel_sum_ms_per_step": round(float(med.sum()) / 1e3, 4),
        "per_projection": proj_stats,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "gemv_w4_kernel<G=128,sym,M=1>", "bytes_per_launch": round(bytes_per_launch),
                     "avg_launch_us": round(avg_launch_us, 3)},
    }
    if args.cpu_layers > 0:
        out["cpu_baseline"] = cpu_baseline(synth, args.cpu_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
