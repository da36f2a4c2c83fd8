"""Benchmark of the low-bit weight-only matmul on one MI355X.

Default workload (the headline): a Llama-3-8B-shaped W4 decode step.  One
step = the 224 decode GEMVs of a 32-layer decoder in layer order (q, k, v, o,
gate, up, down; K x N = 4096x4096, 4096x1024, 4096x1024, 4096x4096,
4096x14336, 4096x14336, 14336x4096), M = 1, symmetric INT4 with group size
128, fp16 scales U[0.002, 0.01], fp16 activations N(0,1) (as in a decoder
layer, q/k/v read one input vector and gate/up another; o and down have their
own), fp16 outputs.  Every weight is distinct (3.49 GB of packed
codes, 0.11 GB of scales): the step streams 3,603,169,280 algorithmic bytes
and no cache can hold it.  The projections that read the same layer input
(q/k/v, gate/up) are stacked into one weight matrix each, as serving stacks
store them, and run as one launch, so a layer is 4 launches in dependency
order (--mode batched packs each projection on its own and runs a group as
one lowbit_gemv_batched launch; --mode unfused runs 7; --mode chain runs the
whole step as one persistent launch whose stages wait for each other on the
GPU).  The step
is captured once as a HIP graph and replayed.  Printed: one JSON line with the step's effective HBM GB/s (the
metric), tokens/s (= steps/s at M = 1), the dominant kernel's roofline entry
and the CPU oracle's rate on a bounded sample of the same step.

Other workloads (--workload), one JSON line each:
  decode-asym : the same 224 GEMVs with asymmetric INT4, group size 32, int8
                zero points U{0..15}, M in {1, 2, 4, 8}, 1% outlier channels x20
  prefill     : W4 GEMM, M in {512, 2048, 8192}, (K, N) in {(4096, 14336),
                (14336, 4096)}, bf16 in/out, symmetric G=128
  decode-w4a8 : the decode-asym step with dynamic per-token INT8 activations
                (W4A8 on the int8 matrix cores), M in {1, 2, 4, 8}
  decode-bits : the decode step with uniform b-bit weights (--bits, default
                2,3,8; symmetric, G=128, M=1)
  moe         : a whole 3-bit LUT-codebook MoE layer, 128 experts, top-8 over
                256 tokens, hidden 2048, intermediate 768: MXFP8 of the hidden
                rows, alignment, gate/up GEMM, SiLU*up -> MXFP8, down GEMM,
                router-weighted combine
  tiny        : the 1x256x256 G=32 GEMV, latency per call (graph of 100 calls,
                and one call with a host synchronize), the oracle beside it

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import glob
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "W4 decode GEMV effective HBM GB/s (% of peak) and tokens/s at 8B shapes"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
LAYERS = 32


def w4_bytes(K, N, M, G, asym):
    """Bytes a W4 product must move at least once: codes (0.5 B/weight), fp16
    scales (2/G B/weight), int8 zero points (1/G B/weight, asymmetric), the
    fp16 input and output rows."""
    return N * K // 2 + N * (K // G) * 2 + (N * (K // G) if asym else 0) + M * K * 2 + M * N * 2


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
GROUPS_FUSED = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def stack_weights(ws):
    """The projections of one group as one weight matrix, rows in group order
    (q, k, v -> 6144 rows; gate, up -> 28672): the layout serving stacks keep
    for projections that read the same input.  Row n of the stacked product
    is row n of its projection's product."""
    out = {}
    for key in ws[0]:
        out[key] = None if ws[0][key] is None else np.concatenate([w[key] for w in ws], axis=0)
    return out


def build_step(lb, synth, torch, M, G, asym, workload_id, layout="stacked", outlier_frac=0.0):
    """Pack every weight of the 32-layer step on the GPU; return the launch list.
    As in a decoder layer, the projections of one group read the same input
    row(s): q/k/v share one activation vector, gate/up share one (drawn with
    the seed of the group's first projection); o and down have their own.
    layout: "stacked" (a group's weights stacked into one matrix, one
    single-problem launch per group), "batched" (each projection packed on
    its own, one lowbit_gemv_batched call per group) or "unfused" (one
    launch per projection)."""
    fmt = lb.LOWBIT_W4_ASYM if asym else lb.LOWBIT_W4_SYM
    projs = {name: (pid, K, N) for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS)}
    launches = []
    keep = []

    def pack(w, N, K):
        nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
        packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
        codes = torch.from_numpy(w["qweight"]).cuda()
        scales = torch.from_numpy(w["scales"].view(np.uint16)).cuda()
        zeros = torch.from_numpy(w["zeros"]).cuda() if asym else None
        lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, codes, scales, zeros, packed, nb))
        return packed

    for layer in range(LAYERS):
        for group in GROUPS_FUSED:
            pid0, K0, _ = projs[group[0]]
            x = torch.from_numpy(synth.activations_f16(M, K0, outlier_frac=outlier_frac, workload_id=workload_id,
                                                       layer=layer, part=pid0)).cuda()
            ws = []
            for name in group:
                pid, K, N = projs[name]
                ws.append(synth.w4_weights(N, K, G, asym=asym, scale_range=(0.002, 0.01), workload_id=workload_id,
                                           layer=layer, part=pid))
            items = []
            if layout == "stacked":
                N = sum(projs[name][2] for name in group)
                y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                items.append((pack(stack_weights(ws), N, K0), x, y, N, K0))
            else:
                for name, w in zip(group, ws):
                    _, K, N = projs[name]
                    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                    items.append((pack(w, N, K), x, y, N, K))
            del ws
            keep.append(items)
            if layout != "unfused":
                launches.append(dict(names=group, probs=lb.make_gemv_problems(items), count=len(items),
                                     bytes=sum(w4_bytes(K, N, M, G, asym) for (_, _, _, N, K) in items)))
            else:
                for (name, it) in zip(group, items):
                    launches.append(dict(names=(name,), probs=lb.make_gemv_problems([it]), count=1,
                                         bytes=w4_bytes(it[4], it[3], M, G, asym)))
    torch.cuda.synchronize()
    return fmt, launches, keep


def run_step(lb, fmt, M, G, launches, stream):
    for L in launches:
        st = lb.lowbit_gemv_batched(fmt, M, G, L["count"], L["probs"], stream)
        if st != 0:
            raise lb.LowbitError(st)


def build_chain(lb, torch, fmt, M, G, keep):
    """The whole step as one lowbit_gemv_chain: stage = launch group in layer
    order (q+k+v | o | gate+up | down per layer), so every group waits for the
    previous one exactly as the launches of the batched step do."""
    items, stages = [], []
    for gi, group in enumerate(keep):
        for it in group:
            items.append(it)
            stages.append(gi)
    probs = lb.make_gemv_problems(items)
    nb = lb.lowbit_gemv_chain_bytes(len(items), stages[-1] + 1)
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    chain = lb.lowbit_gemv_chain()
    lb.check(lb.lowbit_gemv_chain_init(chain, fmt, M, G, len(items), probs, stages, 0, buf, nb))
    return chain, (buf, probs)


def run_chain(lb, chain, stream):
    st = lb.lowbit_gemv_chain_run(chain, stream)
    if st != 0:
        raise lb.LowbitError(st)


def capture(torch, fn, stream):
    with torch.cuda.stream(stream):
        fn()                                                    # eager warm-up
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
    torch.cuda.synchronize()
    return graph


SCLK_SAMPLES = []                   # MHz, sampled during every graph-timed region


class ClockSampler:
    """Polls the driver's current shader-clock level (sysfs pp_dpm_sclk, the
    line marked '*') every 2 ms on a host thread while the block runs."""

    def __init__(self):
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.stop = threading.Event()
        self.thread = None

    def _read(self):
        for p in self.paths:
            try:
                for line in open(p).read().splitlines():
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self.stop.is_set():
            v = self._read()
            if v is not None:
                SCLK_SAMPLES.append(v)
            self.stop.wait(0.002)

    def __enter__(self):
        if self.paths:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()
        return self

    def __exit__(self, *exc):
        if self.thread is not None:
            self.stop.set()
            self.thread.join()


class PinnedOneCore:
    """Runs the block on one host core (the oracle legs are single-threaded)."""

    def __enter__(self):
        self.saved = None
        if hasattr(os, "sched_getaffinity"):
            self.saved = os.sched_getaffinity(0)
            os.sched_setaffinity(0, {min(self.saved)})
        return self

    def __exit__(self, *exc):
        if self.saved is not None:
            os.sched_setaffinity(0, self.saved)


def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "cpus_available": n}


def time_graph(torch, graph, stream, steps, warmup):
    """Exactly `steps` replays after `warmup`, synchronized on both sides.
    Returns (wall ms per replay, GPU-event ms per replay)."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with ClockSampler():
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for _ in range(steps):
                graph.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps


READ_CEILING_BYTES = 2 << 30        # 8x the 256 MB MALL


def read_ceiling(torch, lb, stream, reps=20):
    """The practical ceiling of HBM reads on this machine: lowbit_hbm_read (every
    16-byte block of a 2 GiB buffer read once, non-temporal loads) captured
    four times in a graph and replayed; bytes read per launch / time per
    launch, the best of three timed blocks.  Its shader-clock samples are kept
    out of the workload's."""
    buf = torch.zeros(READ_CEILING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(lb.LOWBIT_HBM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    st = stream.cuda_stream

    def run():
        for _ in range(4):
            lb.check(lb.lowbit_hbm_read(buf, READ_CEILING_BYTES, sink, st))
    n0 = len(SCLK_SAMPLES)
    graph = capture(torch, run, stream)
    gpu_ms = min(time_graph(torch, graph, stream, reps, 2)[1] for _ in range(3))   # best of three timed blocks
    del SCLK_SAMPLES[n0:]
    del graph, buf
    us = gpu_ms * 1e3 / 4
    return {"GBps": round(READ_CEILING_BYTES / (us * 1e-6) / 1e9, 1), "bytes_per_launch": READ_CEILING_BYTES,
            "us_per_launch": round(us, 2),
            "kernel": "hbm_read_kernel (lowbit_hbm_read: 1024 workgroups of 4 waves, a contiguous chunk per "
                      "wave, 16 KiB of 16-byte non-temporal loads in flight per wave)",
            "timing": "HIP events on the launch stream around graph replays of 4 launches, best of 3 blocks"}


KERNEL_SOURCES = ("bit_weight_only_pack_amd/csrc/gemv_w4.hip", "bit_weight_only_pack_amd/csrc/gemv_tile.hpp",
                  "bit_weight_only_pack_amd/csrc/lowbit_internal.hpp")
W4A8_KERNEL_SOURCES = ("bit_weight_only_pack_amd/csrc/gemv_w4a8.hip", "bit_weight_only_pack_amd/csrc/gemv_tile.hpp",
                       "bit_weight_only_pack_amd/csrc/lowbit_internal.hpp")
WB_KERNEL_SOURCES = ("bit_weight_only_pack_amd/csrc/gemv_wb.hip", "bit_weight_only_pack_amd/csrc/gemv_tile.hpp",
                     "bit_weight_only_pack_amd/csrc/lowbit_internal.hpp")
MOE_KERNEL_SOURCES = ("bit_weight_only_pack_amd/csrc/moe_lut3.hip", "bit_weight_only_pack_amd/csrc/moe_align.hpp",
                      "bit_weight_only_pack_amd/csrc/mxfp8.hpp", "bit_weight_only_pack_amd/csrc/lowbit_internal.hpp")


def kernel_source_hash(paths=KERNEL_SOURCES):
    """sha256 over the sources of a kernel (default: the decode GEMV's),
    recorded with its counter profile, so a profile of an older kernel is not
    reported."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(name, paths=KERNEL_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter profile
    (FETCH_SIZE and WRITE_SIZE runs, calibrated), and the profile's name;
    (None, reason) when there is none or it was taken on other kernel
    sources than the ones this tree builds."""
    path = os.path.join(ROOT, "profiles", name)
    if not name or not os.path.exists(path):
        return None, "no counter profile"
    value, src = None, None
    for line in open(path):
        if line.startswith("traffic_bytes_per_launch:"):
            value = float(line.split(":")[1])
        if line.startswith("kernel_source_sha256:"):
            src = line.split(":")[1].strip()
    if value is None:
        return None, "no counter profile"
    if src != kernel_source_hash(paths):
        return None, "profiles/%s was taken on other kernel sources" % name
    return value, "profiles/%s (rocprofv3 FETCH_SIZE and WRITE_SIZE runs, calibrated)" % name


def time_launch_groups(torch, lb, fmt, M, G, launches, stream, steps, warmup, run=None):
    """Mean duration of each launch group's launches: the group's launches of
    all layers, in layer order, captured as one graph and replayed (HIP events
    on the launch stream around the timed replays) -- the kernel's own
    average launch duration, back to back as in the step.  run(Ls) issues a
    list of launches (default: the W4A16 batched GEMV)."""
    if run is None:
        def run(Ls):
            run_step(lb, fmt, M, G, Ls, stream.cuda_stream)
    groups = {}
    for L in launches:
        groups.setdefault("+".join(L["names"]), []).append(L)
    out = {}
    reps = 4                   # copies of the group per graph: a replay's GPU time well above its launch cost
    for name, Ls in groups.items():
        g = capture(torch, lambda: [run(Ls) for _ in range(reps)], stream)
        _, gpu_ms = time_graph(torch, g, stream, steps, warmup)
        us = gpu_ms * 1e3 / (reps * len(Ls))
        nbytes = sum(L["bytes"] for L in Ls) / len(Ls)
        out[name] = dict(us=round(us, 3), bytes_per_launch=round(nbytes), GBps=round(nbytes / (us * 1e-6) / 1e9, 1),
                         launches=len(Ls))
        del g
    return out


def dominant_groups(per_group, layout):
    """(group names, mean us per launch, mean algorithmic bytes per launch) of
    the launches the step's dominant kernel runs: with stacked weights the
    single-problem streaming kernel runs q+k+v, o and gate+up; with batched
    ones the batch kernel runs q+k+v and gate+up."""
    names = ("q+k+v", "o", "gate+up") if layout == "stacked" else ("q+k+v", "gate+up")
    dom = [per_group[n] for n in names]
    us = sum(d["us"] * d["launches"] for d in dom) / sum(d["launches"] for d in dom)
    nb = sum(d["bytes_per_launch"] * d["launches"] for d in dom) / sum(d["launches"] for d in dom)
    return names, us, nb


def cpu_baseline_decode(synth, layers, M, G, asym, workload_id, outlier_frac=0.0, a8=False):
    """The CPU oracle on the first `layers` layers of the same step (single
    thread); a8: the W4A8 product (dynamic INT8 activations)."""
    import oracle
    projs = {name: (pid, K, N) for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS)}
    t_total = 0.0
    nbytes = 0
    for layer in range(layers):
        for group in GROUPS_FUSED:
            pid0, K0, _ = projs[group[0]]
            x = synth.activations_f16(M, K0, outlier_frac=outlier_frac, workload_id=workload_id, layer=layer,
                                      part=pid0)
            for name in group:
                pid, K, N = projs[name]
                w = synth.w4_weights(N, K, G, asym=asym, scale_range=(0.002, 0.01), workload_id=workload_id,
                                     layer=layer, part=pid)
                with PinnedOneCore():
                    t0 = time.perf_counter()
                    if a8:
                        oracle.w4a8_matmul(x, w["qweight"], w["scales"], w["zeros"], G)
                    else:
                        oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")
                    t_total += time.perf_counter() - t0
                nbytes += w4_bytes(K, N, M, G, asym)
    return dict(value=round(nbytes / t_total / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample="layers 0..%d of the 32-layer step (%d GEMVs, %.1f MB), one thread, %.1f s"
                       % (layers - 1, 7 * layers, nbytes / 1e6, t_total),
                tokens_per_s=round(M * layers / LAYERS / t_total, 6))


def bench_decode(args, torch, lb, synth):
    M, G, asym, wid = 1, 128, False, 1
    mode = args.mode
    fmt, launches, keep = build_step(lb, synth, torch, M, G, asym, wid,
                                     layout="stacked" if mode == "chain" else mode)
    step_bytes = sum(L["bytes"] for L in launches)
    stream = torch.cuda.Stream()
    if mode == "chain":
        chain, chain_keep = build_chain(lb, torch, fmt, M, G, keep)
        graph = capture(torch, lambda: run_chain(lb, chain, stream.cuda_stream), stream)
    else:
        graph = capture(torch, lambda: run_step(lb, fmt, M, G, launches, stream.cuda_stream), stream)
    ms_per_step, gpu_ms = time_graph(torch, graph, stream, args.steps, args.warmup)
    st_err = 0
    per_group = None
    if mode == "chain":
        # one launch per step: its duration is the event-timed replay region per step
        st, st_err = lb.lowbit_gemv_chain_error(chain, stream.cuda_stream)
        lb.check(st)
        if st_err:
            raise RuntimeError("chain dependency wait timed out (error word %d)" % st_err)
        roof = dict(kernel="gemv_chain_kernel<G=128,sym,MR=1> (the whole step, one launch)",
                    bytes_per_launch=step_bytes, avg_launch_us=gpu_ms * 1e3, traffic_name="")
    else:
        per_group = time_launch_groups(torch, lb, fmt, M, G, launches, stream, args.steps, args.warmup)
        if mode in ("stacked", "batched"):
            # the dominant kernel.  Stacked: gemv_w4_v2_single<128,sym,MR=1,T=4>
            # runs the q+k+v, o and gate+up launches (3 of every 4, about 3/4 of
            # the step's time).  Batched: gemv_w4_v2_kernel<128,sym,MR=1,T=4,NP=4>
            # runs q+k+v and gate+up.  Its figure is the bytes of those launches
            # over their measured durations.
            if mode == "stacked":
                names = ("q+k+v", "o", "gate+up")
                kname = "gemv_w4_v2_single<G=128,sym,MR=1,T=4> (the q+k+v, o and gate+up launches)"
                tname = "w4_gemv_decode_step_traffic.txt"
            else:
                names = ("q+k+v", "gate+up")
                kname = "gemv_w4_v2_kernel<G=128,sym,MR=1,T=4,NP=4> (the q+k+v and gate+up launches)"
                tname = ""
            dom = [per_group[n] for n in names]
            us = sum(d["us"] * d["launches"] for d in dom) / sum(d["launches"] for d in dom)
            nb = sum(d["bytes_per_launch"] * d["launches"] for d in dom) / sum(d["launches"] for d in dom)
            roof = dict(kernel=kname, bytes_per_launch=nb, avg_launch_us=us, traffic_name=tname)
        else:
            roof = dict(kernel="gemv_w4_v2 (one launch per GEMV, M=1)", bytes_per_launch=step_bytes / len(launches),
                        avg_launch_us=gpu_ms * 1e3 / len(launches), traffic_name="")
    achieved = roof["bytes_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e9
    traffic, traffic_source = read_traffic(roof["traffic_name"]) if roof["traffic_name"] else (None, "not taken")
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
        "config": {"workload": "llama3-8b-w4-decode-step", "layers": LAYERS, "gemvs_per_step": 7 * LAYERS,
                   "launches_per_step": len(launches) if mode != "chain" else 1, "M": M, "group_size": G, "mode": mode,
                   "format": "int4 symmetric, fp16 scales", "bytes_per_step": step_bytes},
        "tokens_per_s": round(1e3 / ms_per_step, 2),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_source": traffic_source, "kernel": roof["kernel"],
                     "bytes_per_launch": round(roof["bytes_per_launch"]),
                     "avg_launch_us": round(roof["avg_launch_us"], 3),
                     "timing": "HIP events on the launch stream around graph replays of this kernel's launches"},
        "step_mean_per_launch": {"launches_per_step": len(launches) if mode != "chain" else 1,
                                 "us": round(gpu_ms * 1e3 / (len(launches) if mode != "chain" else 1), 3),
                                 "GBps": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1)},
    }
    if per_group is not None:
        out["per_launch_group"] = per_group
    del keep
    if args.cpu_layers > 0:
        out["cpu_baseline"] = cpu_baseline_decode(synth, args.cpu_layers, M, G, asym, wid)
    return out


def bench_decode_asym(args, torch, lb, synth):
    G, asym, wid = 32, True, 2
    res = {}
    for M in (1, 2, 4, 8):
        fmt, launches, keep = build_step(lb, synth, torch, M, G, asym, wid, layout=args.layout, outlier_frac=0.01)
        step_bytes = sum(L["bytes"] for L in launches)
        stream = torch.cuda.Stream()
        graph = capture(torch, lambda: run_step(lb, fmt, M, G, launches, stream.cuda_stream), stream)
        ms, _ = time_graph(torch, graph, stream, args.steps, args.warmup)
        pg = time_launch_groups(torch, lb, fmt, M, G, launches, stream, max(5, args.steps // 5), 2)
        res["M=%d" % M] = dict(ms_per_step=round(ms, 4), GBps=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                               tokens_per_s=round(M * 1e3 / ms, 1), bytes_per_step=step_bytes,
                               kernel_sum_ms=round(sum(v["us"] * v["launches"] for v in pg.values()) / 1e3, 4),
                               per_launch_group=pg)
        del graph, keep, launches
        torch.cuda.empty_cache()
    r1 = res["M=1"]
    names, us, nb = dominant_groups(r1["per_launch_group"], args.layout)
    ach = nb / (us * 1e-6) / 1e9
    kname = ("gemv_w4_v2_single<G=32,asym,MR=1,T=4>" if args.layout == "stacked"
             else "gemv_w4_v2_kernel<G=32,asym,MR=1,T=4,NP=4>")
    traffic, traffic_source = (read_traffic("w4_gemv_asym_step_traffic.txt") if args.layout == "stacked"
                               else (None, "not taken for the batched layout"))
    return {"metric": "W4 asymmetric G=32 decode step effective HBM GB/s (M=1; M=2, 4, 8 in per_M)",
            "value": r1["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": r1["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "dtype": "f16", "data": "synthetic (seeded; INT4 codes, fp16 scales, int8 zero points, 1 % outlier "
                                    "fp16 inputs)", "vs_baseline": None,
            "config": {"workload": "llama3-8b-w4-asym-g32-decode-step", "M": 1, "M_list": [1, 2, 4, 8],
                       "group_size": G, "layout": args.layout},
            "tokens_per_s": r1["tokens_per_s"],
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_source": traffic_source,
                         "kernel": "%s (the %s launches, M=1)" % (kname, ", ".join(names)),
                         "bytes_per_launch": round(nb), "avg_launch_us": round(us, 3),
                         "timing": "HIP events on the launch stream around graph replays of this kernel's "
                                   "launches"},
            "per_M": res}


def run_step_a8(lb, fmt, M, G, launches, ws, wsb, stream):
    for L in launches:
        st = lb.lowbit_gemv_w4a8_batched(fmt, M, G, L["count"], L["probs"], ws, wsb, stream)
        if st != 0:
            raise lb.LowbitError(st)


def bench_decode_w4a8(args, torch, lb, synth):
    """The 224-GEMV step with W4A8 (dynamic per-token INT8 activations, the
    ARM pages' recipe: asymmetric INT4, group size 32) at M = 1, 2, 4, 8; one
    shared workspace serves every launch of the step (they run in stream
    order).  The W4A16 step of the same weights and inputs at M = 1 is timed
    beside it."""
    G, asym, wid = 32, True, 2
    res = {}
    m1 = None
    for M in [int(v) for v in args.m_list.split(",")]:
        fmt, launches, keep = build_step(lb, synth, torch, M, G, asym, wid, layout=args.layout, outlier_frac=0.01)
        step_bytes = sum(L["bytes"] for L in launches)
        wsb = max(lb.lowbit_gemv_w4a8_batched_workspace_bytes(fmt, M, G, L["count"], L["probs"]) for L in launches)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.Stream()
        graph = capture(torch, lambda: run_step_a8(lb, fmt, M, G, launches, ws, wsb, stream.cuda_stream), stream)
        ms, gpu_ms = time_graph(torch, graph, stream, args.steps, args.warmup)

        pg = time_launch_groups(torch, lb, fmt, M, G, launches, stream, max(5, args.steps // 5), 2,
                                run=lambda Ls: run_step_a8(lb, fmt, M, G, Ls, ws, wsb, stream.cuda_stream))
        res["M=%d" % M] = dict(ms_per_step=round(ms, 4), GBps=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                               tokens_per_s=round(M * 1e3 / ms, 1), bytes_per_step=step_bytes,
                               workspace_bytes=wsb,
                               kernel_sum_ms=round(sum(v["us"] * v["launches"] for v in pg.values()) / 1e3, 4),
                               per_launch_group=pg)
        if M == 1:
            g16 = capture(torch, lambda: run_step(lb, fmt, M, G, launches, stream.cuda_stream), stream)
            ms16, _ = time_graph(torch, g16, stream, args.steps, args.warmup)
            res["M=1"]["w4a16_same_step_ms"] = round(ms16, 4)
            del g16
            m1 = dict(ms=ms, gpu_ms=gpu_ms, bytes=step_bytes, n=len(launches), pg=pg)
        del graph, keep, launches, ws
        torch.cuda.empty_cache()
    names, avg_us, bpl = dominant_groups(m1["pg"], args.layout)
    ach = bpl / (avg_us * 1e-6) / 1e9
    kname = ("gemv_w4a8_single<G=32,asym,MR=1,T=4,FUSED>" if args.layout == "stacked"
             else "gemv_w4a8_batch<G=32,asym,MR=1,T=4,FUSED>")
    traffic, traffic_source = (read_traffic("w4a8_gemv_decode_step_traffic.txt", W4A8_KERNEL_SOURCES)
                               if args.layout == "stacked" else (None, "not taken for the batched layout"))
    out = {"metric": "W4A8 (dynamic INT8 activations) decode step effective HBM GB/s",
           "value": res["M=1"]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res["M=1"]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "i8 x u4 (int32 accumulate), fp32 scales, f16 out",
           "data": "synthetic (seeded; asymmetric INT4 G=32, zero points U{0..15}, N(0,1) fp16 inputs with 1% "
                   "outlier channels x20)",
           "config": {"workload": "llama3-8b-w4a8-asym-g32-decode-step", "M": [int(v) for v in args.m_list.split(",")],
                      "group_size": G, "layout": args.layout,
                      "launches_per_step": m1["n"]},
           "tokens_per_s": res["M=1"]["tokens_per_s"],
           "pct_of_hbm_peak": round(100 * res["M=1"]["GBps"] / HBM_PEAK_GBPS, 2),
           "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_source": traffic_source,
                        "kernel": "%s (the %s launches, M=1)" % (kname, ", ".join(names)),
                        "bytes_per_launch": round(bpl), "avg_launch_us": round(avg_us, 3),
                        "timing": "HIP events on the launch stream around graph replays of this kernel's "
                                  "launches"},
           "per_M": res}
    if args.cpu_layers > 0:
        out["cpu_baseline"] = cpu_baseline_decode(synth, 3 * args.cpu_layers, 1, G, asym, wid, outlier_frac=0.01,
                                                  a8=True)
    return out


def wb_bytes(K, N, M, G, bits):
    """Bytes a b-bit product must move at least once: codes (b/8 B/weight),
    fp16 scales, fp16 input and output rows (symmetric: no zero points)."""
    return N * K * bits // 8 + N * (K // G) * 2 + M * K * 2 + M * N * 2


def build_step_wb(lb, synth, torch, bits, G, workload_id, layout="stacked"):
    """The 224-GEMV step with uniform b-bit weights (symmetric), packed on the
    GPU layer by layer; the launch groups and layouts of build_step."""
    M = 1
    fmt = lb.LOWBIT_UINT(bits)
    projs = {name: (pid, K, N) for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS)}
    launches, keep = [], []

    def pack(w, N, K):
        nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
        packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
        codes = torch.from_numpy(w["codes"]).cuda()
        scales = torch.from_numpy(w["scales"].view(np.uint16)).cuda()
        lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, codes, scales, None, packed, nb))
        return packed

    for layer in range(LAYERS):
        for group in GROUPS_FUSED:
            pid0, K0, _ = projs[group[0]]
            x = torch.from_numpy(synth.activations_f16(M, K0, workload_id=workload_id, layer=layer, part=pid0)).cuda()
            ws = [synth.wb_weights(projs[name][2], projs[name][1], G, bits, workload_id=workload_id, layer=layer,
                                   part=projs[name][0]) for name in group]
            items = []
            if layout == "stacked":
                N = sum(projs[name][2] for name in group)
                y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                items.append((pack(stack_weights(ws), N, K0), x, y, N, K0))
            else:
                for name, w in zip(group, ws):
                    _, K, N = projs[name]
                    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                    items.append((pack(w, N, K), x, y, N, K))
            del ws
            keep.append(items)
            launches.append(dict(names=group, probs=lb.make_gemv_problems(items), count=len(items),
                                 bytes=sum(wb_bytes(K, N, M, G, bits) for (_, _, _, N, K) in items)))
        torch.cuda.synchronize()
    return fmt, launches, keep


def bench_decode_bits(args, torch, lb, synth):
    """The 8B decode step (M = 1, symmetric, G = 128) with uniform b-bit
    weights for each b of --bits; fewer bits stream fewer bytes."""
    G, M, wid = 128, 1, 6
    res = {}
    ref = None
    for bits in [int(v) for v in args.bits.split(",")]:
        fmt, launches, keep = build_step_wb(lb, synth, torch, bits, G, wid, args.layout)
        step_bytes = sum(L["bytes"] for L in launches)
        stream = torch.cuda.Stream()
        graph = capture(torch, lambda: run_step(lb, fmt, M, G, launches, stream.cuda_stream), stream)
        ms, gpu_ms = time_graph(torch, graph, stream, args.steps, args.warmup)
        pg = time_launch_groups(torch, lb, fmt, M, G, launches, stream, max(5, args.steps // 5), 2)
        res["b=%d" % bits] = dict(ms_per_step=round(ms, 4), GBps=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                                  tokens_per_s=round(1e3 / ms, 1), bytes_per_step=step_bytes,
                                  bytes_per_weight=bits / 8 + 2 / G, per_launch_group=pg)
        if ref is None or bits == 3:
            ref = dict(bits=bits, pg=pg)
        del graph, keep, launches
        torch.cuda.empty_cache()
    names, avg_us, bpl = dominant_groups(ref["pg"], args.layout)
    ach = bpl / (avg_us * 1e-6) / 1e9
    kname = ("gemv_wb_single<b=%d,G=128,sym,MR=1,T=4>" if args.layout == "stacked"
             else "gemv_wb_batch<b=%d,G=128,sym,MR=1,T=4>") % ref["bits"]
    key = "b=%d" % ref["bits"]
    traffic, traffic_source = (read_traffic("wb_gemv_decode_step_traffic.txt", WB_KERNEL_SOURCES)
                               if args.layout == "stacked" and ref["bits"] == 3
                               else (None, "taken for b = 3 with the stacked layout only"))
    out = {"metric": "b-bit decode step effective HBM GB/s and tokens/s at 8B shapes", "value": res[key]["GBps"],
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res[key]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded; uniform b-bit codes, U[0.002,0.01] fp16 scales, N(0,1) fp16 inputs)",
           "config": {"workload": "llama3-8b-uint-decode-step", "bits": [int(v) for v in args.bits.split(",")],
                      "value_bits": ref["bits"], "M": M, "group_size": G, "launches_per_step": 4 * LAYERS,
                      "layout": args.layout},
           "tokens_per_s": res[key]["tokens_per_s"],
           "pct_of_hbm_peak": round(100 * res[key]["GBps"] / HBM_PEAK_GBPS, 2),
           "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_source": traffic_source,
                        "kernel": "%s (the %s launches)" % (kname, ", ".join(names)),
                        "bytes_per_launch": round(bpl), "avg_launch_us": round(avg_us, 3),
                        "timing": "HIP events on the launch stream around graph replays of this kernel's "
                                  "launches"},
           "per_bits": res}
    if args.cpu_layers > 0:
        import oracle
        projs = {name: (pid, K, N) for pid, (name, K, N) in enumerate(synth.LLAMA3_8B_PROJS)}
        t_total, nbytes = 0.0, 0
        for group in GROUPS_FUSED:
            pid0, K0, _ = projs[group[0]]
            x = synth.activations_f16(M, K0, workload_id=wid, layer=0, part=pid0)
            for name in group:
                pid, K, N = projs[name]
                w = synth.wb_weights(N, K, G, ref["bits"], workload_id=wid, layer=0, part=pid)
                with PinnedOneCore():
                    t0 = time.perf_counter()
                    oracle.wb_matmul(x, w["codes"], w["scales"], None, ref["bits"], G)
                    t_total += time.perf_counter() - t0
                nbytes += wb_bytes(K, N, M, G, ref["bits"])
        out["cpu_baseline"] = {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": "layer 0 of the step at b=%d (7 GEMVs, %.1f MB), one thread, %.1f s"
                                         % (ref["bits"], nbytes / 1e6, t_total),
                               "tokens_per_s": round(1 / LAYERS / t_total, 6)}
    return out


def bench_prefill(args, torch, lb, synth):
    fmt, G = lb.LOWBIT_W4_SYM, 128
    res = {}
    total_flop, total_ms = 0.0, 0.0
    for K, N in ((4096, 14336), (14336, 4096)):
        w = synth.w4_weights(N, K, G, workload_id=3, layer=0, part=N)
        nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
        packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
        lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, torch.from_numpy(w["qweight"]).cuda(),
                                        torch.from_numpy(w["scales"].view(np.uint16)).cuda(), None, packed, nb))
        for M in (512, 2048, 8192):
            a = torch.from_numpy(synth.activations_bf16(M, K, workload_id=3, layer=M, part=K).view(np.int16)).cuda()
            c = torch.empty((M, N), dtype=torch.int16, device="cuda")
            wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMM, fmt, M, N, K, G)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
            stream = torch.cuda.Stream()

            def fn():
                st = lb.lowbit_gemm(fmt, M, N, K, G, packed, a, lb.LOWBIT_BF16, c, lb.LOWBIT_BF16, ws, wsb,
                                    stream.cuda_stream)
                if st != 0:
                    raise lb.LowbitError(st)
            graph = capture(torch, fn, stream)
            ms, _ = time_graph(torch, graph, stream, max(3, args.steps // 5), 2)
            flop = 2.0 * M * N * K
            tf = flop / (ms * 1e-3) / 1e12
            # context only: a dense bf16 GEMM of the same shape (torch.matmul,
            # the vendor library), the matrix cores' achievable rate on it
            a_bf = a.view(torch.bfloat16)
            b_dense = torch.randn((K, N), dtype=torch.bfloat16, device="cuda")
            c_bf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            with torch.cuda.stream(stream):
                for _ in range(2):
                    torch.matmul(a_bf, b_dense, out=c_bf)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = max(3, args.steps // 5)
                e0.record(stream)
                for _ in range(reps):
                    torch.matmul(a_bf, b_dense, out=c_bf)
                e1.record(stream)
            torch.cuda.synchronize()
            dense_ms = e0.elapsed_time(e1) / reps
            res["M=%d K=%d N=%d" % (M, K, N)] = dict(us=round(ms * 1e3, 1), TFLOPs=round(tf, 1),
                                                     pct_mfma_peak=round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2),
                                                     dense_bf16_matmul_us=round(dense_ms * 1e3, 1),
                                                     dense_bf16_matmul_TFLOPs=round(flop / (dense_ms * 1e-3) / 1e12, 1))
            total_flop += flop
            total_ms += ms
            del graph, b_dense, c_bf
    agg = total_flop / (total_ms * 1e-3) / 1e12
    return {"metric": "W4 prefill GEMM TFLOP/s (bf16 MFMA, fp32 accumulate)", "value": round(agg, 1),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": max(3, args.steps // 5), "warmup": 2,
            "ms_per_step": round(total_ms, 4), "higher_is_better": True, "scaling": "weak", "dtype": "bf16",
            "data": "synthetic",
            "vs_baseline": None, "config": {"workload": "w4-prefill-gemm", "group_size": G},
            "roofline": {"bound": "mfma", "achieved": round(agg, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(agg / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
            "per_shape": res}


def bench_moe(args, torch, lb, synth):
    """One whole MoE layer through lowbit_moe_layer, captured as one graph:
    MXFP8 of the hidden rows and routing alignment (one launch), gate/up
    grouped GEMM with SiLU(gate) * up -> MXFP8 in its epilogue, down grouped
    GEMM, router-weighted combine.  Two distinct weight sets (together larger
    than the MALL) alternate: one graph replay runs the layer on each, and the
    reported step is one layer; its bytes are those of the layer's own
    kernels.  The per-kernel breakdown times the same stages through their
    own entry points (quant_x and align separately), alternating the sets as
    well, plus the unfused pair (gate/up GEMM to bf16 rows, then SiLU * up ->
    MXFP8) for comparison.  The dominant kernel's roofline entry is the fused
    gate/up GEMM's."""
    T, E, top_k, bm, H, I = 256, 128, 8, 16, 2048, 768
    L3 = lb.LOWBIT_LUT3_E4M3
    S = T * top_k
    topk_np = synth.moe_routing(T, E, top_k, workload_id=4)
    w_np = synth.moe_topk_weights(T, E, top_k, workload_id=4)
    x_np = synth.activations_bf16(T, H, workload_id=4, part=2)
    topk = torch.from_numpy(topk_np).cuda()
    wts = torch.from_numpy(w_np).cuda()
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    cap = S + E * (bm - 1)
    ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npp = torch.empty(1, dtype=torch.int32, device="cuda")
    xq = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
    gu = torch.empty((S, 2 * I), dtype=torch.int16, device="cuda")
    aq = torch.empty((S, I), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((S, I // 32), dtype=torch.uint8, device="cuda")
    down = torch.empty((S, H), dtype=torch.int16, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()
    # two distinct weight sets (2 x 237 MB, more than the 256 MB MALL), used
    # alternately, so the timed layers read their experts from HBM
    packs = [{}, {}]
    weights = {}
    for ws_id in range(2):
        for name, (N, K, part) in (("w13", (2 * I, H, 0)), ("w2", (H, I, 1))):
            d = synth.lut3_weights(E, N, K, workload_id=4, layer=ws_id, part=part)
            nb = lb.lowbit_packed_bytes(L3, E, N, K, 0)
            packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
            lb.check(lb.lowbit_pack_weights(L3, E, N, K, 0, torch.from_numpy(d["idx"]).cuda(),
                                            torch.from_numpy(d["cb"]).cuda(), torch.from_numpy(d["ex"]).cuda(),
                                            packed, nb))
            packs[ws_id][name] = (packed, nb)
            if ws_id == 0:
                weights[name] = d
    st = stream.cuda_stream

    def stages(pk):
        # (name, call, algorithmic bytes, part of the layer)
        return [
            ("quant_x", lambda: lb.lowbit_mxfp8_quant(x, T, H, xq, xs, st), T * H * 2 + T * H + T * H // 32, True),
            ("align", lambda: lb.lowbit_moe_align(topk, T, top_k, E, bm, None, ids, offs, blk, npp, st), S * 4, True),
            ("gate_up", lambda: lb.lowbit_moe_gemm(L3, E, 2 * I, H, pk["w13"][0], E, xq, xs, T, top_k, ids, offs, blk,
                                                   S, bm, gu, st),
             pk["w13"][1] + T * H + T * H // 32 + S * 2 * I * 2, False),
            ("silu_mul_quant", lambda: lb.lowbit_moe_silu_mul_quant(gu, S, I, aq, as_, st),
             S * 2 * I * 2 + S * I + S * I // 32, False),
            ("gate_up_silu", lambda: lb.lowbit_moe_gemm_silu_quant(L3, E, I, H, pk["w13"][0], E, xq, xs, T, top_k, ids,
                                                                   offs, blk, S, bm, aq, as_, st),
             pk["w13"][1] + T * H + T * H // 32 + S * I + S * I // 32, True),
            ("down", lambda: lb.lowbit_moe_gemm(L3, E, H, I, pk["w2"][0], E, aq, as_, S, 1, ids, offs, blk, S, bm, down,
                                                st),
             pk["w2"][1] + S * I + S * I // 32 + S * H * 2, True),
            ("combine", lambda: lb.lowbit_moe_combine(down, wts, T, top_k, H, y, st), S * H * 2 + S * 4 + T * H * 2,
             True),
        ]
    steps_by_set = [stages(packs[0]), stages(packs[1])]
    steps = steps_by_set[0]

    wsb = lb.lowbit_moe_layer_workspace_bytes(T, top_k, E, H, I, bm)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def layer_pair():
        for pk in packs:
            lb.check(lb.lowbit_moe_layer(pk["w13"][0], pk["w2"][0], E, E, H, I, x, topk, wts, T, top_k, None, bm,
                                         y, ws, wsb, st))
    graph = capture(torch, layer_pair, stream)
    ms2, gpu_ms2 = time_graph(torch, graph, stream, args.steps, args.warmup)
    ms, gpu_ms = ms2 / 2, gpu_ms2 / 2                           # per layer
    per = {name: [] for name, _, _, _ in steps}
    with torch.cuda.stream(stream):
        for rep in range(6):
            evs = []
            torch.cuda._sleep(20_000_000)
            for name, fn, _, _ in steps_by_set[rep % 2]:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                lb.check(fn())
                b.record(stream)
                evs.append((name, a, b))
            torch.cuda.synchronize()
            for name, a, b in evs:
                per[name].append(a.elapsed_time(b) * 1e3)
    us = {k: float(np.median(v)) for k, v in per.items()}
    nbytes = {name: b for name, _, b, _ in steps}
    layer_bytes = sum(b for _, _, b, in_layer in steps if in_layer)
    gbps = layer_bytes / (ms * 1e-3) / 1e9
    gu_gbps = nbytes["gate_up_silu"] / (us["gate_up_silu"] * 1e-6) / 1e9
    moe_traffic, moe_traffic_source = read_traffic("moe_lut3_layer_traffic.txt", MOE_KERNEL_SOURCES)
    out = {"metric": "3-bit LUT MoE layer (MXFP8 in, align, gate/up with SiLU*up MXFP8, down, combine) "
                     "effective HBM GB/s",
           "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": 2 * args.steps,
           "warmup": 2 * args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8 (MXFP8 x LUT3 E4M3), fp32 accumulate, bf16 in/out",
           "data": "synthetic (seeded; N(0,1) router logits -> softmax top-8, N(0,1) bf16 hidden rows)",
           "config": {"workload": "lut3-moe-layer-256tok-128e-top8", "tokens": T, "experts": E, "top_k": top_k,
                      "block_m": bm, "hidden": H, "intermediate": I, "bytes_per_layer": layer_bytes,
                      "weight_sets": 2, "layers_per_replay": 2},
           "tokens_per_s": round(T * 1e3 / ms, 1),
           "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
           "gpu_ms_per_step": round(gpu_ms, 4),
           "roofline": {"bound": "hbm", "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": moe_traffic,
                        "traffic_source": moe_traffic_source,
                        "kernel": "moe_lut3_gemm_lds_kernel (gate/up, SiLU*up MXFP8 epilogue)",
                        "bytes_per_launch": nbytes["gate_up_silu"], "avg_launch_us": round(us["gate_up_silu"], 3)},
           "per_kernel_us": {k: round(v, 2) for k, v in us.items()},
           "per_kernel_GBps": {k: round(nbytes[k] / (us[k] * 1e-6) / 1e9, 1) for k in us if k != "align"}}
    if args.cpu_layers > 0:
        import oracle
        tok = np.arange(0, T, T // 16)
        with PinnedOneCore():
            t0 = time.perf_counter()
            oracle.moe_layer(weights["w13"], weights["w2"], x_np[tok], topk_np[tok], w_np[tok])
            dt = time.perf_counter() - t0
        full = dt * T / len(tok)
        out["cpu_baseline"] = {"value": round(layer_bytes / full / 1e9, 5), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": "%d of %d tokens (the whole layer on them), one thread, %.1f s; layer time "
                                         "extrapolated by token count" % (len(tok), T, dt),
                               "tokens_per_s": round(len(tok) / dt, 3)}
    return out


def bench_tiny(args, torch, lb, synth):
    """The tiny GEMV workload (M=1, K=256, N=256, G=32, symmetric, scales
    U[0.005, 0.02]): latency per call.  On the GPU: a graph of CALLS
    back-to-back calls (stream order, each a full launch) replayed, and a graph
    of one call replayed with a host synchronize after each replay (launch +
    completion as a caller sees it).  Beside it the CPU oracle on the same
    inputs, one thread on one pinned core."""
    N = K = 256
    G, M, CALLS = 32, 1, 100
    fmt = lb.LOWBIT_W4_SYM
    w = synth.w4_weights(N, K, G, scale_range=(0.005, 0.02), workload_id=0)
    x_np = synth.activations_f16(M, K, workload_id=0)
    nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
    packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, torch.from_numpy(w["qweight"]).cuda(),
                                    torch.from_numpy(w["scales"].view(np.uint16)).cuda(), None, packed, nb))
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()
    st = stream.cuda_stream

    def calls(n):
        for _ in range(n):
            r = lb.lowbit_gemv(fmt, M, N, K, G, packed, x, y, None, 0, st)
            if r != 0:
                raise lb.LowbitError(r)
    g100 = capture(torch, lambda: calls(CALLS), stream)
    ms100, gpu100 = time_graph(torch, g100, stream, args.steps, args.warmup)
    g1 = capture(torch, lambda: calls(1), stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            g1.replay()
    torch.cuda.synchronize()
    lat = []
    for _ in range(max(args.steps, 20)):
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            g1.replay()
        stream.synchronize()
        lat.append((time.perf_counter() - t0) * 1e6)
    # parity of the timed output against the oracle (smoke-level check)
    import oracle
    _, ref = oracle.w4_matmul(x_np, "f16", w["qweight"], w["scales"], None, G, "f16")
    got = y.cpu().numpy().astype(np.float64)
    refd = ref.view(np.float16).astype(np.float64)
    rel = float(np.linalg.norm(got - refd) / np.linalg.norm(refd))
    reps = 2000
    with PinnedOneCore():
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.w4_matmul(x_np, "f16", w["qweight"], w["scales"], None, G, "f16")
        cpu_s = (time.perf_counter() - t0) / reps
    nbytes = w4_bytes(K, N, M, G, False)
    us_call = gpu100 * 1e3 / CALLS
    out = {"metric": "W4A16 GEMV 1x256x256 G=32 latency (us per call)", "value": round(us_call, 3), "unit": "us",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(gpu100 / CALLS, 6),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded; INT4 codes U{0..15}, fp16 scales U[0.005,0.02], N(0,1) fp16 input)",
           "config": {"workload": "w4a16-gemv-1x256x256-g32", "M": M, "N": N, "K": K, "group_size": G,
                      "calls_per_graph": CALLS, "bytes_per_call": nbytes},
           "us_per_call_graph_of_%d" % CALLS: round(us_call, 3),
           "us_single_call_with_host_sync": {"median": round(float(np.median(lat)), 2),
                                             "p10": round(float(np.percentile(lat, 10)), 2),
                                             "p90": round(float(np.percentile(lat, 90)), 2)},
           "parity_rel_l2_vs_oracle": rel,
           "roofline": {"bound": "hbm", "achieved": round(nbytes / (us_call * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(nbytes / (us_call * 1e-6) / 1e9 / HBM_PEAK_GBPS, 6),
                        "traffic": None, "kernel": "gemv_w4_v2_single<G=32,sym,MR=1,T=2> (one workgroup per "
                                                   "16-row strip: 16 workgroups)",
                        "bytes_per_launch": nbytes, "avg_launch_us": round(us_call, 3),
                        "note": "latency-bound: 37,888 bytes stay in L2, the figure is launch and dependency cost"},
           "cpu_baseline": {"value": round(cpu_s * 1e6, 2), "unit": "us", "cores": 1, "kind": "oracle",
                            "sample": "the same GEMV, %d calls on one pinned core, %.2f s" % (reps, cpu_s * reps),
                            "ms_per_call": round(cpu_s * 1e3, 4)}}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode-asym", "decode-w4a8", "decode-bits", "prefill", "moe", "tiny"])
    ap.add_argument("--mode", default="stacked", choices=["stacked", "chain", "batched", "unfused"],
                    help="decode: stacked = the GEMVs sharing an input as one stacked weight matrix, one "
                         "launch each (4 per layer); batched = the same groups with each projection packed on "
                         "its own, one lowbit_gemv_batched launch per group; unfused = one launch per GEMV "
                         "(7 per layer); chain = the whole step as one persistent launch with stage "
                         "dependencies (stacked weights)")
    ap.add_argument("--layout", default="stacked", choices=["stacked", "batched"],
                    help="decode-asym, decode-w4a8, decode-bits: weights of the GEMVs sharing an input stacked "
                         "into one matrix, or packed one by one and batched")
    ap.add_argument("--cpu-layers", type=int, default=4, help="decode: layers the CPU oracle runs (0 = skip)")
    ap.add_argument("--m-list", default="1,2,4,8", help="decode-w4a8: token counts to run (must include 1)")
    ap.add_argument("--bits", default="2,3,8", help="decode-bits: code widths to run (1..8)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (a kernel of known traffic for counter runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step, prefill GEMM and MoE run on a single MI355X "
              "(--gpus %d requested); multi-GPU sharding is described, not run." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_pack_amd as lb
    from bit_weight_only_pack_amd import synth

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fn = {"decode": bench_decode, "decode-asym": bench_decode_asym, "decode-w4a8": bench_decode_w4a8,
          "decode-bits": bench_decode_bits, "prefill": bench_prefill, "moe": bench_moe,
          "tiny": bench_tiny}[args.workload]
    out = fn(args, torch, lb, synth)
    if args.workload in ("decode", "decode-asym", "decode-w4a8", "decode-bits", "moe"):
        # the practical read ceiling of this machine beside the HBM roofline (measured after the workload)
        ceil = read_ceiling(torch, lb, torch.cuda.Stream())
        out["hbm_read_ceiling"] = ceil
        out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / ceil["GBps"], 4)
    if SCLK_SAMPLES:
        v = sorted(SCLK_SAMPLES)
        out["gpu_sclk_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v),
                               "source": "sysfs pp_dpm_sclk, polled every 2 ms during the timed replays"}
    if "cpu_baseline" in out:
        out["cpu_baseline"].update(host_info())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
