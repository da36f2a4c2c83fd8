"""Graph replays of the entry points that bench.py captures in HIP graphs:
each call is captured once, the eager result recorded, and the graph replayed
three times with other eager work and synchronizations between the replays;
the output is refilled before every replay, and every replay must equal the
eager result bit for bit (the kernels are deterministic and enqueue no memset
nodes)."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
from bit_weight_only_pack_amd import synth
from gpu_util import dev, pack_w4

pytestmark = pytest.mark.gpu

WL = 700


def _replays(call, out, fill, other):
    """Eager result of call(), then three graph replays of it."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        out.fill_(fill)
        call(stream.cuda_stream)
    torch.cuda.synchronize()
    eager = out.clone()
    # the call wrote its output (a fill left in place would make every replay match)
    if out.dtype.is_floating_point and fill != fill:
        assert not torch.isnan(eager).any()
    else:
        assert not torch.equal(eager, torch.full_like(eager, fill))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call(stream.cuda_stream)
    torch.cuda.synchronize()
    got = []
    for rep in range(3):
        out.fill_(fill)
        other(rep)                                   # eager work between the replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        got.append(out.clone())
    return eager, got


def _other_gemm(rep):
    w = synth.w4_weights(64, 256, 32, workload_id=WL, part=90 + rep)
    fmt, packed, _ = pack_w4(w, 32)
    a = dev(synth.activations_bf16(8, 256, workload_id=WL, part=rep).view(np.int16))
    c = torch.empty((8, 64), dtype=torch.int16, device="cuda")
    lb.check(lb.lowbit_gemm(fmt, 8, 64, 256, 32, packed, a, lb.LOWBIT_BF16, c, lb.LOWBIT_BF16))


@pytest.mark.parametrize("M,N,K,G", [(64, 256, 4096, 128), (256, 384, 512, 128), (130, 272, 1024, 32)])
def test_gemm_graph_replays(M, N, K, G):
    w = synth.w4_weights(N, K, G, workload_id=WL, layer=M, part=N)
    fmt, packed, _ = pack_w4(w, G)
    a = dev(synth.activations_bf16(M, K, workload_id=WL, layer=M, part=K).view(np.int16))
    c = torch.empty((M, N), dtype=torch.int16, device="cuda")
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMM, fmt, M, N, K, G)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def call(st):
        lb.check(lb.lowbit_gemm(fmt, M, N, K, G, packed, a, lb.LOWBIT_BF16, c, lb.LOWBIT_BF16, ws, wsb, st))
    eager, got = _replays(call, c, -1, _other_gemm)
    for g in got:
        assert torch.equal(g, eager)


def test_gemv_batched_graph_replays():
    G, M = 128, 1
    shapes = [(1024, 4096), (256, 4096), (512, 4096)]
    probs, keep = [], []
    x = dev(synth.activations_f16(M, 4096, workload_id=WL, part=5))
    out = torch.empty(M * sum(N for N, _ in shapes), dtype=torch.float16, device="cuda")
    off = 0
    for i, (N, K) in enumerate(shapes):
        w = synth.w4_weights(N, K, G, workload_id=WL, part=10 + i)
        fmt, packed, _ = pack_w4(w, G)
        y = out[off:off + M * N].view(M, N)           # every output is a view of `out`
        off += M * N
        probs.append((packed, x, y, N, K))
        keep.append(packed)
    arr = lb.make_gemv_problems(probs)

    def call(st):
        lb.check(lb.lowbit_gemv_batched(lb.LOWBIT_W4_SYM, M, G, len(probs), arr, st))

    eager, got = _replays(call, out, float("nan"), _other_gemm)
    for g in got:
        assert torch.equal(g, eager)


def test_gemv_w4a8_batched_graph_replays():
    G, M = 32, 4
    shapes = [(512, 2048), (256, 2048)]
    x = dev(synth.activations_f16(M, 2048, workload_id=WL, part=6))
    out = torch.empty(M * sum(N for N, _ in shapes), dtype=torch.float16, device="cuda")
    probs, keep = [], []
    off = 0
    for i, (N, K) in enumerate(shapes):
        w = synth.w4_weights(N, K, G, asym=True, workload_id=WL, part=20 + i)
        fmt, packed, _ = pack_w4(w, G)
        y = out[off:off + M * N].view(M, N)
        off += M * N
        probs.append((packed, x, y, N, K))
        keep.append(packed)
    arr = lb.make_gemv_problems(probs)
    wsb = lb.lowbit_gemv_w4a8_batched_workspace_bytes(lb.LOWBIT_W4_ASYM, M, G, len(probs), arr)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def call(st):
        lb.check(lb.lowbit_gemv_w4a8_batched(lb.LOWBIT_W4_ASYM, M, G, len(probs), arr, ws, wsb, st))

    eager, got = _replays(call, out, float("nan"), _other_gemm)
    for g in got:
        assert torch.equal(g, eager)


def test_moe_layer_graph_replays():
    T, E, top_k, H, I, bm = 64, 16, 4, 512, 256, 16
    L3 = lb.LOWBIT_LUT3_E4M3
    packs = []
    for N, K, part in ((2 * I, H, 0), (H, I, 1)):
        d = synth.lut3_weights(E, N, K, workload_id=WL, part=part)
        nb = lb.lowbit_packed_bytes(L3, E, N, K, 0)
        p = torch.empty(nb, dtype=torch.uint8, device="cuda")
        lb.check(lb.lowbit_pack_weights(L3, E, N, K, 0, dev(d["idx"]), dev(d["cb"]), dev(d["ex"]), p, nb))
        packs.append(p)
    x = dev(synth.activations_bf16(T, H, workload_id=WL, part=3).view(np.int16))
    topk = dev(synth.moe_routing(T, E, top_k, workload_id=WL))
    wts = dev(synth.moe_topk_weights(T, E, top_k, workload_id=WL))
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    wsb = lb.lowbit_moe_layer_workspace_bytes(T, top_k, E, H, I, bm)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def call(st):
        lb.check(lb.lowbit_moe_layer(packs[0], packs[1], E, E, H, I, x, topk, wts, T, top_k, None, bm, y, ws, wsb,
                                     st))
    eager, got = _replays(call, y, 0, _other_gemm)
    for g in got:
        assert torch.equal(g, eager)
