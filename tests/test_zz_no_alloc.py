"""lowbit_gemv_w4a8_batched_noalloc (the W4A8 batched GEMV whose activation
blocks live in the library's static device scratch, for callers that cannot
allocate; 512 KiB) against lowbit_gemv_w4a8_batched with a caller workspace, through
the C ABI: outputs bit-identical, on consecutive calls whose second input is
smaller than the first (the scratch keeps the first call's bytes), at one
token (no scratch), and a plan larger than the scratch is refused before
anything is enqueued."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64, pack_w4

pytestmark = pytest.mark.gpu

WL = 150


def _problems(shapes, M, G, tag):
    items, ws_, xs = [], [], []
    for i, (K, N) in enumerate(shapes):
        w = synth.w4_weights(N, K, G, asym=True, workload_id=WL, layer=tag, part=i)
        x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=tag + M, part=i)
        _, packed, _ = pack_w4(w, G)
        items.append((packed, dev(x)))
        ws_.append(w)
        xs.append(x)
    return items, ws_, xs


def _run(shapes, items, M, G, noalloc):
    ys = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda") for (_, N) in shapes]
    probs = lb.make_gemv_problems([(p, x, y, N, K) for (p, x), y, (K, N) in zip(items, ys, shapes)])
    if noalloc:
        lb.check(lb.lowbit_gemv_w4a8_batched_noalloc(lb.LOWBIT_W4_ASYM, M, G, len(shapes), probs))
    else:
        wsb = lb.lowbit_gemv_w4a8_batched_workspace_bytes(lb.LOWBIT_W4_ASYM, M, G, len(shapes), probs)
        ws = torch.full((max(wsb, 1),), 0xCD, dtype=torch.uint8, device="cuda")
        lb.check(lb.lowbit_gemv_w4a8_batched(lb.LOWBIT_W4_ASYM, M, G, len(shapes), probs, ws, wsb))
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def test_noalloc_equals_workspace_form_on_two_calls():
    G = 32
    # first call: q/k/v shapes at M = 8 (the larger scratch image), then a
    # smaller one: two ragged problems at M = 2
    big = [(4096, 4096), (4096, 1024), (4096, 1024)]
    small = [(1056, 300), (512, 64)]
    for shapes, M, tag in ((big, 8, 1), (small, 2, 2)):
        items, ws_, xs = _problems(shapes, M, G, tag)
        got = _run(shapes, items, M, G, noalloc=True)
        want = _run(shapes, items, M, G, noalloc=False)
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint16), w.view(np.uint16))
        # and against the oracle, as every W4A8 product
        for g, w, x in zip(got, ws_, xs):
            _, ref = oracle.w4a8_matmul(x, w["qweight"], w["scales"], w["zeros"], G)
            assert_close(f16_to_f64(g), f16_to_f64(ref), "noalloc M=%d" % M)


def test_noalloc_one_token_and_down_shape():
    G = 32
    for shapes, M in (([(4096, 4096), (4096, 1024)], 1), ([(14336, 512)], 8)):
        items, _, _ = _problems(shapes, M, G, 3)
        got = _run(shapes, items, M, G, noalloc=True)
        want = _run(shapes, items, M, G, noalloc=False)
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint16), w.view(np.uint16))


def test_noalloc_refuses_plans_beyond_the_scratch():
    FAKE = 1 << 20
    # 8 problems of M = 8, K = 14336: about 1 MB of activation blocks, more
    # than the 512 KiB scratch (one such problem, the down projection, fits)
    probs = lb.make_gemv_problems([(FAKE, FAKE, FAKE, 64, 14336)] * 8)
    need = lb.lowbit_gemv_w4a8_batched_workspace_bytes(lb.LOWBIT_W4_ASYM, 8, 32, 8, probs)
    assert need > (512 << 10)
    assert lb.lowbit_gemv_w4a8_batched_noalloc(lb.LOWBIT_W4_ASYM, 8, 32, 8, probs) == lb.LOWBIT_E_WORKSPACE
