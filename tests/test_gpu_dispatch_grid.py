"""GPU parity over the GEMV launchers' whole dispatch grid, against the CPU
oracle, through the C ABI.

Each GEMV family (W4A16, uniform b-bit, W4A8) picks a kernel instantiation
from the problem: the group size G, symmetric or asymmetric weights, the
accumulators per lane (1 for M = 1, 2 for M <= 8, 4 above), the K tiles per wave
(K = 256 -> 2, K = 2048 -> 4, K = 9216 -> 5 of an 8-tile wave) and one problem
or a batch.  These small cases (N = 48, three 16-row strips, the last K tile
complete) reach every combination, so no instantiation that a decode workload
may select goes unchecked.  At M = 4 and K = 9216 the W4A16 activation block
no longer fits the streaming kernel's LDS and the per-wave activation-ring
kernel runs; K = 20480 (more than 8 tiles per wave) reaches the round-based
kernel.

Bar: rel-L2 <= 1e-3 and max |error| <= 1e-2 * max |y_ref| against the
oracle's fp16-rounded output ("Low Bit ARM kernels", group-wise quantization;
"Low Bit Metal Kernels", int4_matmul: each nibble dequantized with its
group's scale before the multiply-add)."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64, gemv, pack_w4

pytestmark = pytest.mark.gpu

WL = 140
N = 48
GRID_K = [256, 2048, 9216]
GRID_M = [1, 2, 4]


def _w4(K, G, asym, part):
    return synth.w4_weights(N, K, G, asym=asym, workload_id=WL, layer=K // 128, part=G * 10 + part)


def _x(M, K, part):
    return synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=M, part=K + part)


def _y(M, n=N):
    return torch.full((M, n), float("nan"), dtype=torch.float16, device="cuda")


# ---------------------------------------------------------------- W4A16
@pytest.mark.parametrize("K", GRID_K)
@pytest.mark.parametrize("M", GRID_M)
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_w4_gemv_grid(G, asym, M, K):
    w = _w4(K, G, asym, 0)
    x = _x(M, K, 0)
    fmt, packed, _ = pack_w4(w, G)
    y = _y(M)
    lb.check(lb.lowbit_gemv(fmt, M, N, K, G, packed, dev(x), y, None, 0))
    torch.cuda.synchronize()
    _, ref = oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")
    assert_close(f16_to_f64(y.cpu().numpy()), f16_to_f64(ref), "W4 G=%d asym=%s M=%d K=%d" % (G, asym, M, K))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("G,asym", [(128, False), (32, True)])
def test_w4_gemv_round_based_long_k(G, asym, M):
    """K = 20480 (160 K tiles): more than 8 tiles per wave even with 16
    waves, so neither streaming form applies and the round-based kernel
    (activations staged a round of K tiles at a time) runs, with one, two
    (M = 2..8) and four (M = 16) accumulators per lane."""
    K = 20480
    w = _w4(K, G, asym, 30)
    x = _x(M, K, 30)
    fmt, packed, _ = pack_w4(w, G)
    y = _y(M)
    lb.check(lb.lowbit_gemv(fmt, M, N, K, G, packed, dev(x), y, None, 0))
    torch.cuda.synchronize()
    _, ref = oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")
    assert_close(f16_to_f64(y.cpu().numpy()), f16_to_f64(ref), "round-based G=%d asym=%s M=%d" % (G, asym, M))


@pytest.mark.parametrize("count", [3, 6])          # 4-problem and 8-problem batch kernels
@pytest.mark.parametrize("M", GRID_M)
@pytest.mark.parametrize("K", [2048, 9216])
@pytest.mark.parametrize("G,asym", [(32, True), (128, False), (64, True)])
def test_w4_gemv_batched_grid(G, asym, K, M, count):
    items, ref = [], []
    for i in range(count):
        w = _w4(K, G, asym, 10 + i)
        x = _x(M, K, 10 + i)
        fmt, packed, _ = pack_w4(w, G)
        items.append((packed, dev(x), _y(M), N, K))
        ref.append(f16_to_f64(oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")[1]))
    probs = lb.make_gemv_problems(items)
    lb.check(lb.lowbit_gemv_batched(fmt, M, G, count, probs))
    torch.cuda.synchronize()
    for i, it in enumerate(items):
        assert_close(f16_to_f64(it[2].cpu().numpy()), ref[i], "batched %d/%d" % (i, count))


TWO_STRIP_CASES = ([(32, True, 2048, M) for M in (4, 5, 8, 16)] + [(128, False, 2048, M) for M in (4, 5, 8, 16)] +
                   [(G, asym, K, 8) for G in (32, 64, 128) for asym in (False, True) for K in (256, 2048)
                    if (G, asym, K) not in ((32, True, 2048), (128, False, 2048))])


@pytest.mark.parametrize("G,asym,K,M", TWO_STRIP_CASES)
def test_w4_gemv_two_strip_batches(G, asym, K, M):
    """Batches of 2-4 problems with at least 1024 strips and 5 or more tokens
    run two 16-row strips per workgroup (M = 4: one, the other side of the
    boundary), for every group size, both weight forms and both tile counts
    per wave it takes (K = 256: 2, K = 2048: 4).  Each problem here has an odd
    strip count with a ragged last strip (N = 8200: 513 strips, the last of 8
    rows), so the last workgroup of each problem has a strip past the end.
    The outputs equal the one-problem launches' (one strip per workgroup) bit
    for bit, and the oracle within the bar."""
    n = 8200
    ws, xs, packs, singles = [], [], [], []
    for i in range(2):
        w = synth.w4_weights(n, K, G, asym=asym, workload_id=WL, layer=90 + M, part=i)
        x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=90 + M, part=i)
        fmt, packed, _ = pack_w4(w, G)
        y1 = _y(M, n)
        lb.check(lb.lowbit_gemv(fmt, M, n, K, G, packed, dev(x), y1, None, 0))
        ws.append(w)
        xs.append(dev(x))
        packs.append(packed)
        singles.append(y1)
    yb = [_y(M, n) for _ in range(2)]
    probs = lb.make_gemv_problems([(packs[i], xs[i], yb[i], n, K) for i in range(2)])
    lb.check(lb.lowbit_gemv_batched(fmt, M, G, 2, probs))
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 64), np.arange(n - 72, n)])
    for i in range(2):
        got = yb[i].cpu().numpy()
        assert np.array_equal(got.view(np.uint16), singles[i].cpu().numpy().view(np.uint16)), "problem %d" % i
        w = ws[i]
        sub = dict(qweight=w["qweight"][rows], scales=w["scales"][rows],
                   zeros=None if w["zeros"] is None else w["zeros"][rows])
        x = xs[i].cpu().numpy()
        _, ref = oracle.w4_matmul(x, "f16", sub["qweight"], sub["scales"], sub["zeros"], G, "f16")
        assert_close(f16_to_f64(got[:, rows]), f16_to_f64(ref), "two-strip G=%d M=%d problem %d" % (G, M, i))


# ---------------------------------------------------------------- uniform b-bit
@pytest.mark.parametrize("K", [256, 2048, 9216])
@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("bits,G", [(2, 32), (3, 128), (5, 64), (8, 128)])
def test_wb_gemv_grid(bits, G, asym, M, K):
    w = synth.wb_weights(N, K, G, bits, asym=asym, workload_id=WL, layer=bits, part=K + M)
    x = _x(M, K, bits)
    fmt = lb.LOWBIT_UINT(bits, asym)
    nb = lb.lowbit_packed_bytes(fmt, 1, N, K, G)
    packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_pack_weights(fmt, 1, N, K, G, dev(w["codes"]), dev(w["scales"].view(np.uint16)),
                                    dev(w["zeros"]) if asym else None, packed, nb))
    y = _y(M)
    lb.check(lb.lowbit_gemv(fmt, M, N, K, G, packed, dev(x), y, None, 0))
    torch.cuda.synchronize()
    _, ref = oracle.wb_matmul(x, w["codes"], w["scales"], w["zeros"], bits, G)
    assert_close(f16_to_f64(y.cpu().numpy()), f16_to_f64(ref), "b=%d G=%d asym=%s M=%d K=%d" % (bits, G, asym, M, K))


# ---------------------------------------------------------------- W4A8
@pytest.mark.parametrize("K", GRID_K)
@pytest.mark.parametrize("M", GRID_M)
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_w4a8_gemv_grid(G, asym, M, K):
    w = _w4(K, G, asym, 20)
    x = _x(M, K, 20)
    fmt, packed, _ = pack_w4(w, G)
    y = _y(M)
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV_W4A8, fmt, M, N, K, G)
    ws = torch.full((max(wsb, 1),), 0xAB, dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_gemv_w4a8(fmt, M, N, K, G, packed, dev(x), y, ws, wsb))
    torch.cuda.synchronize()
    _, ref = oracle.w4a8_matmul(x, w["qweight"], w["scales"], w["zeros"], G)
    assert_close(f16_to_f64(y.cpu().numpy()), f16_to_f64(ref), "W4A8 G=%d asym=%s M=%d K=%d" % (G, asym, M, K))


@pytest.mark.parametrize("G,asym,K,M", TWO_STRIP_CASES)
def test_w4_gemv_two_strip_single_problem(G, asym, K, M):
    """One problem of at least 1024 strips with 5 or more tokens (a stacked
    weight matrix) runs two strips per workgroup with its fields as kernel
    arguments (M = 4: one).  N = 16392 gives 1025 strips, the last of 8 rows,
    so the last workgroup has a strip past the end.  The output equals two
    launches over the matrix's halves (512 and 513 strips, one strip per
    workgroup) bit for bit, and the oracle within the bar."""
    n, h = 16392, 8192
    w = synth.w4_weights(n, K, G, asym=asym, workload_id=WL, layer=95 + M, part=K)
    x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=95 + M, part=K)
    y = gemv(w, x, G)
    halves = [{k: None if v is None else v[a:b] for k, v in w.items()} for a, b in ((0, h), (h, n))]
    sep = np.concatenate([gemv(wh, x, G) for wh in halves], axis=1)
    assert np.array_equal(y.view(np.uint16), sep.view(np.uint16))
    rows = np.concatenate([np.arange(0, 64), np.arange(h - 8, h + 8), np.arange(n - 40, n)])
    _, ref = oracle.w4_matmul(x, "f16", w["qweight"][rows], w["scales"][rows],
                              None if w["zeros"] is None else w["zeros"][rows], G, "f16")
    assert_close(f16_to_f64(y[:, rows]), f16_to_f64(ref), "two-strip single G=%d M=%d" % (G, M))


# ---------------------------------------------------------------- the down projection at small batch
@pytest.mark.parametrize("M", [2, 3, 4, 8])
def test_w4_gemv_down_shape_sym_g128_small_batch(M):
    """K = 14336, N = 4096, symmetric G = 128 at M = 2 (the streaming kernel
    with two accumulator rows and eight tiles per wave) and M = 3, 4, 8 (the
    per-wave activation-ring kernel); 128 seeded weight rows against the
    oracle."""
    K, Nd, G = 14336, 4096, 128
    w = synth.w4_weights(Nd, K, G, scale_range=(0.002, 0.01), workload_id=1, layer=M, part=6)
    x = synth.activations_f16(M, K, workload_id=1, layer=M, part=6)
    fmt, packed, _ = pack_w4(w, G)
    y = _y(M, Nd)
    lb.check(lb.lowbit_gemv(fmt, M, Nd, K, G, packed, dev(x), y, None, 0))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(60 + M).choice(Nd, size=128, replace=False))
    _, ref = oracle.w4_matmul(x, "f16", w["qweight"][rows], w["scales"][rows], None, G, "f16")
    assert_close(f16_to_f64(y.cpu().numpy())[:, rows], f16_to_f64(ref), "down sym M=%d" % M)
