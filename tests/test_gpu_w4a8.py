"""GPU parity of the W4A8 path (dynamic per-token INT8 activations x packed
INT4 weights on the int8 matrix cores) against the CPU oracle, through the C
ABI.  Activation codes and scales: bit-exact (both sides take the integer
decisions in binary32).  Products: rel-L2 <= 1e-3 and max |error| <= 1e-2 *
max |y_ref| against the oracle's fp16-rounded output; the one-hot case, codes
at the zero point and zero rows bit-exact."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64, pack_w4

pytestmark = pytest.mark.gpu

WL = 110  # workload id range used by these tests


def _weights(N, K, G, asym, part=0):
    return synth.w4_weights(N, K, G, asym=asym, workload_id=WL, layer=N, part=K * 10 + part)


def _ref(w, x, G):
    _, yb = oracle.w4a8_matmul(x, w["qweight"], w["scales"], w["zeros"], G)
    return f16_to_f64(yb)


def gemv_a8(w, x, G, packed=None):
    q = w["qweight"]
    N, K = q.shape[0], 2 * q.shape[1]
    M = x.shape[0]
    if packed is None:
        fmt, packed, _ = pack_w4(w, G)
    else:
        fmt = lb.LOWBIT_W4_ASYM if w["zeros"] is not None else lb.LOWBIT_W4_SYM
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV_W4A8, fmt, M, N, K, G)
    ws = torch.full((max(wsb, 1),), 0xAB, dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_gemv_w4a8(fmt, M, N, K, G, packed, dev(x), y, ws, wsb))
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ---------------------------------------------------------------- activation quantization
@pytest.mark.parametrize("M,K,outliers", [(1, 4096, 0.0), (8, 14336, 0.01), (3, 96, 0.0), (5, 8, 0.0),
                                          (16, 1024, 0.01)])
def test_quant_act_bitexact(M, K, outliers):
    x = synth.activations_f16(M, K, outlier_frac=outliers, workload_id=WL, layer=M, part=K)
    if M >= 3:
        x[1] *= np.float16(0.001)      # rows of very different magnitudes
        x[2] = 0                       # a zero row
    xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    lb.check(lb.lowbit_quant_act_i8(M, K, dev(x), xq, sx))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act_i8(x)
    assert np.array_equal(xq.cpu().numpy(), rq)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quant_act_ties_and_grid():
    """Rows on the quantization grid (largest magnitude 127 * 2^e): integer and
    half-integer multiples of 2^e, whose codes are exact (ties to even)."""
    vals = np.concatenate([np.arange(-127, 128), np.arange(-126, 127) + 0.5, [127.0] * 4])   # K = 512
    x = np.stack([(vals * 2.0 ** e).astype(np.float16) for e in (-4, 0, 3)])
    xq = torch.zeros(x.shape, dtype=torch.int8, device="cuda")
    sx = torch.zeros((3,), dtype=torch.float32, device="cuda")
    lb.check(lb.lowbit_quant_act_i8(3, x.shape[1], dev(x), xq, sx))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act_i8(x)
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(sx.cpu().numpy(), rs)


# ---------------------------------------------------------------- GEMV parity
@pytest.mark.parametrize("M,N,K,G,asym", [
    (1, 256, 256, 32, False),          # the tiny GEMV shape
    (1, 300, 1056, 32, True),          # ragged N, K not a multiple of 128
    (1, 512, 4096, 128, False),
    (2, 64, 1536, 64, True),
    (3, 200, 2048, 32, True),
    (4, 96, 4096, 128, True),          # 4 token rows (workspace)
    (8, 80, 4096, 32, False),
    (2, 48, 14336, 32, True),          # workspace, long K
    (16, 32, 1024, 64, False),
    (1, 16, 16384, 128, True),         # the longest K (8 tiles per wave)
])
def test_gemv_w4a8_parity(M, N, K, G, asym):
    w = _weights(N, K, G, asym)
    x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=M, part=N)
    assert_close(f16_to_f64(gemv_a8(w, x, G)), _ref(w, x, G), "M=%d N=%d K=%d G=%d asym=%s" % (M, N, K, G, asym))


@pytest.mark.parametrize("G,asym", [(32, True), (128, False)])
@pytest.mark.parametrize("M", [1, 8])
def test_gemv_w4a8_one_hot_is_exact(G, asym, M):
    """x = 127 e_k gives scale 1 and one code 127, so y = RNE_fp16(127 w[:, k])
    exactly (every intermediate is an exact integer or an exact product)."""
    N, K = 64, 512
    w = synth.w4_weights(N, K, G, asym=asym, workload_id=WL, layer=3, part=G)
    x = np.zeros((M, K), np.float16)
    for m in range(M):
        x[m, (37 * m + 5) % K] = 127
    y = gemv_a8(w, x, G)
    _, yb = oracle.w4a8_matmul(x, w["qweight"], w["scales"], w["zeros"], G)
    assert np.array_equal(y.view(np.uint16), yb)


def test_gemv_w4a8_zero_point_and_zero_rows():
    N, K, G = 48, 1024, 32
    r = np.random.default_rng(5)
    z = r.integers(0, 16, size=(N, K // G)).astype(np.int8)
    codes = np.repeat(z.astype(np.uint8), G, axis=1)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w = dict(qweight=q, scales=np.full((N, K // G), 0.01, np.float16), zeros=z)
    x = synth.activations_f16(3, K, workload_id=WL, part=7)
    assert np.all(gemv_a8(w, x, G) == 0)
    w2 = _weights(N, K, G, True, part=1)
    x[1] = 0
    y = gemv_a8(w2, x, G)
    assert np.all(y[1] == 0)
    assert_close(f16_to_f64(y), _ref(w2, x, G), "zero row")


def test_gemv_w4a8_deterministic():
    w = _weights(1024, 4096, 32, True, part=2)
    x = synth.activations_f16(1, 4096, workload_id=WL, part=8)
    fmt, packed, _ = pack_w4(w, 32)
    a = gemv_a8(w, x, 32, packed)
    b = gemv_a8(w, x, 32, packed)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


# ---------------------------------------------------------------- full 8B shapes
@pytest.mark.parametrize("proj", [p[0] for p in synth.LLAMA3_8B_PROJS])
def test_gemv_w4a8_llama3_8b_shapes_m1(proj):
    """Every Llama-3-8B projection at full size, M=1, asymmetric G=32 (the
    W4A8 decode workload), all outputs against the oracle."""
    _, K, N = next(p for p in synth.LLAMA3_8B_PROJS if p[0] == proj)
    pid = [p[0] for p in synth.LLAMA3_8B_PROJS].index(proj)
    w = synth.w4_weights(N, K, 32, asym=True, workload_id=5, layer=0, part=pid)
    x = synth.activations_f16(1, K, outlier_frac=0.01, workload_id=5, layer=0, part=pid)
    assert_close(f16_to_f64(gemv_a8(w, x, 32)), _ref(w, x, 32), proj)


@pytest.mark.parametrize("proj", ["q", "gate", "down"])
@pytest.mark.parametrize("M", [2, 4, 8])
def test_gemv_w4a8_llama3_8b_shapes_batch(proj, M):
    """M = 2, 4, 8 at full size (workspace front end); a seeded
    sample of 128 weight rows against the oracle."""
    _, K, N = next(p for p in synth.LLAMA3_8B_PROJS if p[0] == proj)
    pid = [p[0] for p in synth.LLAMA3_8B_PROJS].index(proj)
    w = synth.w4_weights(N, K, 32, asym=True, workload_id=5, layer=M, part=pid)
    x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=5, layer=M, part=pid)
    y = f16_to_f64(gemv_a8(w, x, 32))
    rows = np.sort(np.random.default_rng(pid + 10 * M).choice(N, size=128, replace=False))
    sub = dict(qweight=w["qweight"][rows], scales=w["scales"][rows], zeros=w["zeros"][rows])
    assert_close(y[:, rows], _ref(sub, x, 32), "%s M=%d" % (proj, M))


# ---------------------------------------------------------------- batched
@pytest.mark.parametrize("M", [1, 8])
def test_gemv_w4a8_batched_matches_single_bitexact(M):
    """q/k/v-shaped problems in one launch give exactly the single-GEMV
    results (same K, so the same wave split and summation order; M = 8 goes
    through the workspace); a ragged problem in the same launch (another wave
    split than alone) against the oracle."""
    shapes = [(4096, 4096), (4096, 1024), (4096, 1024), (1056, 300)]
    ws_, xs, packs = [], [], []
    for i, (K, N) in enumerate(shapes):
        w = synth.w4_weights(N, K, 32, asym=True, workload_id=WL, layer=90 + M, part=i)
        ws_.append(w)
        xs.append(synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=90 + M, part=i))
        packs.append(pack_w4(w, 32)[1])
    singles = [gemv_a8(w, x, 32, p) for w, x, p in zip(ws_, xs, packs)]
    xd = [dev(x) for x in xs]
    yd = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda") for _, N in shapes]
    probs = lb.make_gemv_problems([(packs[i], xd[i], yd[i], shapes[i][1], shapes[i][0]) for i in range(len(shapes))])
    wsb = lb.lowbit_gemv_w4a8_batched_workspace_bytes(lb.LOWBIT_W4_ASYM, M, 32, len(shapes), probs)
    assert (wsb > 0) == (M > 1)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_gemv_w4a8_batched(lb.LOWBIT_W4_ASYM, M, 32, len(shapes), probs, ws, wsb))
    torch.cuda.synchronize()
    for y, s in zip(yd[:3], singles[:3]):
        assert np.array_equal(y.cpu().numpy().view(np.uint16), s.view(np.uint16))
    assert_close(f16_to_f64(yd[3].cpu().numpy()), _ref(ws_[3], xs[3], 32), "batched ragged")
