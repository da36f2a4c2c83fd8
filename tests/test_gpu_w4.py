"""GPU parity of the W4 path (pack, unpack, dequant, GEMV) against the CPU
oracle, through the C ABI.  Unpack/dequant: bit-exact.  GEMV: rel-L2 <= 1e-3
and max |error| <= 1e-2 * max |y_ref| against the oracle's fp16-rounded
output; special cases (one-hot input) bit-exact."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64, gemv, pack_w4

pytestmark = pytest.mark.gpu

WL = 100  # workload id range used by these tests


def _weights(N, K, G, asym, part=0, scale_range=(0.002, 0.01)):
    return synth.w4_weights(N, K, G, asym=asym, scale_range=scale_range, workload_id=WL, layer=N, part=K * 10 + part)


def _ref(w, x, G):
    _, yb = oracle.w4_matmul(x, "f16", w["qweight"], w["scales"], w["zeros"], G, "f16")
    return f16_to_f64(yb)


# ---------------------------------------------------------------- pack / unpack / dequant
@pytest.mark.parametrize("N,K,G,asym,E", [
    (256, 256, 32, False, 1),
    (100, 96, 32, True, 1),        # ragged N and K
    (48, 1024, 128, False, 2),     # two matrices in one blob
    (17, 192, 64, True, 1),
    (1024, 4096, 128, False, 1),
])
def test_pack_unpack_roundtrip_bitexact(N, K, G, asym, E):
    ws = [_weights(N, K, G, asym, part=e) for e in range(E)]
    w = dict(qweight=np.stack([v["qweight"] for v in ws]), scales=np.stack([v["scales"] for v in ws]),
             zeros=np.stack([v["zeros"] for v in ws]) if asym else None)
    fmt, packed, nbytes = pack_w4(w, G, E=E)
    codes = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((E, N, K // G), dtype=torch.int16, device="cuda")
    zeros = torch.zeros((E, N, K // G), dtype=torch.int8, device="cuda") if asym else None
    lb.check(lb.lowbit_unpack_weights(fmt, E, N, K, G, packed, nbytes, codes, scales, zeros))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), w["qweight"])
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), w["scales"].view(np.uint16))
    if asym:
        assert np.array_equal(zeros.cpu().numpy(), w["zeros"])


def test_pack_is_deterministic_and_fully_written():
    w = _weights(40, 160, 32, True)
    fmt, p1, nb = pack_w4(w, 32)
    p2 = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
    codes, scales, zeros = dev(w["qweight"]), dev(w["scales"].view(np.uint16)), dev(w["zeros"])
    lb.check(lb.lowbit_pack_weights(fmt, 1, 40, 160, 32, codes, scales, zeros, p2, nb))
    torch.cuda.synchronize()
    assert torch.equal(p1[:nb], p2)


@pytest.mark.parametrize("N,K,G,asym", [(256, 256, 32, False), (100, 96, 32, True), (64, 512, 64, True),
                                        (33, 384, 128, False)])
def test_dequant_bitexact(N, K, G, asym):
    w = _weights(N, K, G, asym)
    if asym:  # zero points over the whole int8 range
        w["zeros"] = np.random.default_rng(5).integers(-128, 128, size=w["zeros"].shape).astype(np.int8)
    fmt, packed, nbytes = pack_w4(w, G)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    lb.check(lb.lowbit_dequant(fmt, N, K, G, packed, nbytes, out))
    torch.cuda.synchronize()
    ref = oracle.w4_dequant(w["qweight"], w["scales"], w["zeros"], G)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- GEMV parity
def test_gemv_tiny_workload():
    """M=1, K=256, N=256, G=32, symmetric; scales U[0.005,0.02] (the tiny GEMV workload)."""
    w = synth.w4_weights(256, 256, 32, scale_range=(0.005, 0.02), workload_id=0)
    x = synth.activations_f16(1, 256, workload_id=0)
    assert_close(f16_to_f64(gemv(w, x, 32)), _ref(w, x, 32), "tiny")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 12, 16])
@pytest.mark.parametrize("N,K,G,asym", [
    (256, 256, 32, False),
    (300, 1056, 32, True),      # ragged N, ragged last K tile (1056 = 8*128 + 32)
    (1000, 2048, 64, True),
    (48, 4096, 128, False),
    (16, 128, 128, True),       # a single tile
])
def test_gemv_parity(M, N, K, G, asym):
    w = _weights(N, K, G, asym)
    x = synth.activations_f16(M, K, outlier_frac=0.01 if asym else 0.0, workload_id=WL, layer=M, part=K)
    assert_close(f16_to_f64(gemv(w, x, G)), _ref(w, x, G), "M=%d N=%d K=%d G=%d" % (M, N, K, G))


@pytest.mark.parametrize("G,asym", [(32, True), (128, False), (64, False)])
def test_gemv_one_hot_is_exact(G, asym):
    """x = e_k per row => y[m][n] = RNE_fp16(w[n][k_m]) bit-exactly."""
    N, K = 96, 512
    w = _weights(N, K, G, asym)
    ks = [0, 1, 37, 128, 255, 300, 510, 511]
    x = np.zeros((len(ks), K), np.float16)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = gemv(w, x, G)
    W = oracle.w4_dequant(w["qweight"], w["scales"], w["zeros"], G)
    want = np.stack([W[:, k] for k in ks]).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


def test_gemv_deterministic():
    w = _weights(512, 4096, 128, False)
    x = synth.activations_f16(4, 4096, workload_id=WL, part=1)
    fmt, packed, _ = pack_w4(w, 128)
    y1 = gemv(w, x, 128, packed)
    y2 = gemv(w, x, 128, packed)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_gemv_empty_and_zero_k():
    w = _weights(32, 128, 32, False)
    fmt, packed, _ = pack_w4(w, 32)
    assert lb.lowbit_gemv(fmt, 0, 32, 128, 32, packed, None, None) == lb.LOWBIT_OK
    # K = 0: an empty sum, every output is +0
    y = torch.full((2, 32), 7.0, dtype=torch.float16, device="cuda")
    nb = lb.lowbit_packed_bytes(fmt, 1, 32, 0, 32)
    p0 = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
    x0 = torch.zeros((2, 8), dtype=torch.float16, device="cuda")
    lb.check(lb.lowbit_gemv(fmt, 2, 32, 0, 32, p0, x0, y))
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_gemv_codes_at_zero_point_give_zero():
    N, K, G = 64, 256, 32
    z = np.random.default_rng(3).integers(0, 16, size=(N, K // G)).astype(np.int8)
    codes = np.repeat(z.astype(np.uint8), G, axis=1)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w = dict(qweight=q, scales=np.full((N, K // G), 0.01, np.float16), zeros=z)
    x = synth.activations_f16(3, K, workload_id=WL, part=9)
    assert np.all(gemv(w, x, G) == 0)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("M", [1, 8])
def test_gemv_full_int8_zero_points(G, M):
    """Zero points over the whole int8 range, both ends included (the layout
    accepts any int8 z; q - z then spans -128 .. 143): asymmetric G = 32 forms
    the exact operand q - z from 1152 + q and 1152 + z (z + 128 in the low
    byte), G = 64 / 128 run the offset chains.  Against the oracle."""
    N, K = 256, 1024
    rng = np.random.default_rng(77 + G + M)
    w = _weights(N, K, G, True, part=7)
    z = rng.integers(-128, 128, size=(N, K // G)).astype(np.int8)
    z[0, :] = -128
    z[1, :] = 127
    z[2, 0::2] = -128
    z[2, 1::2] = 127
    w["zeros"] = z
    x = synth.activations_f16(M, K, workload_id=WL, layer=M, part=G)
    assert_close(f16_to_f64(gemv(w, x, G)), _ref(w, x, G), "full int8 z G=%d M=%d" % (G, M))


# ---------------------------------------------------------------- full 8B shapes
@pytest.mark.parametrize("proj", [p[0] for p in synth.LLAMA3_8B_PROJS])
def test_gemv_llama3_8b_shapes_sym(proj):
    """Every Llama-3-8B projection at full size, M=1, symmetric G=128 (the
    decode-step workload), all outputs against the oracle."""
    _, K, N = next(p for p in synth.LLAMA3_8B_PROJS if p[0] == proj)
    pid = [p[0] for p in synth.LLAMA3_8B_PROJS].index(proj)
    w = synth.w4_weights(N, K, 128, scale_range=(0.002, 0.01), workload_id=1, layer=0, part=pid)
    x = synth.activations_f16(1, K, workload_id=1, layer=0, part=pid)
    assert_close(f16_to_f64(gemv(w, x, 128)), _ref(w, x, 128), proj)


@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_gemv_llama3_8b_shapes_asym_g32(proj, M):
    """Asymmetric G=32 with 1% outlier channels x20 at full size; outputs of a
    seeded sample of 128 weight rows are checked against the oracle.  The
    down projection (K = 14336) at M = 2 runs the streaming kernel with two
    accumulator rows and eight tiles per wave, the one the asymmetric decode
    step times at M = 2."""
    _, K, N = next(p for p in synth.LLAMA3_8B_PROJS if p[0] == proj)
    pid = [p[0] for p in synth.LLAMA3_8B_PROJS].index(proj)
    w = synth.w4_weights(N, K, 32, asym=True, workload_id=2, layer=0, part=pid)
    x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=2, layer=M, part=pid)
    y = f16_to_f64(gemv(w, x, 32))
    rows = np.sort(np.random.default_rng(pid).choice(N, size=128, replace=False))
    sub = dict(qweight=w["qweight"][rows], scales=w["scales"][rows], zeros=w["zeros"][rows])
    assert_close(y[:, rows], _ref(sub, x, 32), "%s M=%d" % (proj, M))


# ---------------------------------------------------------------- stacked projections
@pytest.mark.parametrize("group,M,G,asym", [(("q", "k", "v"), 1, 128, False), (("gate", "up"), 8, 32, True)])
def test_gemv_stacked_equals_separate(group, M, G, asym):
    """Projections that read the same input, stacked into one weight matrix
    (q, k, v: 6144 rows; gate, up: 28672 rows, which at M = 8 runs two strips
    per workgroup), give each projection's own single-GEMV output bit for
    bit: every 16-row strip is computed the same way whatever the matrix it
    sits in."""
    projs = {name: (K, N) for name, K, N in synth.LLAMA3_8B_PROJS}
    K = projs[group[0]][0]
    ws = [synth.w4_weights(projs[n][1], K, G, asym=asym, workload_id=WL, layer=85, part=i)
          for i, n in enumerate(group)]
    x = synth.activations_f16(M, K, outlier_frac=0.01 if asym else 0.0, workload_id=WL, layer=85)
    sep = np.concatenate([gemv(w, x, G) for w in ws], axis=1)
    st = {k: None if ws[0][k] is None else np.concatenate([w[k] for w in ws], axis=0) for k in ws[0]}
    y = gemv(st, x, G)
    assert y.shape == sep.shape
    assert np.array_equal(y.view(np.uint16), sep.view(np.uint16))


# ---------------------------------------------------------------- batched GEMV
def test_gemv_batched_matches_single_bitexact():
    """q/k/v-shaped problems (same K) in one launch give exactly the single-GEMV results."""
    shapes = [(4096, 4096), (4096, 1024), (4096, 1024)]
    ws, xs, packs = [], [], []
    for i, (K, N) in enumerate(shapes):
        w = synth.w4_weights(N, K, 128, workload_id=WL, layer=77, part=i)
        ws.append(w)
        xs.append(synth.activations_f16(1, K, workload_id=WL, layer=77, part=i))
        packs.append(pack_w4(w, 128)[1])
    singles = [gemv(w, x, 128, p) for w, x, p in zip(ws, xs, packs)]
    xd = [dev(x) for x in xs]
    yd = [torch.full((1, N), float("nan"), dtype=torch.float16, device="cuda") for _, N in shapes]
    probs = lb.make_gemv_problems([(packs[i], xd[i], yd[i], shapes[i][1], shapes[i][0]) for i in range(3)])
    lb.check(lb.lowbit_gemv_batched(lb.LOWBIT_W4_SYM, 1, 128, 3, probs))
    torch.cuda.synchronize()
    for y, s in zip(yd, singles):
        assert np.array_equal(y.cpu().numpy().view(np.uint16), s.view(np.uint16))


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_batched_mixed_shapes(M):
    """Different K and ragged N in one launch (asymmetric G=32), each against the oracle."""
    shapes = [(4096, 4096), (14336, 512), (1056, 300), (256, 16)]
    items = []
    for i, (K, N) in enumerate(shapes):
        w = synth.w4_weights(N, K, 32, asym=True, workload_id=WL, layer=78, part=i)
        x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=78 + M, part=i)
        fmt, packed, _ = pack_w4(w, 32)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        items.append((w, x, packed, dev(x), y, N, K))
    probs = lb.make_gemv_problems([(p, xd, y, N, K) for (_, _, p, xd, y, N, K) in items])
    lb.check(lb.lowbit_gemv_batched(lb.LOWBIT_W4_ASYM, M, 32, len(items), probs))
    torch.cuda.synchronize()
    for (w, x, _, _, y, N, K) in items:
        assert_close(f16_to_f64(y.cpu().numpy()), _ref(w, x, 32), "batched K=%d N=%d" % (K, N))
