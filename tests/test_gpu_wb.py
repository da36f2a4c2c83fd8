"""GPU parity of the uniform b-bit formats (LOWBIT_UINT(bits, asym), b = 1..8)
against the CPU oracle, through the C ABI: pack / unpack round trips and
dequantization bit-exact; GEMV rel-L2 <= 1e-3 and max |error| <= 1e-2 *
max |y_ref| against the oracle's fp16-rounded output; one-hot inputs and codes
at the zero point bit-exact."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, dev, f16_to_f64

pytestmark = pytest.mark.gpu

WL = 130
BITS = [1, 2, 3, 4, 5, 6, 7, 8]


def _w(N, K, G, bits, asym, part=0):
    return synth.wb_weights(N, K, G, bits, asym=asym, workload_id=WL, layer=bits, part=N * 7 + K + part)


def pack(w, G, bits, E=1):
    c = w["codes"]
    N, K = c.shape[-2], c.shape[-1]
    asym = w["zeros"] is not None
    fmt = lb.LOWBIT_UINT(bits, asym)
    nb = lb.lowbit_packed_bytes(fmt, E, N, K, G)
    p = torch.full((max(nb, 1),), 0x5A, dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_pack_weights(fmt, E, N, K, G, dev(c), dev(w["scales"].view(np.uint16)),
                                    dev(w["zeros"]) if asym else None, p, nb))
    return fmt, p, nb


def gemv(w, x, G, bits, packed=None):
    c = w["codes"]
    N, K = c.shape
    M = x.shape[0]
    fmt = lb.LOWBIT_UINT(bits, w["zeros"] is not None)
    if packed is None:
        _, packed, _ = pack(w, G, bits)
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    lb.check(lb.lowbit_gemv(fmt, M, N, K, G, packed, dev(x), y, None, 0))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _ref(w, x, G, bits):
    _, yb = oracle.wb_matmul(x, w["codes"], w["scales"], w["zeros"], bits, G)
    return f16_to_f64(yb)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("asym", [False, True])
def test_wb_pack_roundtrip_and_dequant_bitexact(bits, asym):
    N, K, G, E = 40, 416, 32, 2                         # ragged N and K, two matrices
    ws = [_w(N, K, G, bits, asym, part=e) for e in range(E)]
    w = dict(codes=np.stack([v["codes"] for v in ws]), scales=np.stack([v["scales"] for v in ws]),
             zeros=np.stack([v["zeros"] for v in ws]) if asym else None)
    fmt, p, nb = pack(w, G, bits, E)
    codes = torch.zeros((E, N, K), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((E, N, K // G), dtype=torch.int16, device="cuda")
    zeros = torch.zeros((E, N, K // G), dtype=torch.int8, device="cuda") if asym else None
    lb.check(lb.lowbit_unpack_weights(fmt, E, N, K, G, p, nb, codes, scales, zeros))
    one = nb // E
    wd = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    lb.check(lb.lowbit_dequant(fmt, N, K, G, p[one:], one, wd))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), w["codes"])
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), w["scales"].view(np.uint16))
    if asym:
        assert np.array_equal(zeros.cpu().numpy(), w["zeros"])
    ref = oracle.wb_dequant(ws[1]["codes"], ws[1]["scales"], ws[1]["zeros"], bits, G)
    assert np.array_equal(wd.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_uint4_packs_to_the_int4_blob():
    """At b = 4 the b-bit layout is the INT4 layout: the same codes packed from
    bytes (LOWBIT_UINT(4)) and from nibble pairs (LOWBIT_W4) give one blob."""
    for asym in (False, True):
        w = _w(48, 512, 64, 4, asym)
        _, p8, nb = pack(w, 64, 4)
        q = (w["codes"][:, 0::2] | (w["codes"][:, 1::2] << 4)).astype(np.uint8)
        fmt = lb.LOWBIT_W4_ASYM if asym else lb.LOWBIT_W4_SYM
        nb4 = lb.lowbit_packed_bytes(fmt, 1, 48, 512, 64)
        assert nb4 == nb
        p4 = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
        lb.check(lb.lowbit_pack_weights(fmt, 1, 48, 512, 64, dev(q), dev(w["scales"].view(np.uint16)),
                                        dev(w["zeros"]) if asym else None, p4, nb))
        torch.cuda.synchronize()
        assert torch.equal(p8, p4)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M,N,K,G,asym", [
    (1, 256, 256, 32, False),
    (1, 300, 1056, 32, True),          # ragged N, K not a multiple of 128
    (3, 96, 2048, 128, True),
    (8, 64, 4096, 64, False),
    (12, 48, 1024, 32, True),          # four accumulators per lane (M > 8)
    (1, 64, 16384, 128, False),        # the longest K the b-bit GEMV accepts
    (4, 48, 16384, 32, True),          # longest K with the most tokens whose x and partial sums fit the LDS
])
def test_wb_gemv_parity(bits, M, N, K, G, asym):
    w = _w(N, K, G, bits, asym, part=M)
    x = synth.activations_f16(M, K, outlier_frac=0.01, workload_id=WL, layer=bits, part=N + M)
    assert_close(f16_to_f64(gemv(w, x, G, bits)), _ref(w, x, G, bits), "b=%d M=%d N=%d K=%d" % (bits, M, N, K))


@pytest.mark.parametrize("bits", [1, 3, 6, 8])
def test_wb_gemv_one_hot_and_zero_point_exact(bits):
    N, K, G = 64, 512, 32
    w = _w(N, K, G, bits, True, part=9)
    x = np.zeros((2, K), np.float16)
    x[0, 5] = 1
    x[1, 300] = 1
    _, yb = oracle.wb_matmul(x, w["codes"], w["scales"], w["zeros"], bits, G)
    assert np.array_equal(gemv(w, x, G, bits).view(np.uint16), yb)
    mid = dict(codes=np.full((N, K), 1 << (bits - 1), np.uint8), scales=w["scales"], zeros=None)
    xr = synth.activations_f16(3, K, workload_id=WL, part=bits)
    assert np.all(gemv(mid, xr, G, bits) == 0)


@pytest.mark.parametrize("bits", [2, 3, 8])
@pytest.mark.parametrize("proj", ["q", "gate", "down"])
def test_wb_gemv_llama3_8b_shapes(bits, proj):
    """Full-size projections at M = 1, symmetric G = 128; 128 seeded rows
    against the oracle."""
    _, K, N = next(p for p in synth.LLAMA3_8B_PROJS if p[0] == proj)
    pid = [p[0] for p in synth.LLAMA3_8B_PROJS].index(proj)
    w = synth.wb_weights(N, K, 128, bits, workload_id=6, layer=bits, part=pid)
    x = synth.activations_f16(1, K, workload_id=6, layer=bits, part=pid)
    y = f16_to_f64(gemv(w, x, 128, bits))
    rows = np.sort(np.random.default_rng(pid + bits).choice(N, size=128, replace=False))
    sub = dict(codes=w["codes"][rows], scales=w["scales"][rows], zeros=None)
    assert_close(y[:, rows], _ref(sub, x, 128, bits), "%s b=%d" % (proj, bits))


def test_wb_batched_matches_single_bitexact():
    shapes = [(4096, 4096), (4096, 1024), (4096, 1024)]
    bits, G = 3, 128
    ws, xs, packs = [], [], []
    for i, (K, N) in enumerate(shapes):
        w = synth.wb_weights(N, K, G, bits, workload_id=WL, layer=77, part=i)
        ws.append(w)
        xs.append(synth.activations_f16(1, K, workload_id=WL, layer=77, part=i))
        packs.append(pack(w, G, bits)[1])
    singles = [gemv(w, x, G, bits, p) for w, x, p in zip(ws, xs, packs)]
    xd = [dev(x) for x in xs]
    yd = [torch.full((1, N), float("nan"), dtype=torch.float16, device="cuda") for _, N in shapes]
    probs = lb.make_gemv_problems([(packs[i], xd[i], yd[i], shapes[i][1], shapes[i][0]) for i in range(3)])
    lb.check(lb.lowbit_gemv_batched(lb.LOWBIT_UINT(bits), 1, G, 3, probs))
    torch.cuda.synchronize()
    for y, s in zip(yd, singles):
        assert np.array_equal(y.cpu().numpy().view(np.uint16), s.view(np.uint16))
