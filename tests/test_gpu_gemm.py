"""GPU parity of the prefill GEMM (lowbit_gemm) against the CPU oracle, through
the C ABI: rel-L2 <= 1e-3 and max |error| <= 1e-2 * max |ref| against the
oracle's output rounded to the same output type."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, bf16_bits_to_f64, dev, f16_to_f64, pack_w4

pytestmark = pytest.mark.gpu

WL = 300


def _acts(M, K, dtype, part=0):
    if dtype == "bf16":
        return synth.activations_bf16(M, K, workload_id=WL, layer=M, part=K * 10 + part)
    return synth.activations_f16(M, K, workload_id=WL, layer=M, part=K * 10 + part).view(np.uint16)


def _to_f64(bits, dtype):
    return bf16_bits_to_f64(bits) if dtype == "bf16" else f16_to_f64(bits)


def gemm(w, a_bits, a_dtype, c_dtype, G, packed=None):
    q = w["qweight"]
    N, K = q.shape[0], 2 * q.shape[1]
    M = a_bits.shape[0]
    if packed is None:
        fmt, packed, _ = pack_w4(w, G)
    else:
        fmt = lb.LOWBIT_W4_ASYM if w["zeros"] is not None else lb.LOWBIT_W4_SYM
    ad = {"bf16": lb.LOWBIT_BF16, "f16": lb.LOWBIT_F16}[a_dtype]
    cd = {"bf16": lb.LOWBIT_BF16, "f16": lb.LOWBIT_F16}[c_dtype]
    a = dev(np.ascontiguousarray(a_bits).view(np.int16))
    c = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMM, fmt, M, N, K, G)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_gemm(fmt, M, N, K, G, packed, a, ad, c, cd, ws, wsb))
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def _ref(w, a_bits, a_dtype, c_dtype, G, rows=None):
    if rows is None:
        _, yb = oracle.w4_matmul(a_bits, a_dtype, w["qweight"], w["scales"], w["zeros"], G, c_dtype)
    else:
        _, yb = oracle.w4_matmul_rows(a_bits, a_dtype, w["qweight"], w["scales"], w["zeros"], G, c_dtype, rows)
    return _to_f64(yb, c_dtype)


@pytest.mark.parametrize("a_dtype,c_dtype", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f16")])
@pytest.mark.parametrize("M,N,K,G,asym", [
    (1, 128, 128, 128, False),
    (7, 272, 256, 64, True),        # ragged N (17 strips), partial M tile
    (130, 256, 1056, 32, True),     # ragged M over two tiles, ragged last K tile
    (256, 384, 512, 128, False),
    (64, 256, 4096, 128, False),    # split-K path
    (200, 100, 2048, 32, False),    # ragged N inside one strip, split-K
    (130, 272, 384, 128, True),     # group of a whole K tile: three tiles, ragged M and N, zero points
    (33, 528, 256, 128, False),     # group of a whole K tile: two tiles, ragged M and N
])
def test_gemm_parity(M, N, K, G, asym, a_dtype, c_dtype):
    w = synth.w4_weights(N, K, G, asym=asym, workload_id=WL, layer=M, part=N)
    a = _acts(M, K, a_dtype)
    got = _to_f64(gemm(w, a, a_dtype, c_dtype, G), c_dtype)
    assert_close(got, _ref(w, a, a_dtype, c_dtype, G), "M=%d N=%d K=%d G=%d" % (M, N, K, G))


def test_gemm_zero_scales_contribute_nothing():
    M, N, K, G = 96, 160, 512, 32
    w = synth.w4_weights(N, K, G, asym=True, workload_id=WL, part=77)
    r = np.random.default_rng(8)
    s = w["scales"].copy()
    s[r.random(s.shape) < 0.2] = 0.0          # 20% of the groups have scale 0
    s[3, :] = 0.0                              # one output column entirely zero
    s[:, 0] = 0.0                              # the first group of every column
    w["scales"] = s
    a = _acts(M, K, "bf16", part=5)
    got = _to_f64(gemm(w, a, "bf16", "bf16", G), "bf16")
    ref = _ref(w, a, "bf16", "bf16", G)
    assert np.all(got[:, 3] == 0)
    assert_close(got, ref, "zero scales")


def test_gemm_matches_gemv_rows():
    """A single row through the GEMM equals the oracle like the GEMV does
    (cross-check of the two kernels' conventions)."""
    N, K, G = 512, 1024, 128
    w = synth.w4_weights(N, K, G, workload_id=WL, part=3)
    a = _acts(1, K, "f16", part=3)
    got = _to_f64(gemm(w, a, "f16", "f16", G), "f16")
    assert_close(got, _ref(w, a, "f16", "f16", G), "M=1")


def test_gemm_deterministic():
    M, N, K, G = 64, 256, 4096, 128           # split-K: fixed-order reduction
    w = synth.w4_weights(N, K, G, workload_id=WL, part=4)
    fmt, packed, _ = pack_w4(w, G)
    a = _acts(M, K, "bf16", part=4)
    c1 = gemm(w, a, "bf16", "bf16", G, packed)
    c2 = gemm(w, a, "bf16", "bf16", G, packed)
    assert np.array_equal(c1, c2)


@pytest.mark.parametrize("M", [512, 2048, 8192])
@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096)])
def test_gemm_prefill_shapes_sampled(M, K, N):
    """The prefill workload at full size (bf16 in/out, symmetric G=128);
    8 seeded rows x 256 seeded columns are checked against the oracle."""
    G = 128
    w = synth.w4_weights(N, K, G, workload_id=3, layer=0, part=N)
    a = synth.activations_bf16(M, K, workload_id=3, layer=M, part=K)
    c = gemm(w, a, "bf16", "bf16", G)
    r = np.random.default_rng(M + K)
    rows = np.sort(r.choice(M, size=8, replace=False))
    cols = np.sort(r.choice(N, size=256, replace=False))
    sub = dict(qweight=w["qweight"][cols], scales=w["scales"][cols], zeros=None)
    ref = _ref(sub, a, "bf16", "bf16", G, rows=rows)
    got = _to_f64(c[np.ix_(rows, cols)], "bf16")
    assert_close(got, ref, "prefill M=%d K=%d N=%d" % (M, K, N))


def test_gemm_argument_checks():
    w = synth.w4_weights(64, 256, 32, workload_id=WL, part=6)
    fmt, packed, _ = pack_w4(w, 32)
    a = dev(_acts(4, 256, "bf16").view(np.int16))
    c = torch.empty((4, 64), dtype=torch.int16, device="cuda")
    assert lb.lowbit_gemm(fmt, 4, 64, 256, 32, packed, a, 7, c, lb.LOWBIT_BF16) == lb.LOWBIT_E_UNSUPPORTED
    assert lb.lowbit_gemm(fmt, 4, 64, 256, 32, None, a, lb.LOWBIT_BF16, c, lb.LOWBIT_BF16) == lb.LOWBIT_E_INVALID_ARG
    assert lb.lowbit_gemm(fmt, 0, 64, 256, 32, None, None, lb.LOWBIT_BF16, None, lb.LOWBIT_BF16) == lb.LOWBIT_OK
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMM, fmt, 64, 256, 4096, 128)
    assert wsb > 0
    assert lb.lowbit_gemm(fmt, 64, 256, 4096, 128, packed, a, lb.LOWBIT_BF16, c, lb.LOWBIT_BF16, None, 0) \
        == lb.LOWBIT_E_WORKSPACE
