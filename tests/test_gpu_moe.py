"""GPU parity of the 3-bit LUT-codebook MoE path against the CPU oracle:
LUT3 pack/unpack bit-exact, routing alignment bit-exact, grouped GEMM within
rel-L2 <= 1e-3 / max error <= 1e-2 * max |ref| of the oracle's bf16 output
(rows of non-local experts exactly zero)."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
import oracle
from bit_weight_only_pack_amd import synth
from gpu_util import assert_close, bf16_bits_to_f64, dev

pytestmark = pytest.mark.gpu
LUT3 = lb.LOWBIT_LUT3_E4M3


def pack_lut3(d):
    E, N, K = d["idx"].shape
    nb = lb.lowbit_packed_bytes(LUT3, E, N, K, 0)
    packed = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_pack_weights(LUT3, E, N, K, 0, dev(d["idx"]), dev(d["cb"]), dev(d["ex"]), packed, nb))
    return packed, nb


def align(topk, E, bm, emap=None):
    T, top_k = topk.shape
    cap = T * top_k + E * (bm - 1)
    sorted_ids = torch.full((max(cap, 1),), -5, dtype=torch.int32, device="cuda")
    offs = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")
    blk = torch.full((max(cap // bm, 1),), -5, dtype=torch.int32, device="cuda")
    npp = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    lb.check(lb.lowbit_moe_align(dev(topk), T, top_k, E, bm, None if emap is None else dev(emap),
                                 sorted_ids, offs, blk, npp))
    return sorted_ids, offs, blk, npp


@pytest.mark.parametrize("E,N,K", [(2, 16, 128), (3, 8, 64), (2, 40, 320), (1, 1536, 2048)])
def test_lut3_pack_roundtrip(E, N, K):
    d = synth.lut3_weights(E, N, K, workload_id=400, part=N)
    packed, nb = pack_lut3(d)
    idx = torch.zeros((E, N, K), dtype=torch.uint8, device="cuda")
    cb = torch.zeros((E, N // 8, K // 64, 8), dtype=torch.uint8, device="cuda")
    ex = torch.zeros((E, N // 8, K // 64), dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_unpack_weights(LUT3, E, N, K, 0, packed, nb, idx, cb, ex))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), d["idx"])
    assert np.array_equal(cb.cpu().numpy(), d["cb"])
    assert np.array_equal(ex.cpu().numpy(), d["ex"])


@pytest.mark.parametrize("T,E,top_k,bm,use_map", [
    (1, 8, 2, 16, False), (3, 4, 2, 16, True), (256, 128, 8, 16, False), (256, 128, 8, 32, True),
    (2048, 64, 8, 16, False), (7, 1024, 6, 16, False), (50, 1, 1, 48, False), (0, 16, 8, 16, False),
    (20, 4, 2, 4096, False), (5, 1024, 4, 4096, True),    # the largest block the align accepts
])
def test_moe_align_bitexact(T, E, top_k, bm, use_map):
    r = np.random.default_rng(T * 7 + E)
    topk = np.array([r.choice(E, size=top_k, replace=False) for _ in range(T)], dtype=np.int32).reshape(T, top_k)
    emap = None
    if use_map:
        emap = np.full(E, -1, np.int32)
        loc = np.sort(r.choice(E, size=max(1, E // 3), replace=False))
        emap[loc] = np.arange(loc.size, dtype=np.int32)
    ids, offs, blk, npp = align(topk, E, bm, emap)
    torch.cuda.synchronize()
    ref_ids, ref_blk, P = oracle.moe_align(topk, E, bm, emap)
    assert int(npp.item()) == P
    assert np.array_equal(ids.cpu().numpy()[:P], ref_ids)
    assert np.all(ids.cpu().numpy()[P:] == T * top_k)
    assert np.array_equal(blk.cpu().numpy()[:P // bm], ref_blk)
    assert np.all(blk.cpu().numpy()[P // bm:] == -1)        # blocks past the padded length: no expert
    o = offs.cpu().numpy()
    counts = np.bincount(topk.ravel(), minlength=E) if T else np.zeros(E, np.int64)
    assert o[0] == 0 and o[E] == P
    assert np.array_equal(np.diff(o), (counts + bm - 1) // bm * bm)


def run_moe(d, aq, as_, a_row_div, topk, E_global, emap=None, bm=16, d_local=None):
    d_pack = d if d_local is None else d_local
    El, N, K = d_pack["idx"].shape
    packed, _ = pack_lut3(d_pack)
    T, top_k = topk.shape
    ids, offs, blk, npp = align(topk, E_global, bm, emap)
    out = torch.full((T * top_k, N), 0x7FC0, dtype=torch.int16, device="cuda")   # NaN: every row must be written
    lb.check(lb.lowbit_moe_gemm(LUT3, El, N, K, packed, E_global, dev(aq), dev(as_), aq.shape[0], a_row_div,
                                ids, offs, blk, T * top_k, bm, out))
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def _ref(d_local, aq, as_, a_row_div, topk, emap):
    _, ob = oracle.moe_gemm(d_local["idx"], d_local["cb"], d_local["ex"], aq, as_, a_row_div, topk, emap)
    return ob


@pytest.mark.parametrize("T,E,top_k,N,K,gate_up", [
    (3, 4, 2, 8, 64, True),          # half a strip, half a K step
    (3, 4, 2, 24, 192, False),       # down style (a row per slot), ragged
    (16, 8, 2, 256, 256, True),
    (40, 4, 3, 64, 512, True),       # > 64 rows per expert: several passes
])
def test_moe_gemm_parity(T, E, top_k, N, K, gate_up):
    d = synth.lut3_weights(E, N, K, workload_id=410, part=N + K)
    topk = synth.moe_routing(T, E, top_k, workload_id=410, layer=T)
    rows = T if gate_up else T * top_k
    aq, as_ = synth.mxfp8_activations(rows, K, workload_id=410, part=K)
    div = top_k if gate_up else 1
    got = run_moe(d, aq, as_, div, topk, E)
    ref = _ref(d, aq, as_, div, topk, None)
    assert_close(bf16_bits_to_f64(got), bf16_bits_to_f64(ref), "moe T=%d E=%d N=%d K=%d" % (T, E, N, K))


def test_moe_gemm_expert_parallel_zero_rows():
    """Experts not local to this device (expert_map = -1) produce zero rows."""
    T, E, top_k, N, K = 24, 8, 2, 64, 256
    d = synth.lut3_weights(E, N, K, workload_id=411)
    topk = synth.moe_routing(T, E, top_k, workload_id=411)
    emap = np.array([0, -1, 1, -1, -1, 2, -1, 3], np.int32)
    local = [0, 2, 5, 7]
    d_local = dict(idx=d["idx"][local], cb=d["cb"][local], ex=d["ex"][local])
    aq, as_ = synth.mxfp8_activations(T, K, workload_id=411)
    got = run_moe(d, aq, as_, top_k, topk, E, emap=emap, d_local=d_local)
    ref = _ref(d_local, aq, as_, top_k, topk, emap)
    nonlocal_rows = emap[topk.ravel()] < 0
    assert np.all(got[nonlocal_rows] == 0)
    assert_close(bf16_bits_to_f64(got), bf16_bits_to_f64(ref), "EP")


def test_moe_gemm_worked_example():
    """The hand-worked codebook example: y = 2 * 0.25 - 6 * 2^-12 -> bf16 0.498046875."""
    E, N, K = 1, 8, 64
    cb = np.zeros((E, 1, 1, 8), np.uint8)
    cb[0, 0, 0] = [0x38, 0xB8, 0x40, 0x30, 0x00, 0x7E, 0x01, 0xC4]
    ex = np.full((E, 1, 1), 124, np.uint8)
    idx = np.full((E, N, K), 4, np.uint8)
    idx[0, 0, 0], idx[0, 0, 1] = 2, 6
    d = dict(idx=idx, cb=cb, ex=ex)
    aq = np.zeros((1, K), np.uint8)
    aq[0, 0], aq[0, 1] = 0x38, 0xC4
    as_ = np.array([[128, 127]], np.uint8)
    got = run_moe(d, aq, as_, 1, np.array([[0]], np.int32), 1)
    want = torch.tensor([0.498046875], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert got[0, 0] == want[0] and np.all(got[0, 1:] == 0)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_moe_gemm_full_workload_sampled(proj):
    """128 experts, top-8 over 256 tokens; gate/up K=2048 N=1536, down K=768
    N=2048.  The GPU computes every slot; the slots of 8 seeded tokens are
    checked against the oracle."""
    T, E, top_k = 256, 128, 8
    K, N = (2048, 1536) if proj == "gate_up" else (768, 2048)
    d = synth.lut3_weights(E, N, K, workload_id=4, part=0 if proj == "gate_up" else 1)
    topk = synth.moe_routing(T, E, top_k, workload_id=4)
    rows = T if proj == "gate_up" else T * top_k
    aq, as_ = synth.mxfp8_activations(rows, K, workload_id=4, part=0 if proj == "gate_up" else 1)
    div = top_k if proj == "gate_up" else 1
    got = run_moe(d, aq, as_, div, topk, E)
    toks = np.sort(np.random.default_rng(9).choice(T, size=8, replace=False))
    slots = (toks[:, None] * top_k + np.arange(top_k)[None, :]).ravel()
    if proj == "gate_up":
        ref = _ref(d, aq[toks], as_[toks], top_k, topk[toks], None)
    else:
        ref = _ref(d, aq[slots], as_[slots], 1, topk[toks], None)
    assert_close(bf16_bits_to_f64(got[slots]), bf16_bits_to_f64(ref), proj)


def test_moe_gemm_k_tail_reads_no_stale_lds():
    """K not a multiple of 128: the last K step's MFMAs also read the staged
    activation bytes past K (against zero weights).  Those bytes must be
    zeros written by the kernel, not whatever an earlier kernel left in LDS:
    a first launch stages activations that are all 0xFF (an E4M3 NaN) on
    every compute unit, then the K = 64 and K = 192 cases must still match
    the oracle and be finite."""
    T, E, top_k, N, K = 256, 128, 8, 256, 2048
    d = synth.lut3_weights(E, N, K, workload_id=412)
    topk = synth.moe_routing(T, E, top_k, workload_id=412)
    aq = np.full((T, K), 0xFF, np.uint8)
    as_ = np.full((T, K // 32), 127, np.uint8)
    run_moe(d, aq, as_, top_k, topk, E)                    # poisons LDS; its output is NaN by design
    for (T2, E2, k2, N2, K2, gate_up) in [(3, 4, 2, 8, 64, True), (3, 4, 2, 24, 192, False)]:
        d2 = synth.lut3_weights(E2, N2, K2, workload_id=410, part=N2 + K2)
        topk2 = synth.moe_routing(T2, E2, k2, workload_id=410, layer=T2)
        rows = T2 if gate_up else T2 * k2
        aq2, as2 = synth.mxfp8_activations(rows, K2, workload_id=410, part=K2)
        div = k2 if gate_up else 1
        got = run_moe(d2, aq2, as2, div, topk2, E2)
        ref = _ref(d2, aq2, as2, div, topk2, None)
        assert_close(bf16_bits_to_f64(got), bf16_bits_to_f64(ref), "after stale LDS, K=%d" % K2)
