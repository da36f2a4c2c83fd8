"""Host-side checks of the C ABI (CPU only, no GPU needed):
the library loads, exports every entry point include/lowbit.h declares, the
Python binding covers the same set, and invalid arguments come back as status
codes before anything is enqueued (no HIP call is made on these paths)."""
import ctypes
import os
import re

import pytest

import bit_weight_only_pack_amd as lb
from bit_weight_only_pack_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            with open(os.path.join(ROOT, "include", fn)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(lowbit_\w+)\s*\(", text))
    return names


def test_header_declares_the_hot_path_entry_points():
    d = _declared()
    for name in ("lowbit_pack_weights", "lowbit_gemv"):
        assert name in d


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in sorted(_declared()) if not hasattr(handle, n)]
    assert not missing, missing


def test_binding_matches_header():
    assert set(_lib.SIGNATURES) == _declared()
    for name in _declared():
        assert callable(getattr(lb, name))


def test_strerror_and_version():
    assert lb.lowbit_version() >= 1
    for code in range(5):
        assert isinstance(lb.lowbit_strerror(code), str) and lb.lowbit_strerror(code)
    assert lb.lowbit_strerror(99) == "unknown status"


def test_packed_bytes_closed_form():
    # 16-row x 128-K tiles of 1 KiB + 16 x (128/G) fp16 scales (+ int8 zeros), sections 256-aligned
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 1, 256, 256, 32) == 32 * 1024 + 32 * 16 * 4 * 2
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_ASYM, 1, 256, 256, 32) == 32 * 1024 + 32 * 16 * 4 * 3
    n, k = 4096, 14336
    tiles = (n // 16) * (k // 128)
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 1, n, k, 128) == tiles * 1024 + tiles * 32
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 3, n, k, 128) == 3 * (tiles * 1024 + tiles * 32)
    # ragged shapes round up to whole tiles
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 1, 17, 96, 32) == 2 * 1024 + 256
    # invalid -> 0
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 1, 16, 100, 32) == 0
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, 1, 16, 96, 48) == 0
    assert lb.lowbit_packed_bytes(lb.LOWBIT_W4_SYM, -1, 16, 128, 32) == 0


SYM, ASYM = lb.LOWBIT_W4_SYM, lb.LOWBIT_W4_ASYM
E_ARG, E_UNS, E_WS = lb.LOWBIT_E_INVALID_ARG, lb.LOWBIT_E_UNSUPPORTED, lb.LOWBIT_E_WORKSPACE
FAKE = 1 << 20  # a non-null address that must never be dereferenced on these paths


@pytest.mark.parametrize("args,want", [
    ((SYM, 1, 256, 250, 32), E_ARG),          # K % G
    ((SYM, 1, 256, 256, 48), E_ARG),          # K % G (48 does not divide 256)
    ((SYM, 1, 256, 192, 96), E_UNS),          # group size not in {32, 64, 128}
    ((SYM, 17, 256, 256, 32), E_UNS),         # M above the GEMV limit
    ((SYM, -1, 256, 256, 32), E_ARG),
    ((SYM, 1, -5, 256, 32), E_ARG),
    ((7, 1, 256, 256, 32), E_UNS),            # unknown format
    ((lb.LOWBIT_LUT3_E4M3, 1, 256, 256, 32), E_UNS),
])
def test_gemv_rejects_bad_shapes(args, want):
    assert lb.lowbit_gemv(*args, FAKE, FAKE, FAKE, None, 0) == want


def test_gemv_null_and_alignment():
    assert lb.lowbit_gemv(SYM, 1, 256, 256, 32, None, FAKE, FAKE, None, 0) == E_ARG
    assert lb.lowbit_gemv(SYM, 1, 256, 256, 32, FAKE, None, FAKE, None, 0) == E_ARG
    assert lb.lowbit_gemv(SYM, 1, 256, 256, 32, FAKE, FAKE, None, None, 0) == E_ARG
    assert lb.lowbit_gemv(SYM, 1, 256, 256, 32, FAKE, FAKE + 2, FAKE, None, 0) == E_ARG   # x not 16-B aligned


def test_empty_calls_are_ok_without_touching_memory():
    assert lb.lowbit_gemv(SYM, 0, 256, 256, 32, None, None, None, None, 0) == lb.LOWBIT_OK
    assert lb.lowbit_gemv(SYM, 4, 0, 256, 32, None, None, None, None, 0) == lb.LOWBIT_OK


def test_pack_argument_checks():
    nb = lb.lowbit_packed_bytes(SYM, 1, 64, 256, 32)
    assert lb.lowbit_pack_weights(SYM, 1, 64, 256, 32, FAKE, FAKE, None, FAKE, nb - 1) == E_WS
    assert lb.lowbit_pack_weights(SYM, 1, 64, 256, 32, FAKE, FAKE, FAKE, FAKE, nb) == E_ARG     # zeros with SYM
    nba = lb.lowbit_packed_bytes(ASYM, 1, 64, 256, 32)
    assert lb.lowbit_pack_weights(ASYM, 1, 64, 256, 32, FAKE, FAKE, None, FAKE, nba) == E_ARG   # ASYM needs zeros
    assert lb.lowbit_pack_weights(SYM, 1, 64, 256, 32, None, FAKE, None, FAKE, nb) == E_ARG
    assert lb.lowbit_pack_weights(SYM, 1, 64, 256, 32, FAKE, FAKE, None, None, nb) == E_ARG
    assert lb.lowbit_pack_weights(SYM, -2, 64, 256, 32, FAKE, FAKE, None, FAKE, nb) == E_ARG
    assert lb.lowbit_unpack_weights(SYM, 1, 64, 256, 32, FAKE, nb - 1, FAKE, FAKE, None) == E_WS
    assert lb.lowbit_dequant(SYM, 64, 256, 32, FAKE, nb - 1, FAKE) == E_WS
    assert lb.lowbit_dequant(SYM, 64, 256, 32, None, nb, FAKE) == E_ARG


def test_workspace_query():
    assert lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV, SYM, 1, 4096, 4096, 128) >= 0
    assert lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV, SYM, 1, 4096, 4000, 128) == 0


def test_last_hip_error_starts_clear():
    assert lb.lowbit_last_hip_error() == 0


def test_lut3_packed_bytes_closed_form():
    """3-bit indices + one 8-entry E4M3 codebook and one UE8M0 exponent per
    8 x 64 tile = 3 + 72/512 = 3.140625 bits per weight; the packed blob holds
    exactly that (plus 256-byte section alignment)."""
    E, N, K = 128, 1536, 2048
    nb = lb.lowbit_packed_bytes(lb.LOWBIT_LUT3_E4M3, E, N, K, 0)
    weights = E * N * K
    assert abs(nb * 8 / weights - 3.140625) < 1e-6
    # a 128 x 128 tile: 128*128*3/8 = 6144 index bytes, 512 codebook bytes, 32 exponent bytes
    assert lb.lowbit_packed_bytes(lb.LOWBIT_LUT3_E4M3, 1, 128, 128, 0) == 6144 + 256 + 256  # sections 256-aligned
    assert lb.lowbit_packed_bytes(lb.LOWBIT_LUT3_E4M3, 1, 12, 128, 0) == 0      # N % 8
    assert lb.lowbit_packed_bytes(lb.LOWBIT_LUT3_E4M3, 1, 16, 96, 0) == 0       # K % 64


def test_moe_argument_checks():
    L = lb.LOWBIT_LUT3_E4M3
    assert lb.lowbit_moe_align(FAKE, 4, 2, 0, 16, None, FAKE, FAKE, FAKE, FAKE) == E_ARG
    assert lb.lowbit_moe_align(FAKE, 4, 2, 2048, 16, None, FAKE, FAKE, FAKE, FAKE) == E_UNS
    assert lb.lowbit_moe_align(FAKE, 4, 2, 8, 16, None, None, FAKE, FAKE, FAKE) == E_ARG
    assert lb.lowbit_moe_gemm(SYM, 8, 64, 128, FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, 8, 16, FAKE) == E_UNS
    assert lb.lowbit_moe_gemm(L, 8, 60, 128, FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, 8, 16, FAKE) == E_ARG
    assert lb.lowbit_moe_gemm(L, 8, 64, 128, FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, 8, 24, FAKE) == E_UNS
    # slot 8 with a_row_div 2 reads row 4 of a 4-row activation matrix
    assert lb.lowbit_moe_gemm(L, 8, 64, 128, FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, 9, 16, FAKE) == E_ARG
    assert lb.lowbit_moe_gemm(L, 8, 64, 128, FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, 0, 16, FAKE) == lb.LOWBIT_OK


def test_gemv_batched_argument_checks():
    probs = lb.make_gemv_problems([(FAKE, FAKE, FAKE, 64, 256)] * 9)
    assert lb.lowbit_gemv_batched(SYM, 1, 32, 9, probs) == E_UNS          # more than 8 problems
    assert lb.lowbit_gemv_batched(SYM, 1, 32, 0, probs) == lb.LOWBIT_OK
    assert lb.lowbit_gemv_batched(SYM, 1, 32, -1, probs) == E_ARG
    bad = lb.make_gemv_problems([(FAKE, FAKE, FAKE, 64, 256), (FAKE, FAKE, FAKE, 64, 250)])
    assert lb.lowbit_gemv_batched(SYM, 1, 32, 2, bad) == E_ARG              # K % G in the second problem
    nul = lb.make_gemv_problems([(FAKE, FAKE, None, 64, 256)])
    assert lb.lowbit_gemv_batched(SYM, 1, 32, 1, nul) == E_ARG
    assert lb.lowbit_gemv_batched(SYM, 17, 32, 1, probs) == E_UNS


def test_w4a8_argument_checks_and_workspace_plan():
    """W4A8: shape limits, the workspace rule (none when the launch quantizes
    the activations itself) and the activation-quantization checks, all
    decided on the host before anything is enqueued."""
    OP = lb.LOWBIT_OP_GEMV_W4A8
    assert lb.lowbit_workspace_bytes(OP, ASYM, 1, 14336, 4096, 32) == 0       # M=1: fused for every K
    assert lb.lowbit_workspace_bytes(OP, ASYM, 1, 4096, 14336, 32) == 0
    assert lb.lowbit_workspace_bytes(OP, SYM, 2, 4096, 4096, 128) > 0         # from M = 2: quantized once, into the workspace
    ws8 = lb.lowbit_workspace_bytes(OP, ASYM, 8, 4096, 14336, 32)
    # codes (M*K bytes) + code sums (K/G groups x 8 slots x 4 bytes) + scales, whole KiB
    assert ws8 == -(-(8 * 14336 + (14336 // 32) * 8 * 4 + 64) // 1024) * 1024
    assert lb.lowbit_gemv_w4a8(ASYM, 8, 4096, 14336, 32, FAKE, FAKE, FAKE, None, 0) == E_WS
    assert lb.lowbit_gemv_w4a8(ASYM, 8, 4096, 14336, 32, FAKE, FAKE, FAKE, FAKE, ws8 - 1) == E_WS
    assert lb.lowbit_gemv_w4a8(SYM, 1, 64, 16384 + 128, 128, FAKE, FAKE, FAKE, None, 0) == E_UNS   # K > 16384
    assert lb.lowbit_gemv_w4a8(SYM, 17, 64, 256, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS
    assert lb.lowbit_gemv_w4a8(SYM, 1, 64, 250, 32, FAKE, FAKE, FAKE, None, 0) == E_ARG
    assert lb.lowbit_gemv_w4a8(SYM, 1, 64, 256, 32, FAKE, FAKE + 2, FAKE, None, 0) == E_ARG
    assert lb.lowbit_gemv_w4a8(SYM, 0, 64, 256, 32, None, None, None, None, 0) == lb.LOWBIT_OK
    assert lb.lowbit_quant_act_i8(2, 12, FAKE, FAKE, FAKE) == E_ARG          # K % 8
    assert lb.lowbit_quant_act_i8(2, 16, FAKE + 4, FAKE, FAKE) == E_ARG      # x alignment
    assert lb.lowbit_quant_act_i8(2, 16, FAKE, FAKE, None) == E_ARG
    assert lb.lowbit_quant_act_i8(0, 16, None, None, None) == lb.LOWBIT_OK
    probs = lb.make_gemv_problems([(FAKE, FAKE, FAKE, 4096, 4096)] * 3)
    assert lb.lowbit_gemv_w4a8_batched_workspace_bytes(SYM, 1, 128, 3, probs) == 0
    wsb = lb.lowbit_gemv_w4a8_batched_workspace_bytes(SYM, 8, 32, 3, probs)
    assert wsb == 3 * lb.lowbit_workspace_bytes(OP, SYM, 8, 4096, 4096, 32) > 0
    assert lb.lowbit_gemv_w4a8_batched(SYM, 8, 32, 3, probs, FAKE, wsb - 1) == E_WS
    assert lb.lowbit_gemv_w4a8_batched(SYM, 1, 32, 9, probs, None, 0) == E_UNS


def test_moe_layer_argument_checks():
    """The MoE layer entry points validate on the host: block sizes of the
    MXFP8 rows (K % 32), the layer's K multiples of 64, workspace size and
    alignment, null pointers; empty calls return OK without touching memory."""
    assert lb.lowbit_mxfp8_quant(FAKE, 4, 48, FAKE, FAKE) == E_ARG                # K % 32
    assert lb.lowbit_mxfp8_quant(FAKE + 8, 4, 64, FAKE, FAKE) == E_ARG            # x alignment
    assert lb.lowbit_mxfp8_quant(None, 0, 64, None, None) == lb.LOWBIT_OK
    assert lb.lowbit_moe_silu_mul_quant(FAKE, 4, 40, FAKE, FAKE) == E_ARG         # I % 32
    assert lb.lowbit_moe_silu_mul_quant(FAKE, 4, 64, None, FAKE) == E_ARG
    L3 = lb.LOWBIT_LUT3_E4M3
    fused = lambda fmt, I, K, bm, q: lb.lowbit_moe_gemm_silu_quant(fmt, 4, I, K, FAKE, 4, FAKE, FAKE, 8, 2, FAKE,
                                                                   FAKE, FAKE, 16, bm, q, FAKE)
    assert fused(lb.LOWBIT_W4_SYM, 128, 256, 16, FAKE) == E_UNS
    assert fused(L3, 192, 256, 16, FAKE) == E_UNS                                  # I % 128
    assert fused(L3, 128, 4928, 16, FAKE) == E_UNS                                 # K past the staging area
    assert fused(L3, 128, 256, 24, FAKE) == E_UNS                                  # block_m % 16
    assert fused(L3, 128, 250, 16, FAKE) == E_ARG                                  # K % 64
    assert fused(L3, 128, 256, 16, None) == E_ARG
    assert lb.lowbit_moe_gemm_silu_quant(L3, 4, 128, 256, None, 4, None, None, 0, 2, None, None, None, 0, 16, None,
                                         None) == lb.LOWBIT_OK
    assert lb.lowbit_moe_combine(FAKE, FAKE, 4, 2, 60, FAKE) == E_ARG             # H % 8
    assert lb.lowbit_moe_combine(None, None, 0, 2, 64, None) == lb.LOWBIT_OK
    wsb = lb.lowbit_moe_layer_workspace_bytes(256, 8, 128, 2048, 768, 16)
    slots = 256 * 8
    assert wsb >= slots * (2 * 768 * 2 + 768 + 768 // 32 + 2048 * 2) + 256 * (2048 + 2048 // 32)
    assert lb.lowbit_moe_layer_workspace_bytes(256, 8, 128, 2000, 768, 16) == 0   # H % 64
    assert lb.lowbit_moe_layer_workspace_bytes(256, 8, 128, 2048, 768, 24) == 0   # block_m % 16
    args = (FAKE, FAKE, 128, 128, 2048, 768, FAKE, FAKE, FAKE, 256, 8, None, 16, FAKE)
    assert lb.lowbit_moe_layer(*args, FAKE, wsb - 1) == E_WS
    assert lb.lowbit_moe_layer(*args, FAKE + 128, wsb) == E_ARG                   # workspace alignment
    assert lb.lowbit_moe_layer(FAKE, FAKE, 128, 128, 2048, 736, FAKE, FAKE, FAKE, 256, 8, None, 16, FAKE,
                               FAKE, wsb) == E_ARG                                  # I % 64
    assert lb.lowbit_moe_layer(FAKE, FAKE, 64, 128, 2048, 768, FAKE, FAKE, FAKE, 256, 8, None, 16, FAKE,
                               FAKE, wsb) == E_ARG                                  # no map, E > E_local


def test_uint_formats_host_rules():
    """b-bit formats: packed size = tiles x 256 x bits + sections; invalid
    widths and shapes rejected before any launch."""
    for bits in range(1, 9):
        tiles = (64 // 16) * (512 // 128)
        assert lb.lowbit_packed_bytes(lb.LOWBIT_UINT(bits), 1, 64, 512, 128) == \
            -(-tiles * 256 * bits // 256) * 256 + tiles * 16 * 2
    assert lb.lowbit_packed_bytes(lb.LOWBIT_UINT(4), 1, 64, 512, 128) == lb.lowbit_packed_bytes(SYM, 1, 64, 512, 128)
    assert lb.lowbit_packed_bytes(lb.LOWBIT_UINT(9), 1, 64, 512, 128) == 0
    assert lb.lowbit_packed_bytes(lb.LOWBIT_UINT(3), 1, 64, 500, 128) == 0
    f3 = lb.LOWBIT_UINT(3, True)
    nb = lb.lowbit_packed_bytes(f3, 1, 64, 512, 32)
    assert lb.lowbit_pack_weights(f3, 1, 64, 512, 32, FAKE, FAKE, None, FAKE, nb) == E_ARG    # asym needs zeros
    assert lb.lowbit_gemv(f3, 17, 64, 512, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS
    assert lb.lowbit_gemv(f3, 16, 64, 16384, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS            # x over the LDS budget
    assert lb.lowbit_gemv(f3, 5, 64, 16384, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS             # 160 KiB of x + partial sums
    assert lb.lowbit_gemv(f3, 1, 64, 16384 + 128, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS       # > 8 tiles per wave
    assert lb.lowbit_gemm(f3, 64, 64, 512, 32, FAKE, FAKE, lb.LOWBIT_BF16, FAKE, lb.LOWBIT_BF16, None, 0) == E_UNS
    assert lb.lowbit_gemv_w4a8(f3, 1, 64, 512, 32, FAKE, FAKE, FAKE, None, 0) == E_UNS


def test_32bit_offset_limits_rejected_on_the_host():
    """The GEMV and GEMM kernels address operands through 32-bit buffer
    offsets with 2^31 as the out-of-range marker, so a region one descriptor
    spans must stay below 2^31 bytes; larger shapes are refused before any
    launch instead of wrapping."""
    BF = lb.LOWBIT_BF16
    # packed blob of 2^31 bytes or more (N = K = 65536: 2 GiB of codes)
    assert lb.lowbit_gemm(SYM, 16, 65536, 65536, 128, FAKE, FAKE, BF, FAKE, BF, FAKE, 1 << 40) == E_UNS
    # activation rows of 2^31 bytes (M * K * 2)
    assert lb.lowbit_gemm(SYM, 1 << 16, 256, 1 << 14, 128, FAKE, FAKE, BF, FAKE, BF, FAKE, 1 << 40) == E_UNS
    # GEMV: M * K * 2 and one strip of codes (16 rows x K bytes at 8 bits)
    assert lb.lowbit_gemv(SYM, 16, 256, 1 << 26, 128, FAKE, FAKE, FAKE, None, 0) == E_UNS
    assert lb.lowbit_gemv(lb.LOWBIT_UINT(8), 1, 256, 1 << 27, 128, FAKE, FAKE, FAKE, None, 0) == E_UNS
    p = lb.make_gemv_problems([(FAKE, FAKE, FAKE, 256, 1 << 26)])
    assert lb.lowbit_gemv_batched(SYM, 16, 128, 1, p) == E_UNS
    assert lb.lowbit_gemv_w4a8(ASYM, 16, 256, 1 << 26, 32, FAKE, FAKE, FAKE, FAKE, 1 << 40) == E_UNS


def test_hbm_read_argument_checks():
    """The read-ceiling helper rejects ragged sizes and null or misaligned
    pointers before enqueueing anything; an empty read enqueues nothing."""
    assert lb.lowbit_hbm_read(FAKE, 0, FAKE) == lb.LOWBIT_OK
    assert lb.lowbit_hbm_read(None, 0, None) == lb.LOWBIT_OK
    assert lb.lowbit_hbm_read(FAKE, 24, FAKE) == E_ARG          # not a multiple of 16
    assert lb.lowbit_hbm_read(FAKE, -16, FAKE) == E_ARG
    assert lb.lowbit_hbm_read(None, 16, FAKE) == E_ARG
    assert lb.lowbit_hbm_read(FAKE, 16, None) == E_ARG
    assert lb.lowbit_hbm_read(FAKE + 8, 16, FAKE) == E_ARG       # buffer not 16-byte aligned
    assert lb.lowbit_hbm_read(FAKE, 16, FAKE + 2) == E_ARG       # sink not 4-byte aligned
