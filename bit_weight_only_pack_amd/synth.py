"""Seeded synthetic inputs for the low-bit matmul workloads.

This module only draws random numbers and converts them to the storage types
with library conversions (numpy float16, torch bfloat16 / float8).  It holds
none of the arithmetic the library computes: no dequantization, no products,
no packing.  One generator, ``mxfp8_activations``, builds ready-made MXFP8
inputs for the grouped GEMM with its own numpy block-scale rule (an input
recipe only: the library's MXFP8 quantizer is never compared with it, and
the oracle consumes whatever bytes it returns).
Both the GPU tests and the CPU oracle consume the arrays it returns.

Every tensor has its own generator, ``default_rng(SeedSequence([20261203,
workload_id, tensor_id, layer, part]))``, so a tensor's values do not depend on
which other tensors were drawn or in what order.  Floats are drawn in float64.

Workload shapes stand in for the pages' decoder (an 8B dense model at batch 1,
"Low Bit Metal Kernels" and "Low Bit ARM kernels") and for a 30B-A3B-class MoE
layer ("vLLM PR #62759 analysis", 3-bit LUT-B experts with MXFP8
activations).  No dataset or trained weight is used.
"""
import numpy as np

SEED_BASE = 20261203

# tensor ids inside one workload
T_CODES, T_SCALES, T_ZEROS, T_X, T_OUTLIERS, T_ROUTER, T_LUT_IDX, T_LUT_CB, T_LUT_EXP, T_ACT = range(10)

# Llama-3-8B-shaped decoder projections, (name, K, N): K = reduction, N = outputs
LLAMA3_8B_PROJS = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 14336),
    ("up", 4096, 14336),
    ("down", 14336, 4096),
)
LLAMA3_8B_LAYERS = 32


def rng(workload_id, tensor_id, layer=0, part=0):
    return np.random.default_rng(np.random.SeedSequence([SEED_BASE, workload_id, tensor_id, layer, part]))


def w4_weights(N, K, group_size, *, asym=False, scale_range=(0.002, 0.01), zero_range=(0, 15),
               workload_id=0, layer=0, part=0):
    """INT4 codes (uniform 0..15, two per byte, low nibble first), fp16 scales
    uniform in scale_range, and for asym an int8 zero point per group uniform
    in zero_range (inclusive).

    Returns dict(qweight=u8 [N][K/2], scales=f16 [N][K/G], zeros=i8 [N][K/G] or None).
    Uniform bytes are uniform independent nibble pairs.
    """
    assert K % 2 == 0 and K % group_size == 0
    qweight = rng(workload_id, T_CODES, layer, part).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    lo, hi = scale_range
    scales = rng(workload_id, T_SCALES, layer, part).uniform(lo, hi, size=(N, K // group_size)).astype(np.float16)
    zeros = None
    if asym:
        zlo, zhi = zero_range
        zeros = rng(workload_id, T_ZEROS, layer, part).integers(zlo, zhi + 1, size=(N, K // group_size),
                                                                dtype=np.int64).astype(np.int8)
    return dict(qweight=qweight, scales=scales, zeros=zeros)


def wb_weights(N, K, group_size, bits, *, asym=False, scale_range=(0.002, 0.01), workload_id=0, layer=0, part=0):
    """Uniform b-bit weights (b = 1..8): codes u8 [N][K] uniform in [0, 2^b)
    (one per byte), scales fp16 [N][K/G] uniform in scale_range, zeros int8
    [N][K/G] uniform in [0, 2^b) clipped to 127 (asymmetric) or None."""
    codes = rng(workload_id, T_CODES, layer, part).integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    lo, hi = scale_range
    scales = rng(workload_id, T_SCALES, layer, part).uniform(lo, hi, size=(N, K // group_size)).astype(np.float16)
    zeros = None
    if asym:
        zeros = np.minimum(rng(workload_id, T_ZEROS, layer, part).integers(0, 1 << bits, size=(N, K // group_size)),
                           127).astype(np.int8)
    return dict(codes=codes, scales=scales, zeros=zeros)


def outlier_channels(K, frac=0.01, workload_id=0, layer=0, part=0):
    """round(frac*K) distinct channel indices chosen by seed (sorted)."""
    n = int(round(frac * K))
    ch = rng(workload_id, T_OUTLIERS, layer, part).choice(K, size=n, replace=False)
    return np.sort(ch)


def activations_f16(M, K, *, outlier_frac=0.0, outlier_scale=20.0, workload_id=0, layer=0, part=0):
    """fp16 [M][K] ~ N(0,1); with outlier_frac > 0 a fixed set of channels (the
    same for every row) is multiplied by outlier_scale before the cast."""
    x = rng(workload_id, T_X, layer, part).standard_normal((M, K))
    if outlier_frac > 0:
        ch = outlier_channels(K, outlier_frac, workload_id, layer, part)
        x[:, ch] *= outlier_scale
    return x.astype(np.float16)


def _to_bf16_bits(x64):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations_bf16(M, K, *, workload_id=0, layer=0, part=0):
    """bf16 [M][K] ~ N(0,1), returned as uint16 bit patterns (float64 draw ->
    float32 -> RNE bf16)."""
    x = rng(workload_id, T_X, layer, part).standard_normal((M, K))
    return _to_bf16_bits(x)


def _to_e4m3_bytes(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def moe_routing(T, E, top_k, *, workload_id=0, layer=0):
    """Router logits N(0,1) fp32 [T][E]; softmax preserves order, so the top-k
    experts by probability are the top-k logits, descending, lower expert id
    first on ties.  Returns int32 [T][top_k]."""
    logits = rng(workload_id, T_ROUTER, layer).standard_normal((T, E)).astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :top_k].astype(np.int32))


def moe_topk_weights(T, E, top_k, *, workload_id=0, layer=0):
    """Router weights of the experts moe_routing picks (same logits): softmax
    probabilities in float64, the chosen top_k renormalized to sum 1, cast to
    float32.  Returns float32 [T][top_k] in the order of moe_routing's ids."""
    logits = rng(workload_id, T_ROUTER, layer).standard_normal((T, E)).astype(np.float32).astype(np.float64)
    order = np.argsort(-logits.astype(np.float32), axis=1, kind="stable")[:, :top_k]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pk = np.take_along_axis(p, order, axis=1)
    return np.ascontiguousarray((pk / pk.sum(axis=1, keepdims=True)).astype(np.float32))


def lut3_weights(E, N, K, *, exp_range=(120, 124), workload_id=0, layer=0, part=0):
    """3-bit LUT-codebook experts.
    idx u8 [E][N][K] uniform 0..7; codebook u8 (E4M3 bytes) [E][N/8][K/64][8]
    from N(0,1) clipped to +-448 and converted RNE; tile exponent u8 (UE8M0)
    [E][N/8][K/64] uniform in exp_range (inclusive)."""
    assert N % 8 == 0 and K % 64 == 0
    idx = rng(workload_id, T_LUT_IDX, layer, part).integers(0, 8, size=(E, N, K), dtype=np.uint8)
    cbv = rng(workload_id, T_LUT_CB, layer, part).standard_normal((E, N // 8, K // 64, 8))
    cb = _to_e4m3_bytes(np.clip(cbv, -448.0, 448.0))
    lo, hi = exp_range
    ex = rng(workload_id, T_LUT_EXP, layer, part).integers(lo, hi + 1, size=(E, N // 8, K // 64),
                                                          dtype=np.int64).astype(np.uint8)
    return dict(idx=idx, cb=cb, ex=ex)


def mxfp8_activations(R, K, *, workload_id=0, layer=0, part=0):
    """MXFP8 activations for R rows: draw N(0,1), then per (row, 32-K block)
    take the scale exponent 127 + floor(log2(amax)) - 8 (8 = exponent of the
    largest E4M3 value) and store elements x / 2^(that - 127) clipped to +-448,
    RNE to E4M3.  An all-zero block gets exponent 127.
    Returns (aq u8 [R][K], as u8 [R][K/32])."""
    assert K % 32 == 0
    x = rng(workload_id, T_ACT, layer, part).standard_normal((R, K))
    blocks = x.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, p = np.frexp(amax)                       # amax = m * 2^p, m in [0.5, 1)
    e = np.where(amax > 0, p - 1 - 8, 0)        # floor(log2 amax) - 8
    scaled = blocks / np.ldexp(1.0, e)[:, :, None]
    aq = _to_e4m3_bytes(np.clip(scaled, -448.0, 448.0)).reshape(R, K)
    as_ = (e + 127).astype(np.uint8)
    return aq, as_
