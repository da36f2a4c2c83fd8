"""Helpers for the GPU parity tests: device copies, packing through the C ABI,
and the comparison metrics (rel-L2 and max error over the oracle's rounded
output, in float64)."""
import numpy as np
import torch

import bit_weight_only_pack_amd as lb

RTOL_L2 = 1e-3      # matmul outputs: relative L2 error bound
RTOL_MAX = 1e-2     # matmul outputs: max |error| <= RTOL_MAX * max |reference|


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f16_to_f64(bits_or_f16):
    a = np.asarray(bits_or_f16)
    if a.dtype != np.float16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def bf16_bits_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def metrics(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / nref if nref > 0 else np.linalg.norm(y)
    mref = np.max(np.abs(ref)) if ref.size else 0.0
    mx = np.max(np.abs(y - ref)) / mref if mref > 0 else (np.max(np.abs(y)) if y.size else 0.0)
    return rel, mx


def assert_close(y, ref, what=""):
    rel, mx = metrics(y, ref)
    assert rel <= RTOL_L2 and mx <= RTOL_MAX, "%s rel-L2 %.3e max %.3e" % (what, rel, mx)
    return rel, mx


def pack_w4(w, group_size, E=1):
    """Pack canonical W4 arrays (numpy, leading E axis optional) through the C ABI."""
    q = w["qweight"]
    N, K = q.shape[-2], 2 * q.shape[-1]
    asym = w["zeros"] is not None
    fmt = lb.LOWBIT_W4_ASYM if asym else lb.LOWBIT_W4_SYM
    nbytes = lb.lowbit_packed_bytes(fmt, E, N, K, group_size)
    packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    codes = dev(q)
    scales = dev(w["scales"].view(np.uint16))
    zeros = dev(w["zeros"]) if asym else None
    lb.check(lb.lowbit_pack_weights(fmt, E, N, K, group_size, codes, scales, zeros, packed, nbytes))
    return fmt, packed, nbytes


def gemv(w, x, group_size, packed=None):
    """y = x @ W^T through lowbit_gemv; returns fp16 numpy [M][N]."""
    q = w["qweight"]
    N, K = q.shape[0], 2 * q.shape[1]
    M = x.shape[0]
    if packed is None:
        fmt, packed, _ = pack_w4(w, group_size)
    else:
        fmt = lb.LOWBIT_W4_ASYM if w["zeros"] is not None else lb.LOWBIT_W4_SYM
    xd = dev(x)
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    wsb = lb.lowbit_workspace_bytes(lb.LOWBIT_OP_GEMV, fmt, M, N, K, group_size)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    lb.check(lb.lowbit_gemv(fmt, M, N, K, group_size, packed, xd, y, ws, wsb))
    torch.cuda.synchronize()
    return y.cpu().numpy()
