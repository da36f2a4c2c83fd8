"""ctypes binding of liblowbit.so: one Python function per C entry point, same
name, same argument order.  Marshalling only -- every step of the computation
runs in the library's HIP kernels.

Pointer arguments accept a torch tensor (its ``data_ptr()``), a raw integer
address, or None (NULL).  ``stream=None`` means torch's current stream on the
current device.  Functions return the library's int status code unchanged;
``check(status)`` raises LowbitError for a non-zero one.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblowbit.so")

LOWBIT_OK = 0
LOWBIT_E_INVALID_ARG = 1
LOWBIT_E_UNSUPPORTED = 2
LOWBIT_E_WORKSPACE = 3
LOWBIT_E_HIP = 4

LOWBIT_W4_SYM = 0
LOWBIT_W4_ASYM = 1
LOWBIT_LUT3_E4M3 = 2



def LOWBIT_UINT(bits, asym=False):
    """Format id of uniform b-bit codes (the C macro of the same name)."""
    return 16 + 2 * bits + (1 if asym else 0)


LOWBIT_F16 = 0
LOWBIT_BF16 = 1

LOWBIT_OP_GEMV = 0
LOWBIT_OP_GEMM = 1
LOWBIT_OP_GEMV_W4A8 = 2

LOWBIT_HBM_READ_SINK_WORDS = 1024   # sink words of lowbit_hbm_read (include/lowbit.h)
_lib = None

_vp = ctypes.c_void_p


class lowbit_gemv_problem(ctypes.Structure):
    """Mirror of the C struct of the same name in include/lowbit.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]

class lowbit_gemv_chain(ctypes.Structure):
    """Mirror of the C struct of the same name in include/lowbit.h."""
    _fields_ = [("fmt", ctypes.c_int), ("M", ctypes.c_int), ("group_size", ctypes.c_int), ("count", ctypes.c_int),
                ("stages", ctypes.c_int), ("grid", ctypes.c_int), ("xrow", ctypes.c_int),
                ("spin_limit", ctypes.c_uint), ("buf", ctypes.c_void_p), ("buf_bytes", ctypes.c_size_t)]


_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/lowbit.h
SIGNATURES = {
    "lowbit_strerror": (ctypes.c_char_p, [_i]),
    "lowbit_last_hip_error": (_i, []),
    "lowbit_version": (_i, []),
    "lowbit_packed_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "lowbit_pack_weights": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lowbit_unpack_weights": (_i, [_i, _i, _i, _i, _i, _vp, _sz, _vp, _vp, _vp, _vp]),
    "lowbit_dequant": (_i, [_i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "lowbit_hbm_read": (_i, [_vp, ctypes.c_int64, _vp, _vp]),
    "lowbit_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "lowbit_gemv": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lowbit_gemv_batched": (_i, [_i, _i, _i, _i, _vp, _vp]),
    "lowbit_quant_act_i8": (_i, [_i, _i, _vp, _vp, _vp, _vp]),
    "lowbit_gemv_w4a8": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lowbit_gemv_w4a8_batched_workspace_bytes": (_sz, [_i, _i, _i, _i, _vp]),
    "lowbit_gemv_w4a8_batched": (_i, [_i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "lowbit_gemv_w4a8_batched_noalloc": (_i, [_i, _i, _i, _i, _vp, _vp]),
    "lowbit_gemv_chain_bytes": (_sz, [_i, _i]),
    "lowbit_gemv_chain_init": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, ctypes.c_uint, _vp, _sz, _vp]),
    "lowbit_gemv_chain_run": (_i, [_vp, _vp]),
    "lowbit_gemv_chain_error": (_i, [_vp, _vp, _vp]),
    "lowbit_gemm": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _sz, _vp]),
    "lowbit_moe_align": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "lowbit_moe_gemm": (_i, [_i, _i, _i, _i, _vp, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "lowbit_mxfp8_quant": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "lowbit_moe_silu_mul_quant": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "lowbit_moe_gemm_silu_quant": (_i, [_i, _i, _i, _i, _vp, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                        _vp]),
    "lowbit_moe_combine": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    "lowbit_moe_layer_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "lowbit_moe_layer": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _vp, _vp, _sz, _vp]),
}


class LowbitError(RuntimeError):
    def __init__(self, status):
        msg = lib().lowbit_strerror(status).decode()
        if status == LOWBIT_E_HIP:
            msg += " (hipError %d)" % lib().lowbit_last_hip_error()
        super().__init__("lowbit status %d: %s" % (status, msg))
        self.status = status


def lib():
    """Load liblowbit.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblowbit.so is not built (%s); run python -m bit_weight_only_pack_amd.build"
                               % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status):
    if status != LOWBIT_OK:
        raise LowbitError(status)
    return status


def _ptr(p):
    if p is None:
        return None
    if isinstance(p, int):
        return p
    return p.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def lowbit_strerror(status):
    return lib().lowbit_strerror(status).decode()


def lowbit_last_hip_error():
    return lib().lowbit_last_hip_error()


def lowbit_version():
    return lib().lowbit_version()


def lowbit_packed_bytes(fmt, E, N, K, group_size):
    return lib().lowbit_packed_bytes(fmt, E, N, K, group_size)


def lowbit_pack_weights(fmt, E, N, K, group_size, codes, scales, zeros, packed, packed_bytes, stream=None):
    return lib().lowbit_pack_weights(fmt, E, N, K, group_size, _ptr(codes), _ptr(scales), _ptr(zeros),
                                     _ptr(packed), packed_bytes, _stream(stream))


def lowbit_unpack_weights(fmt, E, N, K, group_size, packed, packed_bytes, codes, scales, zeros, stream=None):
    return lib().lowbit_unpack_weights(fmt, E, N, K, group_size, _ptr(packed), packed_bytes, _ptr(codes),
                                       _ptr(scales), _ptr(zeros), _stream(stream))


def lowbit_hbm_read(buf, nbytes, sink, stream=None):
    return lib().lowbit_hbm_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream))


def lowbit_dequant(fmt, N, K, group_size, packed, packed_bytes, w_out, stream=None):
    return lib().lowbit_dequant(fmt, N, K, group_size, _ptr(packed), packed_bytes, _ptr(w_out), _stream(stream))


def lowbit_workspace_bytes(op, fmt, M, N, K, group_size):
    return lib().lowbit_workspace_bytes(op, fmt, M, N, K, group_size)


def lowbit_gemv(fmt, M, N, K, group_size, packed, x, y, workspace=None, ws_bytes=0, stream=None):
    return lib().lowbit_gemv(fmt, M, N, K, group_size, _ptr(packed), _ptr(x), _ptr(y), _ptr(workspace),
                             ws_bytes, _stream(stream))


def lowbit_gemm(fmt, M, N, K, group_size, packed, a, a_dtype, c, c_dtype, workspace=None, ws_bytes=0, stream=None):
    return lib().lowbit_gemm(fmt, M, N, K, group_size, _ptr(packed), _ptr(a), a_dtype, _ptr(c), c_dtype,
                             _ptr(workspace), ws_bytes, _stream(stream))


def lowbit_moe_align(topk_ids, T, top_k, E, block_m, expert_map, sorted_ids, expert_offsets, block_expert,
                     num_post_padded, stream=None):
    return lib().lowbit_moe_align(_ptr(topk_ids), T, top_k, E, block_m, _ptr(expert_map), _ptr(sorted_ids),
                                  _ptr(expert_offsets), _ptr(block_expert), _ptr(num_post_padded), _stream(stream))


def lowbit_moe_gemm(fmt, E_local, N, K, packed, E, a_e4m3, a_ue8m0, a_rows, a_row_div, sorted_ids,
                    expert_offsets, block_expert, num_valid, block_m, out, stream=None):
    return lib().lowbit_moe_gemm(fmt, E_local, N, K, _ptr(packed), E, _ptr(a_e4m3), _ptr(a_ue8m0), a_rows,
                                 a_row_div, _ptr(sorted_ids), _ptr(expert_offsets), _ptr(block_expert), num_valid,
                                 block_m, _ptr(out), _stream(stream))


def lowbit_mxfp8_quant(x, R, K, q, scale, stream=None):
    return lib().lowbit_mxfp8_quant(_ptr(x), R, K, _ptr(q), _ptr(scale), _stream(stream))


def lowbit_moe_silu_mul_quant(gate_up, R, I, q, scale, stream=None):
    return lib().lowbit_moe_silu_mul_quant(_ptr(gate_up), R, I, _ptr(q), _ptr(scale), _stream(stream))


def lowbit_moe_gemm_silu_quant(fmt, E_local, I, K, packed, E, a_e4m3, a_ue8m0, a_rows, a_row_div, sorted_ids,
                               expert_offsets, block_expert, num_valid, block_m, q, scale, stream=None):
    return lib().lowbit_moe_gemm_silu_quant(fmt, E_local, I, K, _ptr(packed), E, _ptr(a_e4m3), _ptr(a_ue8m0), a_rows,
                                            a_row_div, _ptr(sorted_ids), _ptr(expert_offsets), _ptr(block_expert),
                                            num_valid, block_m, _ptr(q), _ptr(scale), _stream(stream))


def lowbit_moe_combine(expert_out, topk_weights, T, top_k, H, y, stream=None):
    return lib().lowbit_moe_combine(_ptr(expert_out), _ptr(topk_weights), T, top_k, H, _ptr(y), _stream(stream))


def lowbit_moe_layer_workspace_bytes(T, top_k, E, H, I, block_m):
    return lib().lowbit_moe_layer_workspace_bytes(T, top_k, E, H, I, block_m)


def lowbit_moe_layer(w13, w2, E_local, E, H, I, x, topk_ids, topk_weights, T, top_k, expert_map, block_m, y,
                     workspace, ws_bytes, stream=None):
    return lib().lowbit_moe_layer(_ptr(w13), _ptr(w2), E_local, E, H, I, _ptr(x), _ptr(topk_ids),
                                  _ptr(topk_weights), T, top_k, _ptr(expert_map), block_m, _ptr(y), _ptr(workspace),
                                  ws_bytes, _stream(stream))


def make_gemv_problems(problems):
    """[(packed, x, y, N, K), ...] -> a ctypes array of lowbit_gemv_problem."""
    arr = (lowbit_gemv_problem * max(len(problems), 1))()
    for i, (packed, x, y, N, K) in enumerate(problems):
        arr[i] = lowbit_gemv_problem(_ptr(packed), _ptr(x), _ptr(y), N, K)
    return arr


def lowbit_gemv_batched(fmt, M, group_size, count, problems, stream=None):
    """problems: a ctypes array from make_gemv_problems (host memory)."""
    return lib().lowbit_gemv_batched(fmt, M, group_size, count, ctypes.cast(problems, ctypes.c_void_p),
                                     _stream(stream))


def lowbit_quant_act_i8(M, K, x, xq, x_scale, stream=None):
    return lib().lowbit_quant_act_i8(M, K, _ptr(x), _ptr(xq), _ptr(x_scale), _stream(stream))


def lowbit_gemv_w4a8(fmt, M, N, K, group_size, packed, x, y, workspace=None, ws_bytes=0, stream=None):
    return lib().lowbit_gemv_w4a8(fmt, M, N, K, group_size, _ptr(packed), _ptr(x), _ptr(y), _ptr(workspace),
                                  ws_bytes, _stream(stream))


def lowbit_gemv_w4a8_batched_workspace_bytes(fmt, M, group_size, count, problems):
    return lib().lowbit_gemv_w4a8_batched_workspace_bytes(fmt, M, group_size, count,
                                                          ctypes.cast(problems, ctypes.c_void_p))


def lowbit_gemv_w4a8_batched(fmt, M, group_size, count, problems, workspace=None, ws_bytes=0, stream=None):
    """problems: a ctypes array from make_gemv_problems (host memory)."""
    return lib().lowbit_gemv_w4a8_batched(fmt, M, group_size, count, ctypes.cast(problems, ctypes.c_void_p),
                                          _ptr(workspace), ws_bytes, _stream(stream))


def lowbit_gemv_w4a8_batched_noalloc(fmt, M, group_size, count, problems, stream=None):
    """problems: a ctypes array from make_gemv_problems (host memory)."""
    return lib().lowbit_gemv_w4a8_batched_noalloc(fmt, M, group_size, count, ctypes.cast(problems, ctypes.c_void_p),
                                                  _stream(stream))


def lowbit_gemv_chain_bytes(count, stages):
    return lib().lowbit_gemv_chain_bytes(count, stages)


def lowbit_gemv_chain_init(chain, fmt, M, group_size, count, problems, stage_of, spin_limit, buf, buf_bytes,
                           stream=None):
    """chain: a lowbit_gemv_chain (filled in); problems: from make_gemv_problems;
    stage_of: a sequence of ints (copied into a host int array)."""
    st = (ctypes.c_int * max(len(stage_of), 1))(*stage_of)
    return lib().lowbit_gemv_chain_init(ctypes.byref(chain), fmt, M, group_size, count,
                                        ctypes.cast(problems, ctypes.c_void_p), ctypes.cast(st, ctypes.c_void_p),
                                        spin_limit, _ptr(buf), buf_bytes, _stream(stream))


def lowbit_gemv_chain_run(chain, stream=None):
    return lib().lowbit_gemv_chain_run(ctypes.byref(chain), _stream(stream))


def lowbit_gemv_chain_error(chain, stream=None):
    """Returns (status, error_word)."""
    v = ctypes.c_uint(0)
    st = lib().lowbit_gemv_chain_error(ctypes.byref(chain), ctypes.byref(v), _stream(stream))
    return st, v.value
