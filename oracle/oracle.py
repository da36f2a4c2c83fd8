"""ctypes loader for the C oracle (test infrastructure only).

Builds ``liblowbit_oracle.so`` from ``lowbit_oracle.c`` with gcc when it is
missing (plain ``-O2``, no fast-math, no vectorisation flags), then exposes
numpy-in / numpy-out wrappers.  All arithmetic happens in the C file.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lowbit_oracle.c")
_LIB = os.path.join(_HERE, "liblowbit_oracle.so")

_default = None


def build(force=False):
    """Compile the oracle with gcc (single-threaded C, -O2, IEEE semantics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
            "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_variant(src_text, out_path):
    """Compile a modified copy of the oracle source (used by the tests that
    plant mistakes in the oracle to show the pins catch them)."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
        "-ffp-contract=off", "-w", "-o", out_path, c_path, "-lm"])
    return Oracle(out_path)


def source_text():
    with open(_SRC) as f:
        return f.read()


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _declare(lib):
    sig = {
        "orc_w4_unpack": [_p, _i64, _i64, _p],
        "orc_w4_dequant": [_p, _p, _p, _i64, _i64, _int, _p],
        "orc_w4_matmul": [_p, _int, _i64, _i64, _i64, _int, _p, _p, _p, _p, _p, _int],
        "orc_w4_matmul_rows": [_p, _int, _i64, _i64, _int, _p, _p, _p, _p, _i64, _p, _p, _int],
        "orc_lut3_dequant": [_p, _p, _p, _i64, _i64, _i64, _p],
        "orc_wb_dequant": [_p, _p, _p, _int, _i64, _i64, _int, _p],
        "orc_wb_matmul": [_p, _i64, _i64, _i64, _int, _int, _p, _p, _p, _p, _p],
        "orc_moe_align": [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _i64],
        "orc_moe_gemm": [_p, _p, _p, _i64, _i64, _i64, _p, _p, _i64, _p, _i64, _i64, _p, _p, _p],
        "orc_quant_act_i8": [_p, _i64, _i64, _p, _p],
        "orc_w4a8_matmul": [_p, _i64, _i64, _i64, _int, _p, _p, _p, _p, _p],
        "orc_mxfp8_quant": [_p, _i64, _i64, _p, _p],
        "orc_silu_mul_bf16": [_p, _i64, _i64, _p],
        "orc_moe_combine": [_p, _p, _i64, _i64, _i64, _p, _p],
        "orc_silu_f32_array": [_p, _i64, _p],
        "orc_exp2_f32_array": [_p, _i64, _p],
        "orc_double_array_to_e4m3": [_p, _i64, _p],
        "orc_f16_array_to_double": [_p, _i64, _p],
        "orc_bf16_array_to_double": [_p, _i64, _p],
        "orc_double_array_to_f16": [_p, _i64, _p],
        "orc_double_array_to_bf16": [_p, _i64, _p],
        "orc_e4m3_array_to_double": [_p, _i64, _p],
        "orc_ue8m0_array_to_double": [_p, _i64, _p],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.orc_moe_align.restype = _i64
    lib.orc_version.restype = _int


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _f16_bits(a):
    """fp16 ndarray (or uint16 bit pattern array) -> contiguous uint16 bits."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16)
    return _c(a, np.uint16)


class Oracle:
    """Numpy wrappers around one build of the C oracle."""

    def __init__(self, lib_path):
        self._lib = ctypes.CDLL(lib_path)
        _declare(self._lib)

    # ---------------------------------------------------------------- formats
    def f16_to_double(self, bits):
        b = _f16_bits(bits).ravel()
        out = np.empty(b.size, np.float64)
        self._lib.orc_f16_array_to_double(_ptr(b), b.size, _ptr(out))
        return out.reshape(np.shape(bits))

    def bf16_to_double(self, bits):
        b = _c(bits, np.uint16).ravel()
        out = np.empty(b.size, np.float64)
        self._lib.orc_bf16_array_to_double(_ptr(b), b.size, _ptr(out))
        return out.reshape(np.shape(bits))

    def double_to_f16(self, v):
        v = _c(v, np.float64).ravel()
        out = np.empty(v.size, np.uint16)
        self._lib.orc_double_array_to_f16(_ptr(v), v.size, _ptr(out))
        return out

    def double_to_bf16(self, v):
        v = _c(v, np.float64).ravel()
        out = np.empty(v.size, np.uint16)
        self._lib.orc_double_array_to_bf16(_ptr(v), v.size, _ptr(out))
        return out

    def e4m3_to_double(self, b):
        b = _c(b, np.uint8).ravel()
        out = np.empty(b.size, np.float64)
        self._lib.orc_e4m3_array_to_double(_ptr(b), b.size, _ptr(out))
        return out

    def ue8m0_to_double(self, b):
        b = _c(b, np.uint8).ravel()
        out = np.empty(b.size, np.float64)
        self._lib.orc_ue8m0_array_to_double(_ptr(b), b.size, _ptr(out))
        return out

    # ---------------------------------------------------------------- INT4
    def w4_unpack(self, qweight):
        """qweight u8 [N][K/2] -> codes u8 [N][K] (low nibble = even k)."""
        q = _c(qweight, np.uint8)
        N, Kh = q.shape
        out = np.empty((N, 2 * Kh), np.uint8)
        self._lib.orc_w4_unpack(_ptr(q), N, 2 * Kh, _ptr(out))
        return out

    def w4_dequant(self, qweight, scales, zeros, group_size):
        """-> float32 [N][K], w = (q - z) * s, exact."""
        q = _c(qweight, np.uint8)
        N, Kh = q.shape
        K = 2 * Kh
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        assert s.shape == (N, K // group_size)
        out = np.empty((N, K), np.float32)
        self._lib.orc_w4_dequant(_ptr(q), _ptr(s), _ptr(z), N, K, group_size, _ptr(out))
        return out

    def w4_matmul(self, x, x_dtype, qweight, scales, zeros, group_size, out_dtype):
        """y = x @ dequant(W).T.

        x: [M][K] as fp16 ndarray (x_dtype "f16") or uint16 bf16 bits (x_dtype "bf16").
        Returns (y64 float64 [M][N], y_bits uint16 [M][N] rounded RNE to out_dtype).
        """
        xd = {"f16": 0, "bf16": 1}[x_dtype]
        od = {"f16": 0, "bf16": 1}[out_dtype]
        xb = _f16_bits(x) if xd == 0 else _c(x, np.uint16)
        M, K = xb.shape
        q = _c(qweight, np.uint8)
        N = q.shape[0]
        assert q.shape == (N, K // 2)
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        y64 = np.empty((M, N), np.float64)
        yb = np.empty((M, N), np.uint16)
        self._lib.orc_w4_matmul(_ptr(xb), xd, M, N, K, group_size, _ptr(q), _ptr(s), _ptr(z),
                              _ptr(y64), _ptr(yb), od)
        return y64, yb

    def w4_matmul_rows(self, x, x_dtype, qweight, scales, zeros, group_size, out_dtype, rows):
        """w4_matmul restricted to the given rows of x (rows are independent)."""
        xd = {"f16": 0, "bf16": 1}[x_dtype]
        od = {"f16": 0, "bf16": 1}[out_dtype]
        xb = _f16_bits(x) if xd == 0 else _c(x, np.uint16)
        M, K = xb.shape
        q = _c(qweight, np.uint8)
        N = q.shape[0]
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        r = _c(rows, np.int64)
        assert r.min() >= 0 and r.max() < M
        y64 = np.empty((r.size, N), np.float64)
        yb = np.empty((r.size, N), np.uint16)
        self._lib.orc_w4_matmul_rows(_ptr(xb), xd, K, N, group_size, _ptr(q), _ptr(s), _ptr(z),
                                   _ptr(r), r.size, _ptr(y64), _ptr(yb), od)
        return y64, yb

    # ---------------------------------------------------------------- b-bit codes
    def wb_dequant(self, codes, scales, zeros, bits, group_size):
        """codes u8 [N][K] (< 2^bits) -> float32 [N][K], w = (q - z) * s, exact."""
        c = _c(codes, np.uint8)
        N, K = c.shape
        assert int(c.max(initial=0)) < (1 << bits)
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        out = np.empty((N, K), np.float32)
        self._lib.orc_wb_dequant(_ptr(c), _ptr(s), _ptr(z), bits, N, K, group_size, _ptr(out))
        return out

    def wb_matmul(self, x, codes, scales, zeros, bits, group_size):
        """fp16 x [M][K] against b-bit weights -> (y64 [M][N], y fp16 bits [M][N])."""
        xb = _f16_bits(x)
        M, K = xb.shape
        c = _c(codes, np.uint8)
        N = c.shape[0]
        assert c.shape == (N, K)
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        y64 = np.empty((M, N), np.float64)
        yb = np.empty((M, N), np.uint16)
        self._lib.orc_wb_matmul(_ptr(xb), M, N, K, group_size, bits, _ptr(c), _ptr(s), _ptr(z), _ptr(y64), _ptr(yb))
        return y64, yb

    # ---------------------------------------------------------------- W4A8
    def quant_act_i8(self, x):
        """fp16 x [M][K] -> (codes int8 [M][K], scales float32 [M]): per-token
        symmetric INT8, decisions in binary32."""
        xb = _f16_bits(x)
        M, K = xb.shape
        xq = np.empty((M, K), np.int8)
        sx = np.empty(M, np.float32)
        self._lib.orc_quant_act_i8(_ptr(xb), M, K, _ptr(xq), _ptr(sx))
        return xq, sx

    def w4a8_matmul(self, x, qweight, scales, zeros, group_size):
        """INT4 weights x dynamically quantized INT8 activations.
        Returns (y64 float64 [M][N], y_bits uint16 fp16 [M][N])."""
        xb = _f16_bits(x)
        M, K = xb.shape
        q = _c(qweight, np.uint8)
        N = q.shape[0]
        assert q.shape == (N, K // 2)
        s = _f16_bits(scales)
        z = None if zeros is None else _c(zeros, np.int8)
        y64 = np.empty((M, N), np.float64)
        yb = np.empty((M, N), np.uint16)
        self._lib.orc_w4a8_matmul(_ptr(xb), M, N, K, group_size, _ptr(q), _ptr(s), _ptr(z), _ptr(y64), _ptr(yb))
        return y64, yb

    # ---------------------------------------------------------------- LUT3 MoE
    def lut3_dequant(self, idx, cb, ex):
        """idx u8 [E][N][K] (0..7), cb u8 [E][N/8][K/64][8], ex u8 [E][N/8][K/64] -> float64 [E][N][K]."""
        i = _c(idx, np.uint8)
        E, N, K = i.shape
        c = _c(cb, np.uint8)
        e = _c(ex, np.uint8)
        assert c.shape == (E, N // 8, K // 64, 8) and e.shape == (E, N // 8, K // 64)
        out = np.empty((E, N, K), np.float64)
        self._lib.orc_lut3_dequant(_ptr(i), _ptr(c), _ptr(e), E, N, K, _ptr(out))
        return out

    def moe_align(self, topk_ids, E, block_m, expert_map=None):
        """-> (sorted_ids int32 [P], block_expert int32 [P/block_m], P)."""
        t = _c(topk_ids, np.int32)
        T, top_k = t.shape
        cap = T * top_k + E * (block_m - 1)
        sorted_ids = np.full(cap, -7, np.int32)
        block_expert = np.full(max(cap // block_m + 1, 1), -7, np.int32)
        m = None if expert_map is None else _c(expert_map, np.int32)
        P = self._lib.orc_moe_align(_ptr(t), T, top_k, E, block_m, _ptr(m),
                                  _ptr(sorted_ids), _ptr(block_expert), cap)
        assert P >= 0
        return sorted_ids[:P].copy(), block_expert[:P // block_m].copy(), int(P)

    def moe_gemm(self, idx, cb, ex, aq, as_, a_row_div, topk_ids, expert_map=None):
        """Grouped product over routed slots -> (y64 float64 [T*top_k][N], out bf16 bits [T*top_k][N])."""
        i = _c(idx, np.uint8)
        E, N, K = i.shape
        c = _c(cb, np.uint8)
        e = _c(ex, np.uint8)
        a = _c(aq, np.uint8)
        s = _c(as_, np.uint8)
        assert a.shape[1] == K and s.shape == (a.shape[0], K // 32)
        t = _c(topk_ids, np.int32)
        T, top_k = t.shape
        assert a.shape[0] * a_row_div >= T * top_k
        m = None if expert_map is None else _c(expert_map, np.int32)
        y64 = np.empty((T * top_k, N), np.float64)
        ob = np.empty((T * top_k, N), np.uint16)
        self._lib.orc_moe_gemm(_ptr(i), _ptr(c), _ptr(e), E, N, K, _ptr(a), _ptr(s), a_row_div,
                             _ptr(t), T, top_k, _ptr(m), _ptr(y64), _ptr(ob))
        return y64, ob

    # ---------------------------------------------------------------- MoE layer
    def double_to_e4m3(self, v):
        v = _c(v, np.float64).ravel()
        out = np.empty(v.size, np.uint8)
        self._lib.orc_double_array_to_e4m3(_ptr(v), v.size, _ptr(out))
        return out

    def exp2_f32(self, t):
        t = _c(t, np.float32).ravel()
        out = np.empty(t.size, np.float32)
        self._lib.orc_exp2_f32_array(_ptr(t), t.size, _ptr(out))
        return out

    def silu_f32(self, g):
        g = _c(g, np.float32).ravel()
        out = np.empty(g.size, np.float32)
        self._lib.orc_silu_f32_array(_ptr(g), g.size, _ptr(out))
        return out

    def mxfp8_quant(self, x_bf16):
        """bf16 bits [R][K] -> (E4M3 bytes [R][K], UE8M0 bytes [R][K/32])."""
        x = _c(x_bf16, np.uint16)
        R, K = x.shape
        assert K % 32 == 0
        q = np.empty((R, K), np.uint8)
        sc = np.empty((R, K // 32), np.uint8)
        self._lib.orc_mxfp8_quant(_ptr(x), R, K, _ptr(q), _ptr(sc))
        return q, sc

    def silu_mul_bf16(self, gu_bf16):
        """bf16 bits [R][2I] (gate | up) -> bf16 bits [R][I]."""
        gu = _c(gu_bf16, np.uint16)
        R, I2 = gu.shape
        act = np.empty((R, I2 // 2), np.uint16)
        self._lib.orc_silu_mul_bf16(_ptr(gu), R, I2 // 2, _ptr(act))
        return act

    def silu_mul_quant(self, gu_bf16):
        """SiLU(gate) * up, then MXFP8: -> (E4M3 [R][I], UE8M0 [R][I/32])."""
        return self.mxfp8_quant(self.silu_mul_bf16(gu_bf16))

    def moe_combine(self, out_bf16, w, top_k):
        """out bf16 bits [T*top_k][H], w f32 [T][top_k] -> (y64 [T][H], y bf16 bits [T][H])."""
        o = _c(out_bf16, np.uint16)
        ww = _c(w, np.float32)
        T = ww.shape[0]
        H = o.shape[1]
        assert ww.shape == (T, top_k) and o.shape[0] == T * top_k
        y64 = np.empty((T, H), np.float64)
        yb = np.empty((T, H), np.uint16)
        self._lib.orc_moe_combine(_ptr(o), _ptr(ww), T, top_k, H, _ptr(y64), _ptr(yb))
        return y64, yb

    def moe_layer(self, w13, w2, x_bf16, topk_ids, topk_w, expert_map=None):
        """The whole layer, step by step: MXFP8 of the hidden rows, gate/up
        grouped GEMM (row of slot sid = sid / top_k), SiLU(gate) * up and
        MXFP8, down grouped GEMM (row = sid), router-weighted combine.
        w13 / w2: dicts of idx, cb, ex (canonical LUT3 arrays).  Returns a dict
        of every intermediate and the output (y64, y bf16 bits)."""
        top_k = topk_ids.shape[1]
        xq, xs = self.mxfp8_quant(x_bf16)
        _, gu = self.moe_gemm(w13["idx"], w13["cb"], w13["ex"], xq, xs, top_k, topk_ids, expert_map)
        aq, as_ = self.silu_mul_quant(gu)
        _, out = self.moe_gemm(w2["idx"], w2["cb"], w2["ex"], aq, as_, 1, topk_ids, expert_map)
        y64, yb = self.moe_combine(out, topk_w, top_k)
        return dict(xq=xq, xs=xs, gate_up=gu, aq=aq, as_=as_, down=out, y64=y64, y=yb)

    def version(self):
        return self._lib.orc_version()


def _get():
    global _default
    if _default is None:
        build()                      # compiles when the library is missing or older than the source
        _default = Oracle(_LIB)
    return _default


def f16_to_double(*a, **k):
    return _get().f16_to_double(*a, **k)


def bf16_to_double(*a, **k):
    return _get().bf16_to_double(*a, **k)


def double_to_f16(*a, **k):
    return _get().double_to_f16(*a, **k)


def double_to_bf16(*a, **k):
    return _get().double_to_bf16(*a, **k)


def e4m3_to_double(*a, **k):
    return _get().e4m3_to_double(*a, **k)


def ue8m0_to_double(*a, **k):
    return _get().ue8m0_to_double(*a, **k)


def w4_unpack(*a, **k):
    return _get().w4_unpack(*a, **k)


def w4_dequant(*a, **k):
    return _get().w4_dequant(*a, **k)


def w4_matmul(*a, **k):
    return _get().w4_matmul(*a, **k)


def w4_matmul_rows(*a, **k):
    return _get().w4_matmul_rows(*a, **k)


def wb_dequant(*a, **k):
    return _get().wb_dequant(*a, **k)


def wb_matmul(*a, **k):
    return _get().wb_matmul(*a, **k)


def quant_act_i8(*a, **k):
    return _get().quant_act_i8(*a, **k)


def w4a8_matmul(*a, **k):
    return _get().w4a8_matmul(*a, **k)


def lut3_dequant(*a, **k):
    return _get().lut3_dequant(*a, **k)


def moe_align(*a, **k):
    return _get().moe_align(*a, **k)


def moe_gemm(*a, **k):
    return _get().moe_gemm(*a, **k)


def double_to_e4m3(*a, **k):
    return _get().double_to_e4m3(*a, **k)


def exp2_f32(*a, **k):
    return _get().exp2_f32(*a, **k)


def silu_f32(*a, **k):
    return _get().silu_f32(*a, **k)


def mxfp8_quant(*a, **k):
    return _get().mxfp8_quant(*a, **k)


def silu_mul_bf16(*a, **k):
    return _get().silu_mul_bf16(*a, **k)


def silu_mul_quant(*a, **k):
    return _get().silu_mul_quant(*a, **k)


def moe_combine(*a, **k):
    return _get().moe_combine(*a, **k)


def moe_layer(*a, **k):
    return _get().moe_layer(*a, **k)


def version(*a, **k):
    return _get().version(*a, **k)


def default():
    """The oracle built from lowbit_oracle.c."""
    return _get()


__all__ = ["build", "build_variant", "source_text", "Oracle", "default", "f16_to_double", "bf16_to_double", "double_to_f16", "double_to_bf16", "e4m3_to_double", "ue8m0_to_double", "w4_unpack", "w4_dequant", "w4_matmul", "w4_matmul_rows", "wb_dequant", "wb_matmul", "quant_act_i8", "w4a8_matmul", "lut3_dequant", "moe_align", "moe_gemm", "double_to_e4m3", "exp2_f32", "silu_f32", "mxfp8_quant", "silu_mul_bf16", "silu_mul_quant", "moe_combine", "moe_layer", "version"]
