"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes one build of the oracle (``oracle.Oracle``) and raises
AssertionError on a mismatch.  They use only:
  * values written out by hand in ``tests/golden`` (cited there);
  * library routines (numpy float16, torch bfloat16 / float8 decodes,
    numpy float64 matmul) on the cases that reduce to them;
  * exact rational arithmetic (``fractions.Fraction``) on tiny inputs;
  * invariants of the definitions (one-hot input, all codes at the zero
    point, power-of-two scaling, K split at a group boundary, routing
    bookkeeping).
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on copies of the oracle with a planted mistake and expects a failure.
"""
import json
import os
from fractions import Fraction as F

import numpy as np
import torch

from bit_weight_only_pack_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex(s):
    return int(s, 16)


def _np_f16_bits(v):
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _same_or_both_nan(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nan = np.isnan(a) & np.isnan(b)
    same = a.view(np.uint64) == b.view(np.uint64)
    return bool(np.all(nan | same))


def _frac_f16(bits):
    """Exact value of fp16 bit patterns via numpy's decode."""
    return [F(float(v)) for v in np.asarray(bits, np.uint16).view(np.float16).astype(np.float64).ravel()]


def _torch_bf16_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _torch_e4m3_to_f64(b):
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_ue8m0_to_f64(b):
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


def _pack_codes(codes):
    """codes u8 [N][K] -> bytes [N][K/2], low nibble = even k (the page's order)."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


# ------------------------------------------------------------------ formats
def check_f16_decode(o):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    assert _same_or_both_nan(o.f16_to_double(bits), ref), "fp16 decode differs from numpy"


def check_f16_encode(o):
    finite = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (finite[:-1] + finite[1:]) / 2.0                   # exact ties
    near = np.concatenate([mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40)])
    r = np.random.default_rng(11)
    rand = np.exp2(r.uniform(-30, 17, 20000)) * r.choice([-1.0, 1.0], 20000)
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -26,
                     2.0 ** -24, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0, np.inf, -np.inf])
    v = np.concatenate([finite, -finite, mids, -mids, near, rand, edge])
    got = o.double_to_f16(v)
    ref = _np_f16_bits(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "fp16 RNE differs from numpy at %r" % (v[bad[:5]],)


def check_bf16_decode(o):
    bits = np.arange(65536, dtype=np.uint16)
    assert _same_or_both_nan(o.bf16_to_double(bits), _torch_bf16_to_f64(bits)), "bf16 decode differs from torch"


def check_bf16_encode(o):
    allb = np.arange(65536, dtype=np.uint16)
    vals = _torch_bf16_to_f64(allb)
    fin = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (fin[:-1] + fin[1:]) / 2.0                         # 9 significant bits: exact in fp32
    r = np.random.default_rng(12)
    rand = (np.exp2(r.uniform(-130, 127, 20000)) * r.choice([-1.0, 1.0], 20000)).astype(np.float32)
    v = np.concatenate([fin, -fin, mids, -mids, rand.astype(np.float64)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.double_to_bf16(v.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "bf16 RNE differs from torch at %r" % (v[bad[:5]],)


def check_e4m3_decode(o):
    b = np.arange(256, dtype=np.uint8)
    assert _same_or_both_nan(o.e4m3_to_double(b), _torch_e4m3_to_f64(b)), "E4M3 decode differs from torch"


def check_ue8m0_decode(o):
    b = np.arange(256, dtype=np.uint8)
    assert _same_or_both_nan(o.ue8m0_to_double(b), _torch_ue8m0_to_f64(b)), "UE8M0 decode differs from torch"


# ------------------------------------------------------------------ INT4: hand-worked values
def check_hand_bytes(o):
    g = _golden("w4_hand_examples.json")
    for scale_hex, frac in g["fp16_scales"].items():
        assert F(float(o.f16_to_double(np.array([_hex(scale_hex)], np.uint16))[0])) == F(frac), scale_hex
    for ex in g["bytes"]:
        q = np.array([[_hex(ex["byte"])]], np.uint8)
        assert list(o.w4_unpack(q)[0]) == ex["codes"], ex["name"]
        s = np.array([[_hex(ex["scale"])]], np.uint16)
        z = None if ex["zero"] == 8 else np.array([[ex["zero"]]], np.int8)
        w = o.w4_dequant(q, s, z, 2)[0]
        assert [F(float(v)) for v in w] == [F(t) for t in ex["w"]], ex["name"]
        assert [F(float(v)) for v in w] == [F(t) for t in ex["w_decimal"]], ex["name"]


def check_sixteen_codes(o):
    g = _golden("w4_hand_examples.json")["sixteen_codes"]
    codes = np.arange(16, dtype=np.uint8)[None, :]
    q = _pack_codes(codes)
    s = np.array([[_hex(g["scale"])]], np.uint16)
    w8 = o.w4_dequant(q, s, None, 16)[0]
    assert [F(float(v)) for v in w8] == [F(t) for t in g["z8_decimal"]], "16-code identity, z=8"
    w5 = o.w4_dequant(q, s, np.array([[5]], np.int8), 16)[0]
    sv = F(1311, 131072)
    assert [F(float(v)) for v in w5] == [(c - 5) * sv for c in range(16)], "16-code identity, z=5"


def check_dequant_exact_all_scales(o):
    """(q - z) * s is exact in fp32 for every finite fp16 scale, every code and
    zero points over the int8 range: compare with the float64 product, which
    is exact here (<= 19 significant bits)."""
    sc = np.arange(0, 0x7c00, dtype=np.uint16)
    sc = np.concatenate([sc, sc | 0x8000])
    n = sc.size
    r = np.random.default_rng(13)
    K = 16
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, 1))
    zeros = r.integers(-128, 128, size=(n, 1)).astype(np.int8)
    w = o.w4_dequant(_pack_codes(codes), sc[:, None], zeros, K)
    ref = (codes.astype(np.float64) - zeros.astype(np.float64)) * sc.view(np.float16).astype(np.float64)[:, None]
    assert np.array_equal(w.astype(np.float64), ref), "dequant not exact"
    wsym = o.w4_dequant(_pack_codes(codes), sc[:, None], None, K)
    refsym = (codes.astype(np.float64) - 8.0) * sc.view(np.float16).astype(np.float64)[:, None]
    assert np.array_equal(wsym.astype(np.float64), refsym), "symmetric dequant not exact"


def check_fp16_tie(o):
    t = _golden("w4_hand_examples.json")["fp16_rounding_tie"]
    q = _pack_codes(np.array([[t["code"], 0]], np.uint8))
    s = np.array([[_hex(t["scale"])]], np.uint16)
    w = o.w4_dequant(q, s, None, 2)[0, 0]
    assert F(float(w)) == F(t["w_exact"])
    h = o.double_to_f16(np.array([float(w)]))
    assert F(float(o.f16_to_double(h)[0])) == F(t["w_f16_rne"]), "tie must round to even"


def check_gemv_2x4(o):
    g = _golden("w4_hand_examples.json")["gemv_2x4"]
    q = np.array([[_hex(b) for b in row] for row in g["qweight"]], np.uint8)
    s = np.array([[_hex(b) for b in row] for row in g["scales"]], np.uint16)
    x = np.array([float(F(v)) for v in g["x"]], np.float16)[None, :]
    for key in ("symmetric", "asymmetric"):
        case = g[key]
        z = None if key == "symmetric" else np.array(case["zeros"], np.int8)
        W = o.w4_dequant(q, s, z, 2)
        assert [[F(float(v)) for v in row] for row in W] == [[F(v) for v in row] for row in case["W"]], key
        y64, yb = o.w4_matmul(x, "f16", q, s, z, 2, "f16")
        assert [F(float(v)) for v in y64[0]] == [F(v) for v in case["y"]], key
        assert np.array_equal(yb[0], _np_f16_bits([float(F(v)) for v in case["y"]])), key


# ------------------------------------------------------------------ INT4: brute force and invariants
def _exact_matmul(x_frac, codes, zeros, s_frac, G):
    """Exact rational y[m][n] = sum_k x[m][k] * (q - z) * s over Python Fractions."""
    M, K = len(x_frac), len(x_frac[0])
    N = codes.shape[0]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = F(0)
            mag = F(0)
            for k in range(K):
                z = 8 if zeros is None else int(zeros[n, k // G])
                t = x_frac[m][k] * (int(codes[n, k]) - z) * s_frac[n][k // G]
                acc += t
                mag += abs(t)
            row.append((acc, mag))
        out.append(row)
    return out


def _check_bruteforce_case(o, M, N, K, G, x_dtype, out_dtype, asym, seed):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    q = _pack_codes(codes)
    s_bits = r.uniform(0.002, 0.05, size=(N, K // G)).astype(np.float16).view(np.uint16)
    s_bits[0, 0] = 0x0203                                      # an fp16 subnormal scale
    zeros = r.integers(-128, 128, size=(N, K // G)).astype(np.int8) if asym else None
    xv = r.standard_normal((M, K)) * 3
    if x_dtype == "f16":
        xb = xv.astype(np.float16).view(np.uint16)
        xf = [[F(float(v)) for v in row] for row in xb.view(np.float16).astype(np.float64)]
    else:
        xb = torch.from_numpy(xv.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xf = [[F(float(v)) for v in row] for row in _torch_bf16_to_f64(xb)]
    sf = [_frac_f16(row) for row in s_bits]
    exact = _exact_matmul(xf, codes, zeros, sf, G)
    y64, yb = o.w4_matmul(xb, x_dtype, q, s_bits, zeros, G, out_dtype)
    for m in range(M):
        for n in range(N):
            e, mag = exact[m][n]
            bound = (K + 1) * F(1, 2 ** 53) * mag
            assert abs(F(float(y64[m, n])) - e) <= bound, ("sum", M, N, K, G, m, n)
            if out_dtype == "f16":
                ref_bits = _np_f16_bits([float(e)])[0]
            else:
                ref_bits = o.double_to_bf16(np.array([float(e)]))[0]
            assert yb[m, n] == ref_bits, ("rounding", M, N, K, G, m, n)


def check_bruteforce_tiny(o):
    _check_bruteforce_case(o, 1, 5, 8, 2, "f16", "f16", False, 1)
    _check_bruteforce_case(o, 3, 7, 64, 32, "f16", "f16", True, 2)
    _check_bruteforce_case(o, 2, 9, 96, 32, "bf16", "bf16", False, 3)
    _check_bruteforce_case(o, 2, 4, 128, 64, "bf16", "bf16", True, 4)
    _check_bruteforce_case(o, 1, 3, 256, 128, "f16", "f16", True, 5)


def check_bruteforce_tiny_gemv_workload(o):
    """All 65,536 terms of the tiny GEMV workload (M=1, K=256, N=256, G=32,
    symmetric) against exact rationals."""
    w = synth.w4_weights(256, 256, 32, scale_range=(0.005, 0.02), workload_id=0)
    x = synth.activations_f16(1, 256, workload_id=0)
    codes = np.empty((256, 256), np.uint8)
    codes[:, 0::2] = w["qweight"] & 0xF
    codes[:, 1::2] = w["qweight"] >> 4
    xf = [[F(float(v)) for v in x[0].astype(np.float64)]]
    sf = [_frac_f16(row) for row in w["scales"].view(np.uint16)]
    exact = _exact_matmul(xf, codes, None, sf, 32)
    y64, yb = o.w4_matmul(x, "f16", w["qweight"], w["scales"], None, 32, "f16")
    for n in range(256):
        e, mag = exact[0][n]
        assert abs(F(float(y64[0, n])) - e) <= 257 * F(1, 2 ** 53) * mag, n
        assert yb[0, n] == _np_f16_bits([float(e)])[0], n


def _random_w4(r, N, K, G, asym):
    codes = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = r.uniform(0.002, 0.02, size=(N, K // G)).astype(np.float16)
    z = r.integers(0, 16, size=(N, K // G)).astype(np.int8) if asym else None
    return codes, _pack_codes(codes), s, z


def check_numpy_matmul(o):
    """Oracle product == numpy float64 matmul of the (pinned) dequantized W."""
    r = np.random.default_rng(21)
    for (M, N, K, G, asym, xd) in ((3, 48, 256, 32, True, "f16"), (5, 40, 384, 128, False, "bf16"),
                                   (1, 96, 512, 64, True, "f16")):
        codes, q, s, z = _random_w4(r, N, K, G, asym)
        xv = r.standard_normal((M, K))
        if xd == "f16":
            xb = xv.astype(np.float16)
            x64 = xb.astype(np.float64)
        else:
            xb = torch.from_numpy(xv.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            x64 = _torch_bf16_to_f64(xb)
        W = o.w4_dequant(q, s, z, G).astype(np.float64)
        ref = x64 @ W.T
        y64, _ = o.w4_matmul(xb, xd, q, s, z, G, "f16")
        err = np.max(np.abs(y64 - ref)) / np.max(np.abs(ref))
        assert err <= 1e-12, ("numpy matmul", M, N, K, G, err)


def check_one_hot(o):
    r = np.random.default_rng(22)
    N, K, G = 32, 128, 32
    codes, q, s, z = _random_w4(r, N, K, G, True)
    W = o.w4_dequant(q, s, z, G)
    for k in (0, 1, 37, 127):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        y64, yb = o.w4_matmul(x, "f16", q, s, z, G, "f16")
        assert np.array_equal(y64[0], W[:, k].astype(np.float64)), k
        assert np.array_equal(yb[0], W[:, k].astype(np.float16).view(np.uint16)), k


def check_codes_at_zero_point(o):
    r = np.random.default_rng(23)
    N, K, G = 16, 128, 32
    z = r.integers(0, 16, size=(N, K // G)).astype(np.int8)
    codes = np.repeat(z.astype(np.uint8), G, axis=1)
    s = r.uniform(0.002, 0.02, size=(N, K // G)).astype(np.float16)
    x = r.standard_normal((2, K)).astype(np.float16)
    y64, _ = o.w4_matmul(x, "f16", _pack_codes(codes), s, z, G, "f16")
    assert np.all(y64 == 0.0), "codes at the zero point must give 0 (asym)"
    codes8 = np.full((N, K), 8, np.uint8)
    y64, _ = o.w4_matmul(x, "f16", _pack_codes(codes8), s, None, G, "f16")
    assert np.all(y64 == 0.0), "code 8 must give 0 (sym)"


def check_pow2_scaling(o):
    r = np.random.default_rng(24)
    N, K, G = 24, 256, 64
    codes, q, s, z = _random_w4(r, N, K, G, True)
    x = np.clip(r.standard_normal((2, K)), -4, 4)
    x = np.where(np.abs(x) < 0.05, 0.5, x).astype(np.float16)
    y0, _ = o.w4_matmul(x, "f16", q, s, z, G, "f16")
    for j in (-3, 5):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** j)
        yj, _ = o.w4_matmul(xs, "f16", q, s, z, G, "f16")
        assert np.array_equal(yj, y0 * 2.0 ** j), j


def check_k_split(o):
    r = np.random.default_rng(25)
    N, K, G = 20, 512, 128
    codes, q, s, z = _random_w4(r, N, K, G, True)
    x = r.standard_normal((2, K)).astype(np.float16)
    y, _ = o.w4_matmul(x, "f16", q, s, z, G, "f16")
    h = 256
    y1, _ = o.w4_matmul(x[:, :h], "f16", q[:, :h // 2], s[:, :h // G], z[:, :h // G], G, "f16")
    y2, _ = o.w4_matmul(x[:, h:], "f16", q[:, h // 2:], s[:, h // G:], z[:, h // G:], G, "f16")
    assert np.max(np.abs(y - (y1 + y2))) <= 1e-12 * np.max(np.abs(y)), "K split at a group boundary"


def check_rows_subset(o):
    r = np.random.default_rng(26)
    N, K, G = 16, 256, 128
    codes, q, s, z = _random_w4(r, N, K, G, False)
    xv = r.standard_normal((9, K)).astype(np.float32)
    xb = torch.from_numpy(xv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y64, yb = o.w4_matmul(xb, "bf16", q, s, z, G, "bf16")
    rows = np.array([8, 0, 3])
    r64, rb = o.w4_matmul_rows(xb, "bf16", q, s, z, G, "bf16", rows)
    assert np.array_equal(r64, y64[rows]) and np.array_equal(rb, yb[rows])


# ------------------------------------------------------------------ b-bit codes (1..8)
def _random_wb(r, N, K, G, bits, asym):
    codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = r.uniform(0.002, 0.02, size=(N, K // G)).astype(np.float16)
    z = r.integers(-128, 128, size=(N, K // G)).astype(np.int8) if asym else None
    return codes, s, z


def check_wb_equals_w4_at_four_bits(o):
    """At 4 bits the b-bit definition is the INT4 one: dequantized weights and
    products equal the (separately pinned) W4 oracle's bit for bit, symmetric
    (z = 2^3 = 8) and asymmetric."""
    r = np.random.default_rng(61)
    for asym in (False, True):
        codes, s, z = _random_wb(r, 24, 256, 32, 4, asym)
        q = _pack_codes(codes)
        assert np.array_equal(o.wb_dequant(codes, s, z, 4, 32), o.w4_dequant(q, s, z, 32))
        x = r.standard_normal((3, 256)).astype(np.float16)
        a = o.wb_matmul(x, codes, s, z, 4, 32)
        b = o.w4_matmul(x, "f16", q, s, z, 32, "f16")
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), asym


def check_wb_dequant_closed_form(o):
    """Every code of every width against (q - z) * s in exact rationals, with
    z = 2^(b-1) (symmetric) and int8 zero points over the full range."""
    r = np.random.default_rng(62)
    for bits in range(1, 9):
        n = 1 << bits
        K = 32 * ((n + 31) // 32)
        codes = (np.arange(K) % n).astype(np.uint8)[None, :].repeat(3, axis=0)
        s = np.array([[0.01], [0.0625], [-3.5]], np.float16).repeat(K // 32, axis=1)
        for z in (None, r.integers(-128, 128, size=(3, K // 32)).astype(np.int8)):
            W = o.wb_dequant(codes, s, z, bits, 32)
            for i in range(3):
                for k in range(K):
                    zz = (1 << (bits - 1)) if z is None else int(z[i, k // 32])
                    assert F(float(W[i, k])) == (int(codes[i, k]) - zz) * F(float(s[i, k // 32])), (bits, i, k)


def check_wb_bruteforce(o):
    """b-bit products against exact rationals for several widths, group
    sizes, both zero-point forms."""
    r = np.random.default_rng(63)
    for bits, G, asym, M, N, K in ((1, 32, False, 2, 5, 64), (2, 64, True, 1, 6, 128), (3, 32, True, 3, 4, 96),
                                   (5, 128, False, 1, 3, 256), (6, 32, True, 2, 4, 64), (7, 64, False, 1, 5, 128),
                                   (8, 32, True, 2, 3, 64)):
        codes, s, z = _random_wb(r, N, K, G, bits, asym)
        x = (r.standard_normal((M, K)) * 2).astype(np.float16)
        xf = [[F(float(v)) for v in row] for row in x.astype(np.float64)]
        sf = [_frac_f16(row) for row in s.view(np.uint16)]
        y64, yb = o.wb_matmul(x, codes, s, z, bits, G)
        for m in range(M):
            for nn in range(N):
                acc, mag = F(0), F(0)
                for k in range(K):
                    zz = (1 << (bits - 1)) if z is None else int(z[nn, k // G])
                    t = xf[m][k] * (int(codes[nn, k]) - zz) * sf[nn][k // G]
                    acc += t
                    mag += abs(t)
                assert abs(F(float(y64[m, nn])) - acc) <= (K + 1) * F(1, 2 ** 53) * mag, (bits, m, nn)
                assert yb[m, nn] == _np_f16_bits([float(acc)])[0], (bits, m, nn)


def check_wb_numpy_and_special(o):
    """numpy float64 matmul of the pinned dequantized W; codes at the
    symmetric zero point give exactly 0; a one-hot x gives the weight column."""
    r = np.random.default_rng(64)
    for bits in (2, 3, 6):
        codes, s, z = _random_wb(r, 40, 384, 128, bits, True)
        x = r.standard_normal((4, 384)).astype(np.float16)
        ref = x.astype(np.float64) @ o.wb_dequant(codes, s, z, bits, 128).astype(np.float64).T
        y64, _ = o.wb_matmul(x, codes, s, z, bits, 128)
        assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.max(np.abs(ref)), bits
        mid = np.full((8, 128), 1 << (bits - 1), np.uint8)
        y64, _ = o.wb_matmul(x[:, :128], mid, s[:8, :1], None, bits, 128)
        assert np.all(y64 == 0), bits
        W = o.wb_dequant(codes, s, z, bits, 128)
        e = np.zeros((1, 384), np.float16)
        e[0, 77] = 1
        y64, yb = o.wb_matmul(e, codes, s, z, bits, 128)
        assert np.array_equal(y64[0], W[:, 77].astype(np.float64)), bits


# ------------------------------------------------------------------ W4A8: dynamic INT8 activations
def check_quant_closed_forms(o):
    """A row whose largest magnitude is 127 * 2^e makes 127 / amax = 2^-e and
    amax / 127 = 2^e exact, so each code is the nearest integer to x / 2^e,
    ties to even (Python's round), with no rounding anywhere else."""
    for e in (-4, 0, 3):
        ints = np.arange(-127, 128)
        halves = np.arange(-126, 127) + 0.5
        for vals, expect in ((ints, ints),
                             (np.append(halves, 127), np.append([round(h) for h in halves], 127))):
            x = (vals * 2.0 ** e).astype(np.float16)
            assert np.array_equal(x.astype(np.float64), vals * 2.0 ** e)
            xq, sx = o.quant_act_i8(x[None, :])
            assert float(sx[0]) == 2.0 ** e, e
            assert np.array_equal(xq[0].astype(np.int64), np.asarray(expect, np.int64)), e


def check_quant_properties(o):
    """Invariants of per-token symmetric quantization on rows of very
    different magnitudes: scale = amax / 127 to one binary32 rounding, the
    largest magnitude maps to +-127, codes keep the sign and order of x and
    lie within half a step (plus the binary32 roundings) of x / s; rows are
    quantized independently; scaling a row by 2^j scales s by 2^j and keeps
    the codes; a zero row gives s = 0 and zero codes."""
    r = np.random.default_rng(31)
    mags = np.array([[0.01], [1.0], [30.0], [1000.0], [1e-3], [3.0]])
    x = (r.standard_normal((6, 384)) * mags).astype(np.float16)
    x[5, 17] = -np.float16(40.0)                     # a negative row maximum
    xq, sx = o.quant_act_i8(x)
    xd = x.astype(np.float64)
    for m in range(x.shape[0]):
        amax = np.max(np.abs(xd[m]))
        s = float(sx[m])
        assert abs(s - amax / 127) <= 2.0 ** -23 * amax / 127, m
        k = int(np.argmax(np.abs(xd[m])))
        assert int(xq[m, k]) == (127 if xd[m, k] > 0 else -127), m
        q = xq[m].astype(np.int64)
        assert np.all(np.abs(q) <= 127)
        assert np.all(np.sign(q) * np.sign(xd[m]) >= 0), m
        order = np.argsort(xd[m], kind="stable")
        assert np.all(np.diff(q[order]) >= 0), m
        assert np.all(np.abs(xd[m] - s * q) <= s * (0.5 + 3e-5)), m
    for m in range(x.shape[0]):
        q1, s1 = o.quant_act_i8(x[m:m + 1])
        assert np.array_equal(q1[0], xq[m]) and s1[0] == sx[m], m
    for j in (-2, 3):
        xs = (xd[1:3] * 2.0 ** j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64), xd[1:3] * 2.0 ** j)
        qj, sj = o.quant_act_i8(xs)
        assert np.array_equal(qj, xq[1:3]) and np.array_equal(sj.astype(np.float64), sx[1:3].astype(np.float64) * 2.0 ** j)
    qz, sz = o.quant_act_i8(np.zeros((2, 64), np.float16))
    assert np.all(qz == 0) and np.all(sz == 0)


def _check_w4a8_bruteforce_case(o, M, N, K, G, asym, seed):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = r.uniform(0.002, 0.05, size=(N, K // G)).astype(np.float16)
    z = r.integers(-128, 128, size=(N, K // G)).astype(np.int8) if asym else None
    x = (r.standard_normal((M, K)) * 2).astype(np.float16)
    xq, sx = o.quant_act_i8(x)
    sf = [_frac_f16(row) for row in s.view(np.uint16)]
    xf = [[F(float(sx[m])) * int(v) for v in xq[m]] for m in range(M)]
    exact = _exact_matmul(xf, codes, z, sf, G)
    y64, yb = o.w4a8_matmul(x, _pack_codes(codes), s, z, G)
    for m in range(M):
        for n in range(N):
            e, mag = exact[m][n]
            assert abs(F(float(y64[m, n])) - e) <= (K + 1) * F(1, 2 ** 53) * mag, ("sum", M, N, K, G, m, n)
            assert yb[m, n] == _np_f16_bits([float(e)])[0], ("rounding", M, N, K, G, m, n)


def check_w4a8_bruteforce(o):
    """The W4A8 product of the oracle's (separately pinned) INT8 codes and
    scales against exact rationals."""
    _check_w4a8_bruteforce_case(o, 1, 5, 64, 32, False, 41)
    _check_w4a8_bruteforce_case(o, 3, 6, 128, 32, True, 42)
    _check_w4a8_bruteforce_case(o, 2, 4, 256, 128, True, 43)
    _check_w4a8_bruteforce_case(o, 4, 3, 192, 64, False, 44)


def check_w4a8_numpy(o):
    """W4A8 product == numpy float64 matmul of the dequantized activations
    (s * codes) and the (pinned) dequantized weights."""
    r = np.random.default_rng(45)
    for (M, N, K, G, asym) in ((1, 64, 512, 32, True), (8, 40, 384, 128, False), (3, 24, 256, 64, True)):
        codes, q, s, z = _random_w4(r, N, K, G, asym)
        x = r.standard_normal((M, K)).astype(np.float16)
        xq, sx = o.quant_act_i8(x)
        ref = (sx.astype(np.float64)[:, None] * xq.astype(np.float64)) @ o.w4_dequant(q, s, z, G).astype(np.float64).T
        y64, _ = o.w4a8_matmul(x, q, s, z, G)
        err = np.max(np.abs(y64 - ref)) / np.max(np.abs(ref))
        assert err <= 1e-12, ("numpy", M, N, K, G, err)


def check_w4a8_on_grid_equals_w4a16(o):
    """Activations already on their quantization grid (row maximum 127 * 2^e,
    every value a multiple of 2^e) dequantize to themselves, so the W4A8
    product equals the W4A16 product bit for bit."""
    r = np.random.default_rng(46)
    N, K, G = 24, 256, 32
    codes, q, s, z = _random_w4(r, N, K, G, True)
    for e in (-5, -1):
        j = r.integers(-127, 128, size=(2, K))
        j[:, 7] = (127, -127)
        x = (j * 2.0 ** e).astype(np.float16)
        y8, b8 = o.w4a8_matmul(x, q, s, z, G)
        y16, b16 = o.w4_matmul(x, "f16", q, s, z, G, "f16")
        assert np.array_equal(y8, y16) and np.array_equal(b8, b16), e


def check_w4a8_special(o):
    """x = 127 e_k: scale 1, code 127 at k, so y = RNE_fp16(127 w[:, k]);
    codes at the zero point give 0; a zero activation row gives 0."""
    r = np.random.default_rng(47)
    N, K, G = 32, 128, 32
    codes, q, s, z = _random_w4(r, N, K, G, True)
    W = o.w4_dequant(q, s, z, G).astype(np.float64)
    for k in (0, 5, 127):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 127
        y64, yb = o.w4a8_matmul(x, q, s, z, G)
        assert np.array_equal(y64[0], 127 * W[:, k]), k
        assert np.array_equal(yb[0], _np_f16_bits(127 * W[:, k])), k
    zc = np.repeat(z.astype(np.uint8), G, axis=1)
    x = r.standard_normal((2, K)).astype(np.float16)
    y64, _ = o.w4a8_matmul(x, _pack_codes(zc), s, z, G)
    assert np.all(y64 == 0.0)
    x[1] = 0
    y64, yb = o.w4a8_matmul(x, q, s, z, G)
    assert np.all(y64[1] == 0.0) and np.all(yb[1] == 0)


# ------------------------------------------------------------------ LUT3 / MXFP8 / MoE
def check_lut3_hand(o):
    g = _golden("lut3_hand_example.json")
    b = np.array([_hex(k) for k in g["e4m3"]], np.uint8)
    got = o.e4m3_to_double(b)
    assert [F(float(v)) for v in got] == [F(v) for v in g["e4m3"].values()], "E4M3 hand values"
    E, N, K = 1, 8, 64
    cb = np.zeros((E, N // 8, K // 64, 8), np.uint8)
    cb[0, 0, 0, :] = [_hex(c) for c in g["codebook"]]
    ex = np.full((E, N // 8, K // 64), g["tile_exponent"], np.uint8)
    idx = np.full((E, N, K), 4, np.uint8)
    idx[0, 0, :8] = np.arange(8)
    w = o.lut3_dequant(idx, cb, ex)
    want = [F(g["decoded_weights"][str(i)]) for i in range(8)]
    assert [F(float(v)) for v in w[0, 0, :8]] == want, "decoded codebook entries"
    # the dot product of the worked example
    idx2 = np.full((E, N, K), 4, np.uint8)
    idx2[0, 0, 0], idx2[0, 0, 1] = 2, 6
    aq = np.zeros((1, K), np.uint8)
    aq[0, 0], aq[0, 1] = [_hex(v) for v in g["activation"]["bytes"]]
    as_ = np.array([[g["activation"]["block_scale"], 127]], np.uint8)
    y64, ob = o.moe_gemm(idx2, cb, ex, aq, as_, 1, np.array([[0]], np.int32))
    assert F(float(y64[0, 0])) == F(g["dot"]["y_exact"]), "worked dot product"
    want_bits = torch.tensor([float(F(g["dot"]["y_bf16_rne"]))], dtype=torch.float32) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
    assert ob[0, 0] == want_bits, "worked dot product, bf16"


def _lut_fracs(idx, cb, ex):
    """Exact rational decoded weights via torch E4M3 decode and 2^(e-127)."""
    E, N, K = idx.shape
    cbv = _torch_e4m3_to_f64(cb.ravel()).reshape(cb.shape)
    out = np.empty((E, N, K), dtype=object)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                out[e, n, k] = F(float(cbv[e, n // 8, k // 64, idx[e, n, k]])) * F(2) ** (int(ex[e, n // 8, k // 64]) - 127)
    return out


def check_lut3_bruteforce(o):
    d = synth.lut3_weights(3, 16, 128, workload_id=90)
    want = _lut_fracs(d["idx"], d["cb"], d["ex"])
    got = o.lut3_dequant(d["idx"], d["cb"], d["ex"])
    assert all(F(float(g)) == w for g, w in zip(got.ravel(), want.ravel())), "LUT3 decode"


def _moe_exact(o, d, aq, as_, a_row_div, topk, emap):
    E, N, K = d["idx"].shape
    W = _lut_fracs(d["idx"], d["cb"], d["ex"])
    av = _torch_e4m3_to_f64(aq.ravel()).reshape(aq.shape)
    T, top_k = topk.shape
    y64, ob = o.moe_gemm(d["idx"], d["cb"], d["ex"], aq, as_, a_row_div, topk, emap)
    for sid in range(T * top_k):
        g = int(topk.ravel()[sid])
        e = g if emap is None else int(emap[g])
        row = sid // a_row_div
        a = [F(float(av[row, k])) * F(2) ** (int(as_[row, k // 32]) - 127) for k in range(K)]
        for n in range(N):
            if e < 0:
                assert y64[sid, n] == 0.0 and ob[sid, n] == 0, ("EP zero", sid, n)
                continue
            terms = [a[k] * W[e, n, k] for k in range(K)]
            ex_ = sum(terms, F(0))
            mag = sum((abs(t) for t in terms), F(0))
            assert abs(F(float(y64[sid, n])) - ex_) <= (K + 1) * F(1, 2 ** 53) * mag, ("moe sum", sid, n)
            assert ob[sid, n] == o.double_to_bf16(np.array([float(ex_)]))[0], ("moe bf16", sid, n)


def check_moe_bruteforce(o):
    E, T, top_k, N, K = 4, 3, 2, 8, 64
    d = synth.lut3_weights(E, N, K, workload_id=91)
    topk = synth.moe_routing(T, E, top_k, workload_id=91)
    emap = np.array([0, 1, -1, 2], np.int32)                  # expert 2 not local
    d_local = dict(idx=d["idx"][[0, 1, 3]], cb=d["cb"][[0, 1, 3]], ex=d["ex"][[0, 1, 3]])
    aq, as_ = synth.mxfp8_activations(T, K, workload_id=91)    # gate/up style: row = token
    _moe_exact(o, d_local, aq, as_, top_k, topk, emap)
    aq2, as2 = synth.mxfp8_activations(T * top_k, K, workload_id=92)  # down style: row = slot
    _moe_exact(o, d, aq2, as2, 1, topk, None)


def check_moe_numpy(o):
    E, T, top_k, N, K = 8, 16, 2, 32, 256
    d = synth.lut3_weights(E, N, K, workload_id=93)
    topk = synth.moe_routing(T, E, top_k, workload_id=93)
    aq, as_ = synth.mxfp8_activations(T, K, workload_id=93)
    W = o.lut3_dequant(d["idx"], d["cb"], d["ex"])
    a = _torch_e4m3_to_f64(aq.ravel()).reshape(T, K) * np.exp2(np.repeat(as_.astype(np.float64) - 127, 32, axis=1))
    y64, _ = o.moe_gemm(d["idx"], d["cb"], d["ex"], aq, as_, top_k, topk)
    for sid in range(T * top_k):
        ref = W[topk.ravel()[sid]] @ a[sid // top_k]
        err = np.max(np.abs(y64[sid] - ref)) / max(np.max(np.abs(ref)), 1e-300)
        assert err <= 1e-12, ("moe numpy", sid, err)


def check_moe_align(o):
    r = np.random.default_rng(31)
    for (T, E, top_k, bm, use_map) in ((64, 16, 4, 16, False), (37, 12, 3, 32, True), (5, 64, 8, 16, True)):
        topk = np.stack([r.choice(E, size=top_k, replace=False) for _ in range(T)]).astype(np.int32)
        emap = None
        if use_map:
            emap = np.full(E, -1, np.int32)
            loc = np.sort(r.choice(E, size=E // 3, replace=False))
            emap[loc] = np.arange(loc.size, dtype=np.int32)
        ids, blk, P = o.moe_align(topk, E, bm, emap)
        nv = T * top_k
        flat = topk.ravel()
        assert P % bm == 0 and ids.size == P and blk.size == P // bm
        counts = np.bincount(flat, minlength=E)
        assert P == int(np.sum((counts + bm - 1) // bm * bm)), "padded length"
        assert sorted(ids[ids < nv].tolist()) == list(range(nv)), "every slot exactly once"
        assert np.all((ids <= nv) & (ids >= 0)), "ids are slots or the sentinel"
        pos = 0
        for e in range(E):
            c = int(counts[e])
            if c == 0:
                continue
            seg = ids[pos:pos + (c + bm - 1) // bm * bm]
            assert np.all(seg[:c] < nv) and np.all(flat[seg[:c]] == e), ("expert segment", e)
            assert np.all(np.diff(seg[:c]) > 0), ("ascending within expert", e)
            assert np.all(seg[c:] == nv), ("sentinel padding", e)
            want = e if emap is None else int(emap[e])
            assert np.all(blk[pos // bm:(pos + seg.size) // bm] == want), ("block expert", e)
            pos += seg.size
        assert pos == P


# ------------------------------------------------------------------ MoE layer: SiLU * up, MXFP8, combine
def _torch_to_e4m3(v):
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _torch_to_bf16_bits(v):
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def check_e4m3_encode(o):
    """Every finite E4M3 value encodes to its own byte; values between
    neighbours round to nearest even as torch's float8_e4m3fn conversion does;
    magnitudes above 448 saturate to 448 (0x7E); the hand bytes of the page
    notes (0x38 = 1, 0x40 = 2, 0xC4 = -3, 0x7E = 448, 0x01 = 2^-9)."""
    b = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    vals = _torch_e4m3_to_f64(b)
    assert np.array_equal(o.double_to_e4m3(vals), b)
    r = np.random.default_rng(51)
    v = np.concatenate([r.uniform(-448, 448, 4000), r.uniform(-0.02, 0.02, 2000),
                        (vals[:-1] + vals[1:]) / 2])                       # midpoints: ties
    v = v[np.abs(v) <= 448].astype(np.float32).astype(np.float64)
    assert np.array_equal(o.double_to_e4m3(v), _torch_to_e4m3(v))
    assert np.all(o.double_to_e4m3(np.array([448.5, 464.0, 479.9, 480, 1e6])) == 0x7E)
    assert np.all(o.double_to_e4m3(np.array([-500.0, -1e9])) == 0xFE)
    assert o.double_to_e4m3(np.array([1.0, 2.0, -3.0, 448.0, 2.0 ** -9])).tolist() == [0x38, 0x40, 0xC4, 0x7E, 0x01]


def check_mxfp8_quant(o):
    """MXFP8 of bf16 rows: a block of E4M3 values times 2^j whose largest
    magnitude lies in [256, 448] keeps its bytes exactly with exponent byte
    127 + j; random blocks decode to within half an E4M3 step of x (largest
    element saturated at 448 * 2^e at most); the largest magnitude lands in
    [256, 448] after scaling; a zero block gets byte 127 and zero codes;
    blocks are independent."""
    r = np.random.default_rng(52)
    good = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], np.uint8)
    gv = _torch_e4m3_to_f64(good)
    for j in (-20, -3, 0, 5):
        codes = r.choice(good, size=(3, 64))
        codes[:, 0] = 0x7E                                     # 448 in every block of row 0..2
        codes[:, 32] = 0xF8                                    # -256 in the second block
        x = _torch_e4m3_to_f64(codes) * 2.0 ** j
        xb = _torch_to_bf16_bits(x)
        assert np.array_equal(o.bf16_to_double(xb).reshape(x.shape), x)   # exact in bf16
        q, sc = o.mxfp8_quant(xb)
        assert np.array_equal(sc, np.full((3, 2), 127 + j, np.uint8)), j
        assert np.array_equal(q, codes), j
    x = r.standard_normal((5, 128)) * np.array([[1e-3], [1.0], [30.0], [1e4], [1.0]])
    x[4, 32:64] = 0.0
    xb = _torch_to_bf16_bits(x)
    xd = o.bf16_to_double(xb).reshape(x.shape)
    q, sc = o.mxfp8_quant(xb)
    assert sc[4, 1] == 127 and np.all(q[4, 32:64] == 0)
    dec = _torch_e4m3_to_f64(q) * np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
    blocks = np.abs(xd).reshape(5, 4, 32)
    amax = blocks.max(axis=2)
    scaled_max = (amax / np.ldexp(1.0, sc.astype(np.int64) - 127))[amax > 0]
    assert np.all((scaled_max >= 256) & (scaled_max < 512))
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(xd), 1e-300))).astype(np.int64) - 3)
    sub = np.ldexp(1.0, sc.astype(np.int64) - 127 - 9).repeat(32, axis=1)           # E4M3 subnormal step
    cap = 448 * np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
    err = np.abs(dec - np.clip(xd, -cap, cap))
    assert np.all(err <= np.maximum(step, sub) / 2 * (1 + 1e-12))
    for rr in range(5):
        q1, s1 = o.mxfp8_quant(xb[rr:rr + 1])
        assert np.array_equal(q1[0], q[rr]) and np.array_equal(s1[0], sc[rr])


def check_silu(o):
    """The stated 2^t routine is exact at integers and within 1 ulp of 2^t;
    SiLU is within (4 + |t| ln2) binary32 ulp of g / (1 + e^-g) (libm,
    double), t = g log2(e) -- rounding log2(e) and then t to binary32 moves
    the exponent by up to 2 |t| 2^-24 -- and exactly 0 at 0; SiLU(g) * up rounds to the bf16
    nearest the double product except where binary32 rounding decides a near
    tie (at most 1 bf16 ulp away)."""
    import math
    k = np.arange(-100, 101).astype(np.float32)
    assert np.array_equal(o.exp2_f32(k).astype(np.float64), 2.0 ** k.astype(np.float64))
    t = np.linspace(-99.5, 99.5, 200001).astype(np.float32)
    ref = np.exp2(t.astype(np.float64))
    e = o.exp2_f32(t).astype(np.float64)
    assert np.all(np.abs(e - ref) <= ref * 2.0 ** -23)
    g = np.concatenate([np.linspace(-60, 60, 100001), [0.0]]).astype(np.float32)
    gd = g.astype(np.float64)
    ref = np.array([v / (1.0 + math.exp(-v)) for v in gd])
    sv = o.silu_f32(g).astype(np.float64)
    mask = np.abs(ref) > 1e-30
    ulps = 4 + np.abs(gd) * np.log2(np.e) * np.log(2)
    assert np.all((np.abs(sv - ref) <= ulps * np.abs(ref) * 2.0 ** -23)[mask])
    assert sv[-1] == 0.0
    r = np.random.default_rng(53)
    gu = _torch_to_bf16_bits(r.standard_normal((64, 256)) * 3)
    act = o.silu_mul_bf16(gu)
    gud = o.bf16_to_double(gu).reshape(64, 256)
    exact = np.array([[gud[i, j] / (1 + math.exp(-gud[i, j])) * gud[i, 128 + j] for j in range(128)] for i in range(64)])
    ref_bits = o.double_to_bf16(exact.ravel()).reshape(64, 128)
    same = act == ref_bits
    assert same.mean() > 0.995
    ad = o.bf16_to_double(act).reshape(64, 128)
    rd = o.bf16_to_double(ref_bits).reshape(64, 128)
    assert np.all(np.abs(ad - rd)[~same] <= np.abs(rd[~same]) * 2.0 ** -7)
    # gate is the first half: gate = 20 gives SiLU ~ 20, gate = -20 gives ~ 0
    u = r.standard_normal(128)
    for gate, factor in ((20.0, 20.0), (-20.0, 0.0)):
        gu2 = _torch_to_bf16_bits(np.concatenate([np.full(128, gate), u])[None, :])
        a2 = o.bf16_to_double(o.silu_mul_bf16(gu2)).ravel()
        ud = o.bf16_to_double(gu2).ravel()[128:]
        assert np.allclose(a2, factor * ud, rtol=1e-2, atol=1e-6), gate


def check_moe_combine(o):
    """Combine: one-hot router weights return the chosen slot's row exactly;
    general weights equal a numpy float64 weighted sum; a slot with a zero
    row adds nothing."""
    r = np.random.default_rng(54)
    T, k, H = 7, 4, 96
    out = _torch_to_bf16_bits(r.standard_normal((T * k, H)))
    od = o.bf16_to_double(out).reshape(T * k, H)
    w = np.zeros((T, k), np.float32)
    pick = r.integers(0, k, T)
    w[np.arange(T), pick] = 1.0
    y64, yb = o.moe_combine(out, w, k)
    assert np.array_equal(yb, out[np.arange(T) * k + pick])
    w = r.dirichlet(np.ones(k), T).astype(np.float32)
    y64, yb = o.moe_combine(out, w, k)
    ref = np.einsum("tj,tjh->th", w.astype(np.float64), od.reshape(T, k, H))
    assert np.max(np.abs(y64 - ref)) <= 1e-15 * np.max(np.abs(ref))
    out2 = out.copy()
    out2[3 * k + 1] = 0
    y2, _ = o.moe_combine(out2, w, k)
    ref2 = ref.copy()
    ref2[3] -= w[3, 1] * od[3 * k + 1]
    assert np.max(np.abs(y2 - ref2)) <= 1e-15 * np.max(np.abs(ref))


def _tiny_moe(seed, T=5, E=4, top_k=2, H=64, I=64):
    d13 = synth.lut3_weights(E, 2 * I, H, workload_id=90, layer=seed, part=0)
    d2 = synth.lut3_weights(E, H, I, workload_id=90, layer=seed, part=1)
    r = np.random.default_rng(seed)
    x = _torch_to_bf16_bits(r.standard_normal((T, H)))
    topk = np.stack([r.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.dirichlet(np.ones(top_k), T).astype(np.float32)
    return d13, d2, x, topk, w


def check_moe_layer_wiring(o):
    """The layer's composition: every expert non-local gives y = 0; one-hot
    router weights give the chosen slot's down row; permuting tokens permutes
    the output rows bit for bit; a token routed twice to one expert gets
    (w1 + w2) times that expert's row."""
    d13, d2, x, topk, w = _tiny_moe(55)
    T, top_k = topk.shape
    res = o.moe_layer(d13, d2, x, topk, w, expert_map=np.full(4, -1, np.int32))
    assert np.all(res["y64"] == 0)
    w1 = np.zeros_like(w)
    w1[:, 1] = 1.0
    res = o.moe_layer(d13, d2, x, topk, w1)
    assert np.array_equal(res["y"], res["down"][np.arange(T) * top_k + 1])
    perm = np.array([3, 0, 4, 2, 1])
    a = o.moe_layer(d13, d2, x, topk, w)
    b = o.moe_layer(d13, d2, x[perm], topk[perm], w[perm])
    assert np.array_equal(b["y64"], a["y64"][perm]) and np.array_equal(b["y"], a["y"][perm])
    t2 = topk.copy()
    t2[:, 1] = t2[:, 0]
    c = o.moe_layer(d13, d2, x, t2, w)
    row = o.bf16_to_double(c["down"]).reshape(T * top_k, -1)[np.arange(T) * top_k]
    assert np.array_equal(c["y64"], (w[:, 0].astype(np.float64) + w[:, 1])[:, None] * row)


ALL_CHECKS = [
    check_f16_decode, check_f16_encode, check_bf16_decode, check_bf16_encode,
    check_e4m3_decode, check_ue8m0_decode,
    check_hand_bytes, check_sixteen_codes, check_dequant_exact_all_scales, check_fp16_tie, check_gemv_2x4,
    check_bruteforce_tiny, check_bruteforce_tiny_gemv_workload, check_numpy_matmul, check_one_hot,
    check_codes_at_zero_point, check_pow2_scaling, check_k_split, check_rows_subset,
    check_wb_equals_w4_at_four_bits, check_wb_dequant_closed_form, check_wb_bruteforce, check_wb_numpy_and_special,
    check_quant_closed_forms, check_quant_properties, check_w4a8_bruteforce, check_w4a8_numpy,
    check_w4a8_on_grid_equals_w4a16, check_w4a8_special,
    check_lut3_hand, check_lut3_bruteforce, check_moe_bruteforce, check_moe_numpy, check_moe_align,
    check_e4m3_encode, check_mxfp8_quant, check_silu, check_moe_combine, check_moe_layer_wiring,
]
