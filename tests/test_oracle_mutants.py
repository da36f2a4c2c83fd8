"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and require that at least one pin fails.  This shows the pins constrain every
part of the oracle: format decodes, nibble order, zero point, sign, indexing,
dropped terms, transposed operands, rounding, the LUT decode and the routing
bookkeeping.  Every mutation keeps all memory accesses in bounds."""
import pytest

import oracle
from oracle_pins import ALL_CHECKS

MATMUL_LOOP = ("            for (int64_t k = 0; k < K; ++k) {\n"
               "                uint8_t byte = qweight[n * (K / 2) + k / 2];\n"
               "                int q = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);\n"
               "                int z = w4_zero(zeros, n, k, K, G);\n"
               "                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n"
               "                double w = (double)(float)")

MUTANTS = [
    ("nibble order swapped", "(k % 2 == 0) ?", "(k % 2 == 1) ?"),
    ("symmetric zero point 7", "if (zeros == NULL) return 8;", "if (zeros == NULL) return 7;"),
    ("sign of (q - z) flipped", "(double)(q - z) * s", "(double)(z - q) * s"),
    ("first K term dropped", MATMUL_LOOP, MATMUL_LOOP.replace("int64_t k = 0;", "int64_t k = 1;")),
    ("scale index transposed", "double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n                double w",
     "double s = orc_f16_to_double(scales[(k / G) * N + n]);\n                double w"),
    ("activation index transposed", "act_value(x, x_dtype, m * K + k)", "act_value(x, x_dtype, k * M + m)"),
    ("accumulator in float", "            double acc = 0.0;\n            for (int64_t k = 0; k < K; ++k) {\n                uint8_t",
     "            float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k) {\n                uint8_t"),
    ("fp16 exponent bias", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("fp16 subnormal scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("bf16 decode bias", "ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    ("ties away from zero", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("bf16 encode exponent", "((E + 127) << 7)", "((E + 126) << 7)"),
    ("fp16 overflow saturates", "if (isinf(r)) return sign | 0x7c00;", "if (isinf(r)) return sign | 0x7bff;"),
    ("b-bit symmetric zero point 2^b", "if (zeros == NULL) return 1 << (bits - 1);", "if (zeros == NULL) return 1 << bits;"),
    ("b-bit code index transposed", "            int q = codes[n * K + k];\n            int z = wb_zero(zeros, bits, n, k, K, G);\n            double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n            w_out",
     "            int q = codes[k * N + n];\n            int z = wb_zero(zeros, bits, n, k, K, G);\n            double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n            w_out"),
    ("b-bit product uses the zero point of group 0", "                int z = wb_zero(zeros, bits, n, k, K, G);\n                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n                acc +=",
     "                int z = wb_zero(zeros, bits, n, 0, K, G);\n                double s = orc_f16_to_double(scales[n * (K / G) + k / G]);\n                acc +="),
    ("activation codes scaled to 128", "127.0f / amax", "128.0f / amax"),
    ("activation ties away from zero", "float r = rintf(t);", "float r = roundf(t);"),
    ("activation codes truncated", "float r = rintf(t);", "float r = truncf(t);"),
    ("activation maximum over a column", "fabsf((float)orc_f16_to_double(x[m * K + k]))",
     "fabsf((float)orc_f16_to_double(x[k * M + m]))"),
    ("activation maximum without magnitude", "float v = fabsf((float)orc_f16_to_double(x[m * K + k]));",
     "float v = (float)orc_f16_to_double(x[m * K + k]);"),
    ("activation scale dropped", "double a = (double)sx[m] * (double)xq[m * K + k];",
     "double a = (double)xq[m * K + k];"),
    ("activation scale of row 0", "double a = (double)sx[m] * (double)xq[m * K + k];",
     "double a = (double)sx[0] * (double)xq[m * K + k];"),
    ("dequantization scale amax / 128", "sx[m] = amax / 127.0f;", "sx[m] = amax / 128.0f;"),
    ("SiLU of -g", "float t = -g * LOG2E;", "float t = g * LOG2E;"),
    ("exp polynomial one degree short", "for (int k = 6; k >= 0; --k) p = fmaf(p, f, c[k]);",
     "for (int k = 5; k >= 0; --k) p = fmaf(p, f, c[k]);"),
    ("gate and up swapped", "float g = (float)orc_bf16_to_double(gu[r * 2 * I + j]);",
     "float g = (float)orc_bf16_to_double(gu[r * 2 * I + I + j]);"),
    ("MXFP8 exponent offset 7", "e = (ex - 1) - 8;", "e = (ex - 1) - 7;"),
    ("E4M3 encode saturates to NaN", "if (isinf(r)) r = 448.0;", "if (isinf(r)) r = 480.0;"),
    ("zero block exponent", "            int e = 0;\n            if (amax > 0.0) {", "            int e = -127;\n            if (amax > 0.0) {"),
    ("combine weight of slot 0", "acc += (double)w[t * top_k + j] *", "acc += (double)w[t * top_k] *"),
    ("combine row order", "orc_bf16_to_double(out[(t * top_k + j) * H + h])", "orc_bf16_to_double(out[(j * T + t) * H + h])"),
    ("E4M3 subnormal", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("E4M3 bias", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    ("E4M3 NaN treated as a number", "if (e == 15 && m == 7)\n        return NAN;", "if (e == 16)\n        return NAN;"),
    ("UE8M0 bias", "ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)"),
    ("codebook read backwards", "cb[tile * 8 + i]", "cb[tile * 8 + (7 - i)]"),
    ("one tile exponent for all", "orc_ue8m0_to_double(ex[tile])", "orc_ue8m0_to_double(ex[0])"),
    ("codebook shared by 16 channels", "(e * (N / 8) + n / 8) * tiles_k", "(e * (N / 8) + n / 16) * tiles_k"),
    ("activation scale per 64 K", "as[r * (K / 32) + k / 32]", "as[r * (K / 32) + k / 64]"),
    ("expert map ignored", "int32_t e = expert_map ? expert_map[g] : g;", "int32_t e = g;"),
    ("row of a slot", "int64_t r = sid / a_row_div;", "int64_t r = sid % a_row_div;"),
    ("padding sentinel", "sorted_ids[pos + i] = (int32_t)num_valid;", "sorted_ids[pos + i] = (int32_t)(num_valid - 1);"),
    ("experts visited descending", "for (int64_t e = 0; e < E; ++e) {\n        int64_t count = 0;",
     "for (int64_t e = E - 1; e >= 0; --e) {\n        int64_t count = 0;"),
    ("no padding to block_m", "int64_t padded = ((count + block_m - 1) / block_m) * block_m;",
     "int64_t padded = count;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert old in src, "mutation anchor not found: " + name
    mutant = oracle.build_variant(src.replace(old, new), str(tmp_path / "mutant.so"))
    failures = []
    for check in ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failures.append(check.__name__)
            break
    assert failures, "no pin catches: " + name
