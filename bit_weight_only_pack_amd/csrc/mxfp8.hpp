// mxfp8.hpp -- the MoE layer's element operations, shared by the stand-alone
// kernels and the gate/up GEMM's fused epilogue so both give the same bytes
// ("vLLM PR #62759 analysis", section "Emulation path": activations are
// quantized to MXFP8 before each expert GEMM; OCP MX: one UE8M0 scale per 32
// consecutive elements, elements in E4M3).
//   * act = RNE_bf16(fl32(SiLU(gate) * up)), SiLU(g) = g / (1 + e^-g) with
//     e^-g = 2^t, t = fl32(-g * fl32(log2 e)), by the stated binary32 routine
//     exp2_f32 below.
//   * MXFP8: per 32-block e = floor(log2 amax) - 8 clamped to [-127, 127] (0 for
//     a zero block), scale byte e + 127, elements = saturating RNE E4M3 of
//     x / 2^e.
#pragma once
#include "lowbit_internal.hpp"

namespace lowbit {
namespace mx {

typedef uint16_t us8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// binary32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// 2^t in binary32: n = rint(t), f = t - n (exact), Taylor polynomial of
// e^(f ln2) through degree 7 in Horner form with fused multiply-adds,
// coefficients (ln 2)^k / k! rounded to binary32, scaled by 2^n; t clamped to
// [-100, 100] so the result stays a normal number.
__device__ __forceinline__ float exp2_f32(float t)
{
    t = __builtin_fminf(__builtin_fmaxf(t, -100.f), 100.f);
    const float n = __builtin_rintf(t);
    const float f = t - n;
    // (ln 2)^k / k! formed in double as term_k = term_{k-1} * ln2 / k (the
    // sequence of roundings the definition uses), then rounded to binary32
    constexpr double kLn2 = 0.693147180559945309417232121458;
    constexpr double t1 = 1.0 * kLn2 / 1.0, t2 = t1 * kLn2 / 2.0, t3 = t2 * kLn2 / 3.0, t4 = t3 * kLn2 / 4.0;
    constexpr double t5 = t4 * kLn2 / 5.0, t6 = t5 * kLn2 / 6.0, t7 = t6 * kLn2 / 7.0;
    constexpr float c0 = 1.0f, c1 = (float)t1, c2 = (float)t2, c3 = (float)t3, c4 = (float)t4, c5 = (float)t5;
    constexpr float c6 = (float)t6, c7 = (float)t7;
    float p = c7;
    p = __builtin_fmaf(p, f, c6);
    p = __builtin_fmaf(p, f, c5);
    p = __builtin_fmaf(p, f, c4);
    p = __builtin_fmaf(p, f, c3);
    p = __builtin_fmaf(p, f, c2);
    p = __builtin_fmaf(p, f, c1);
    p = __builtin_fmaf(p, f, c0);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float silu_f32(float g)
{
    constexpr float kLog2e = 1.44269504088896340736f;
    float t = -g * kLog2e;
    asm volatile("" : "+v"(t));                      // t is rounded on its own (no fused multiply-add)
    const float e = exp2_f32(t);
    float d = 1.0f + e;
    asm volatile("" : "+v"(d));
    return g * __fdiv_rn(1.0f, d);
}

// |v| <= 448 (already clipped), finite -> E4M3 byte, round to nearest even
__device__ __forceinline__ uint32_t e4m3_byte(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x3C800000u) {                           // below 2^-6: multiples of 2^-9, 0..8
        code = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    } else {                                         // keep 3 fraction bits, nearest even, rebias 127 -> 7
        code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    }
    return sign | code;
}

// Quantize 8 consecutive values of a row (one lane) that belong to a 32-block
// held by the lane's quad; writes 8 codes and (first lane of the quad) the
// block's scale byte.
__device__ __forceinline__ void mx_block_put(const float *v, uint8_t *q, uint8_t *scale, bool write_scale)
{
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    int ab = __builtin_bit_cast(int, amax);          // non-negative floats order as integers
    ab = max(ab, __builtin_amdgcn_mov_dpp(ab, 0xB1, 0xF, 0xF, false));
    ab = max(ab, __builtin_amdgcn_mov_dpp(ab, 0x4E, 0xF, 0xF, false));
    amax = __builtin_bit_cast(float, ab);
    int e = 0;
    if (amax > 0.f) {
        e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;   // floor(log2 amax) - 8
        e = min(max(e, -127), 127);
    }
    uint32_t d[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float s = __builtin_ldexpf(v[i], -e);
        s = __builtin_fminf(__builtin_fmaxf(s, -448.f), 448.f);
        d[i / 4] |= e4m3_byte(s) << (8 * (i % 4));
    }
    *reinterpret_cast<uint2 *>(q) = make_uint2(d[0], d[1]);
    if (write_scale) *scale = (uint8_t)(e + 127);
}

}  // namespace mx
}  // namespace lowbit
