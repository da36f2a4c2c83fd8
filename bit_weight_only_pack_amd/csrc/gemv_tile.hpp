// gemv_tile.hpp -- device helpers shared by the W4 GEMV kernels: in-register
// nibble unpack, per-tile group metadata, and the MFMA product of one packed
// 1 KiB tile (16 weight rows x 128 K) with up to 16 activation rows.
#pragma once

#include "lowbit_internal.hpp"

namespace lowbit {
namespace tile {

template <typename T>
__device__ __forceinline__ T bitcast(uint32_t v) { return __builtin_bit_cast(T, v); }

// Cross-wave sum of a workgroup's per-wave partials (W <= 16 waves along K).
// Every partial has one of kRedSlots slots per value; wave w writes slot w,
// and slots W .. 15 hold +0 (written by the waves too), so the summing wave
// reads all sixteen with fixed offsets and adds them as a balanced tree:
// ((s0 + s1) + (s2 + s3)) + ...  The order is fixed, so the result is
// deterministic, and it does not branch on W.
constexpr int kRedSlots = 16;

// writes this wave's partial v into slot `wave` of the value at `base`
// (stride: floats between slots) and +0 into its share of slots W .. 15
__device__ __forceinline__ void red_put(float *base, int stride, int wave, int W, float v)
{
    base[wave * stride] = v;
    for (int w = wave + W; w < kRedSlots; w += W) base[w * stride] = 0.f;
}
__device__ __forceinline__ float red_sum(const float *base, int stride)
{
    float v[kRedSlots];
#pragma unroll
    for (int w = 0; w < kRedSlots; ++w) v[w] = base[w * stride];
#pragma unroll
    for (int s = 1; s < kRedSlots; s *= 2)
#pragma unroll
        for (int i = 0; i < kRedSlots; i += 2 * s) v[i] += v[i + s];
    return v[0];
}

// Token placement in the 16 x 16 MFMA with MR accumulators per lane.  A lane
// holds C rows 4 kq + j (kq = lane / 16, j < 4); only j < MR are kept, and C
// row 4 kq + j carries token kq MR + j, so MR accumulators cover 4 MR tokens
// (M = 1: MR = 1, M <= 8: 2, M <= 16: 4).  A row r therefore reads token
// (r / 4) MR + r % 4; rows with r % 4 >= MR feed C rows that are never kept
// and read a valid token instead.
template <int MR>
__device__ __forceinline__ int a_token(int r, int M)
{
    const int j = r & 3;
    const int t = (r >> 2) * MR + (j < MR ? j : 0);
    return t < M ? t : M - 1;
}
template <int MR>
__device__ __forceinline__ int c_token(int kq, int j) { return kq * MR + j; }

// 8 codes of one dword -> 8 exact fp16 values q - z, element j = K offset j.
// blo = -(1024 + z), bhi = -(64 + z) in both halves.
__device__ __forceinline__ h8 unpack8(uint32_t w, uint32_t magic, h2 blo, h2 bhi)
{
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    const h2 p0 = bitcast<h2>((w & 0x000F000Fu) | magic) + blo;                                   // k+0, k+1
    const h2 p1 = __builtin_elementwise_fma(bitcast<h2>((w & 0x00F000F0u) | magic), sixteenth, bhi);  // k+2, k+3
    const h2 p2 = bitcast<h2>((w8 & 0x000F000Fu) | magic) + blo;                                  // k+4, k+5
    const h2 p3 = __builtin_elementwise_fma(bitcast<h2>((w8 & 0x00F000F0u) | magic), sixteenth, bhi); // k+6, k+7
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// per-tile group metadata of one lane's row: 128/G fp16 scales in s (two per
// dword) and, for asymmetric weights, 128/G int8 zero points in z
// Loads are whole aligned dwords inside the tile's metadata block, so every
// value stays 32-bit from load to use (a narrower value carried around a loop
// would be re-widened where it is defined, forcing a wait for its load
// there): for G = 128 the dword holds the scales of rows r & ~1 and r | 1,
// for G = 64 the zero points of those two rows, and for G = 128 the zero
// points of rows (r & ~3) .. (r | 3); decode_meta picks the lane's part.
template <int G, bool ASYM> struct MetaRaw {
    uint32_t s[(128 / G + 1) / 2];
    uint32_t z;
};

// Loads the group metadata of tile-row `idx` (= tile * 16 + row) from the
// strip's scale / zero-point descriptors; idx < 0 reads zeros.
template <int G, bool ASYM>
__device__ __forceinline__ MetaRaw<G, ASYM> load_meta(__amdgpu_buffer_rsrc_t srs, __amdgpu_buffer_rsrc_t zrs, int idx)
{
    constexpr int GPT = 128 / G;
    MetaRaw<G, ASYM> m;
    if constexpr (G == 128) {
        const uint32_t so = idx < 0 ? kBufferOob : (uint32_t)(idx & ~1) * 2;
        m.s[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, kStreamLoad);
    }
    if constexpr (G == 64) {
        const uint32_t so = idx < 0 ? kBufferOob : (uint32_t)idx * 4;
        m.s[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, kStreamLoad);
    }
    if constexpr (G == 32) {
        const uint32_t so = idx < 0 ? kBufferOob : (uint32_t)idx * 8;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, so, 0, kStreamLoad);
        m.s[0] = v[0];
        m.s[1] = v[1];
    }
    m.z = 0;
    if constexpr (ASYM) {
        uint32_t zo;
        if constexpr (G == 128) zo = idx < 0 ? kBufferOob : (uint32_t)(idx & ~3);
        if constexpr (G == 64) zo = idx < 0 ? kBufferOob : (uint32_t)(idx & ~1) * 2;
        if constexpr (G == 32) zo = idx < 0 ? kBufferOob : (uint32_t)idx * 4;
        m.z = __builtin_amdgcn_raw_buffer_load_b32(zrs, zo, 0, kStreamLoad);
    }
    (void)GPT;
    return m;
}

// Makes the metadata opaque at its point of use, so its decode is not hoisted.
template <int G, bool ASYM>
__device__ __forceinline__ void pin_meta(MetaRaw<G, ASYM> &m)
{
#pragma unroll
    for (int i = 0; i < (128 / G + 1) / 2; ++i) asm volatile("" : "+v"(m.s[i]));
    if constexpr (ASYM) asm volatile("" : "+v"(m.z));
}

// r = the lane's weight row inside the tile (lane % 16)
template <int G, bool ASYM>
__device__ __forceinline__ void decode_meta(const MetaRaw<G, ASYM> &m, int r, float *sc, h2 *blo, h2 *bhi)
{
    constexpr int GPT = 128 / G;
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
        uint16_t hb;
        if constexpr (G == 128) hb = (uint16_t)(m.s[0] >> (16 * (r & 1)));
        else hb = (uint16_t)(m.s[g / 2] >> (16 * (g & 1)));
        sc[g] = (float)__builtin_bit_cast(_Float16, hb);
        int z = 8;
        if constexpr (ASYM) {
            uint32_t zb;
            if constexpr (G == 128) zb = m.z >> (8 * (r & 3));
            else if constexpr (G == 64) zb = m.z >> (16 * (r & 1) + 8 * g);
            else zb = m.z >> (8 * g);
            z = (int)(int8_t)(uint8_t)zb;
        }
        const _Float16 lo = (_Float16)(-1024.0f - (float)z);   // exact: |1024 + z| < 2048
        const _Float16 hi = (_Float16)(-64.0f - (float)z);
        blo[g] = h2{lo, lo};
        bhi[g] = h2{hi, hi};
    }
}

// One 1 KiB tile: 4 MFMAs over 32 K each; per quantization group the MFMA
// chain is scaled in fp32 and added to acc.
template <int G, bool ASYM, int MR>
__device__ __forceinline__ void tile_product(const u4 &q, const MetaRaw<G, ASYM> &mr, const h8 *a,
                                             uint32_t magic, f4 &acc)
{
    constexpr int GPT = 128 / G;
    constexpr int MPG = G / 32;                      // MFMAs per group
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    float sc[GPT];
    h2 blo[GPT], bhi[GPT];
    decode_meta<G, ASYM>(mr, (int)(threadIdx.x & 15), sc, blo, bhi);   // lane % 16 = the lane's weight row
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    f4 c = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = i / MPG;
        const h8 b = unpack8(wd[i], magic, blo[g], bhi[g]);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b, (i % MPG == 0) ? zero4 : c, 0, 0, 0);
        if (i % MPG == MPG - 1) {
#pragma unroll
            for (int j = 0; j < MR; ++j) acc[j] += sc[g] * c[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Offset-split product.  Masking a code into the low mantissa nibble of fp16
// 1024.0 (0x6400) gives 1024 + q exactly; masking it into the next nibble of
// fp16 64.0 (0x5400, where one unit is 1/16) gives 64 + q exactly.  Each dword
// of codes becomes an MFMA operand v with one shift and four mask-or
// operations: v = 1024 + q at K offsets 0, 1, 4, 5 and 64 + q at 2, 3, 6, 7.
// The zero point enters as a second operand p of the same shape (1024 + z or
// 64 + z), multiplied with the same activations by a second MFMA chain, so
//   sum x (q - z) = (x . v) - (x . p).
// Both chains see the same activations in the same order; where q = z the
// operands are identical and the difference is exactly zero.  p does not
// depend on the codes: for symmetric weights it is a constant register, for
// asymmetric ones it is built once per group from the row's zero point.
// ---------------------------------------------------------------------------
constexpr uint32_t kMagicLo = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kMagicHi = 0x54005400u;   // fp16 64.0 in both halves

// 8 codes of one dword -> 1024 + q (K offsets 0, 1, 4, 5), 64 + q (2, 3, 6, 7)
__device__ __forceinline__ h8 unpack8_split(uint32_t w, uint32_t mlo, uint32_t mhi)
{
    const uint32_t w8 = w >> 8;
    const u4 v = {(w & 0x000F000Fu) | mlo, (w & 0x00F000F0u) | mhi, (w8 & 0x000F000Fu) | mlo,
                  (w8 & 0x00F000F0u) | mhi};
    return __builtin_bit_cast(h8, v);
}

// the offset operand of zero point z: 1024 + z and 64 + z in the same slots
__device__ __forceinline__ h8 offset8(int z)
{
    const _Float16 lo = (_Float16)(1024.0f + (float)z);   // exact: integers below 2048
    const _Float16 hi = (_Float16)(64.0f + (float)z);
    return h8{lo, lo, hi, hi, lo, lo, hi, hi};
}

// One 1 KiB tile, offset-split.  psym: the offset operand of the symmetric
// zero point 8, kept in registers by the caller.
template <int G, bool ASYM, int MR>
__device__ __forceinline__ void tile_product_split(const u4 &q, const MetaRaw<G, ASYM> &mr, const h8 *a,
                                                   const h8 &psym, uint32_t mlo, uint32_t mhi, f4 &acc)
{
    constexpr int MPG = G / 32;                      // MFMAs per group
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int r = (int)(threadIdx.x & 15);
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    f4 cv = zero4, cp = zero4;
    h8 p = psym;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = i / MPG;
        if constexpr (ASYM) {
            if (i % MPG == 0) {
                uint32_t zb;
                if constexpr (G == 128) zb = mr.z >> (8 * (r & 3));
                else if constexpr (G == 64) zb = mr.z >> (16 * (r & 1) + 8 * g);
                else zb = mr.z >> (8 * g);
                p = offset8((int)(int8_t)(uint8_t)zb);
            }
        }
        const h8 v = unpack8_split(wd[i], mlo, mhi);
        cv = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], v, (i % MPG == 0) ? zero4 : cv, 0, 0, 0);
        cp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], p, (i % MPG == 0) ? zero4 : cp, 0, 0, 0);
        if (i % MPG == MPG - 1) {
            uint16_t hb;
            if constexpr (G == 128) hb = (uint16_t)(mr.s[0] >> (16 * (r & 1)));
            else hb = (uint16_t)(mr.s[g / 2] >> (16 * (g & 1)));
            const float sc = (float)__builtin_bit_cast(_Float16, hb);
#pragma unroll
            for (int j = 0; j < MR; ++j) acc[j] = __builtin_fmaf(sc, cv[j] - cp[j], acc[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Asymmetric weights with G = 32 (one dword of codes per group and lane): the
// MFMA operand is q - z itself, so one chain per group and no offset chain.
// Codes at K offsets 0, 1, 4, 5 are masked into fp16 1152.0 (0x6480, low
// seven mantissa bits clear), giving 1152 + q; codes at 2, 3, 6, 7 into 64.0
// as in the offset-split form, giving 64 + q.  The zero point becomes
// 1152 + z = 0x6400 | (z + 128) by flipping the top bit of its byte (one
// byte permute per group places it in both halves under 0x64), and
// 64 + z = (1152 + z) - 1088.  All of these are integers (or 64 + q with
// one unit 1/16) that fp16 holds exactly, and so are the differences
// (1152 + q) - (1152 + z) = q - z and (64 + q) - (64 + z) = q - z, which
// IEEE subtraction therefore returns exactly.
// ---------------------------------------------------------------------------
constexpr uint32_t kMagic1152 = 0x64806480u;  // fp16 1152.0 in both halves

// sel[g]: byte-permute selectors {z_g + 128, 0x64, z_g + 128, 0x64}, kept in
// registers by the caller.
__device__ __forceinline__ void zp32_selectors(uint32_t *sel)
{
#pragma unroll
    for (int g = 0; g < 4; ++g) sel[g] = (uint32_t)g | (4u << 8) | ((uint32_t)g << 16) | (4u << 24);
}

template <int MR>
__device__ __forceinline__ void tile_product_zp32(const u4 &q, const MetaRaw<32, true> &mr, const h8 *a,
                                                  uint32_t m1152, uint32_t mhi, const uint32_t *sel, f4 &acc)
{
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    const uint32_t zx = mr.z ^ 0x80808080u;          // byte g: z_g + 128
    const h2 k1088 = {(_Float16)1088.0f, (_Float16)1088.0f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const h2 tlo = bitcast<h2>(__builtin_amdgcn_perm(0x64646464u, zx, sel[g]));   // 1152 + z_g
        const h2 thi = tlo - k1088;                                                   // 64 + z_g
        const uint32_t w = wd[g], w8 = w >> 8;
        const h2 b0 = bitcast<h2>((w & 0x000F000Fu) | m1152) - tlo;    // k+0, k+1
        const h2 b1 = bitcast<h2>((w & 0x00F000F0u) | mhi) - thi;      // k+2, k+3
        const h2 b2 = bitcast<h2>((w8 & 0x000F000Fu) | m1152) - tlo;   // k+4, k+5
        const h2 b3 = bitcast<h2>((w8 & 0x00F000F0u) | mhi) - thi;     // k+6, k+7
        const h8 b = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
        const f4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[g], b, zero4, 0, 0, 0);
        const uint16_t hb = (uint16_t)(mr.s[g / 2] >> (16 * (g & 1)));
        const float sc = (float)__builtin_bit_cast(_Float16, hb);
#pragma unroll
        for (int j = 0; j < MR; ++j) acc[j] = __builtin_fmaf(sc, c[j], acc[j]);
    }
}

// Batch-1 symmetric form: the offset terms of the tile's groups come in
// precomputed (off[g], valid in the lanes that hold C row 0), so only the
// code chain runs here.
template <int G>
__device__ __forceinline__ void tile_product_pre(const u4 &q, const MetaRaw<G, false> &mr, const h8 *a,
                                                 const float *off, uint32_t mlo, uint32_t mhi, f4 &acc)
{
    constexpr int MPG = G / 32;
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int r = (int)(threadIdx.x & 15);
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    f4 cv = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = i / MPG;
        const h8 v = unpack8_split(wd[i], mlo, mhi);
        cv = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], v, (i % MPG == 0) ? zero4 : cv, 0, 0, 0);
        if (i % MPG == MPG - 1) {
            uint16_t hb;
            if constexpr (G == 128) hb = (uint16_t)(mr.s[0] >> (16 * (r & 1)));
            else hb = (uint16_t)(mr.s[g / 2] >> (16 * (g & 1)));
            const float sc = (float)__builtin_bit_cast(_Float16, hb);
            acc[0] = __builtin_fmaf(sc, cv[0] - off[g], acc[0]);
        }
    }
}

}  // namespace tile
}  // namespace lowbit
