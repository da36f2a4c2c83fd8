// gemv_tile.hpp -- device helpers shared by the W4 GEMV kernels: in-register
// nibble unpack, per-tile group metadata, and the MFMA product of one packed
// 1 KiB tile (16 weight rows x 128 K) with up to 16 activation rows.
#pragma once

#include "lowbit_internal.hpp"

namespace lowbit {
namespace tile {

template <typename T>
__device__ __forceinline__ T bitcast(uint32_t v) { return __builtin_bit_cast(T, v); }

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
        m.s[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, 0);
    }
    if constexpr (G == 64) {
        const uint32_t so = idx < 0 ? kBufferOob : (uint32_t)idx * 4;
        m.s[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, 0);
    }
    if constexpr (G == 32) {
        const uint32_t so = idx < 0 ? kBufferOob : (uint32_t)idx * 8;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, so, 0, 0);
        m.s[0] = v[0];
        m.s[1] = v[1];
    }
    m.z = 0;
    if constexpr (ASYM) {
        uint32_t zo;
        if constexpr (G == 128) zo = idx < 0 ? kBufferOob : (uint32_t)(idx & ~3);
        if constexpr (G == 64) zo = idx < 0 ? kBufferOob : (uint32_t)(idx & ~1) * 2;
        if constexpr (G == 32) zo = idx < 0 ? kBufferOob : (uint32_t)idx * 4;
        m.z = __builtin_amdgcn_raw_buffer_load_b32(zrs, zo, 0, 0);
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

}  // namespace tile
}  // namespace lowbit
