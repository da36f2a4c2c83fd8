// gemv_wb.hip -- decode GEMV / small-batch product with uniform b-bit codes,
// b = 1..8 ("Low Bit ARM kernels": one unpack routine per bit width from 1 to
// 8 bits in a bit-width x tile table, group-wise fp16 scales, symmetric or
// with an int8 zero point; fewer bits, fewer weight bytes to stream at decode).
//
//   y[m][n] = sum_k x[m][k] * (q[n][k] - z) * s[n][k / G],  z = 2^(b-1) or int8
//
// MI355X design: the W4 streaming GEMV's schedule (one workgroup per 16-row
// strip, waves split K, x staged in LDS by LDS-direct loads, every weight load
// issued up front with the non-temporal hint, fixed-order cross-wave sum, fp16
// RNE) with the codes split into 4-, 2- and 1-bit planes (lowbit_internal.hpp).
// A shift and a mask of a plane dword give two codes in the two 16-bit halves;
// or-ed together and into fp16 1024.0 they form 1024 + q exactly (q <= 255),
// which feeds the offset-split product of gemv_tile.hpp: x.(1024 + q) -
// x.(1024 + z) by two MFMA chains over the same activations (at batch 1 with
// symmetric weights one chain of offsets serves four tiles), so codes equal
// to the zero point give exactly zero.  b = 3 has its own nibble-aligned
// layout (lowbit_internal.hpp): its codes unpack in the INT4 offset-split form,
// 1024 + q and 64 + q, with a 3-bit mask.
#include "lowbit_internal.hpp"
#include "gemv_tile.hpp"

namespace lowbit {

namespace {

using namespace tile;

constexpr int kWbMaxLds = 160 * 1024;

// 16-byte blocks per K tile of a row of x in LDS: 16, or 20 for the batch-1
// symmetric form, whose shared offset chain reads the same block of four
// consecutive tiles at once (the 64-byte pad puts those reads in different
// banks)
__host__ __device__ constexpr int wb_tile_blocks(bool pre) { return pre ? 20 : 16; }
__host__ __device__ inline int wb_rowp(int kt, bool pre) { return (int)round_up((int64_t)kt * wb_tile_blocks(pre), 64); }
__host__ __device__ inline int wb_lds(int M, int kt, int W, int MR, bool pre)
{
    return M * wb_rowp(kt, pre) * 16 + (W > 1 ? kRedSlots * MR * 64 * 4 : 0);
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// the planes of one lane's tile, as loaded
template <int BITS>
struct WbTile {
    static constexpr int N4 = BITS / 4, N2 = (BITS % 4) >= 2 ? 1 : 0, N1 = BITS & 1;
    u4 a[N4 > 0 ? N4 : 1];
    uint2 b;
    uint32_t c;
};

// tile base byte offset `base`; each plane is a lane-major region of the tile
template <int BITS>
__device__ __forceinline__ WbTile<BITS> load_wb(__amdgpu_buffer_rsrc_t rs, bool ok, uint32_t base, int lane)
{
    using TT = WbTile<BITS>;
    TT w;
    if constexpr (BITS == 3) {                         // the lane's three dwords, one load
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(rs, ok ? base + lane * 12 : kBufferOob, 0, kStreamLoad);
        w.b = make_uint2(v[0], v[1]);
        w.c = v[2];
        return w;
    }
#pragma unroll
    for (int p = 0; p < TT::N4; ++p)
        w.a[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? base + 1024 * p + lane * 16 : kBufferOob, 0,
                                                       kStreamLoad);
    if constexpr (TT::N2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, ok ? base + 1024 * TT::N4 + lane * 8 : kBufferOob, 0,
                                                            kStreamLoad);
        w.b = make_uint2(v[0], v[1]);
    }
    if constexpr (TT::N1)
        w.c = __builtin_amdgcn_raw_buffer_load_b32(
            rs, ok ? base + 1024 * TT::N4 + 512 * TT::N2 + lane * 4 : kBufferOob, 0, kStreamLoad);
    return w;
}

template <int BITS>
__device__ __forceinline__ void pin_wb(WbTile<BITS> &w)
{
    using TT = WbTile<BITS>;
#pragma unroll
    for (int p = 0; p < TT::N4; ++p) asm volatile("" : "+v"(w.a[p]));
    if constexpr (TT::N2) asm volatile("" : "+v"(w.b.x), "+v"(w.b.y));
    if constexpr (TT::N1) asm volatile("" : "+v"(w.c));
}

// the bits of a plane that sit at position `src` of each 16-bit half, moved to
// position `dst`: one shift (none when equal) and a mask
template <int SRC, int DST, uint32_t MASK>
__device__ __forceinline__ uint32_t plane_bits(uint32_t w)
{
    if constexpr (SRC > DST) return (w >> (SRC - DST)) & (MASK << DST);
    else if constexpr (SRC < DST) return (w << (DST - SRC)) & (MASK << DST);
    else return w & (MASK << DST);
}

// MFMA block I (K offsets 0..7 of the lane's 8-K slice), pair Q -> two fp16
// 1024 + q: each plane's pair, shifted into place, or-ed into 1024.0
template <int BITS, int I, int Q>
__device__ __forceinline__ uint32_t wb_pair(const WbTile<BITS> &w, uint32_t magic)
{
    using TT = WbTile<BITS>;
    uint32_t r = magic;
    if constexpr (TT::N4 >= 1) r |= plane_bits<4 * Q, 0, 0x000F000Fu>(w.a[0][I]);
    if constexpr (TT::N4 >= 2) r |= plane_bits<4 * Q, 4, 0x000F000Fu>(w.a[1][I]);
    if constexpr (TT::N2) r |= plane_bits<2 * (4 * (I & 1) + Q), 4 * TT::N4, 0x00030003u>((I >> 1) ? w.b.y : w.b.x);
    if constexpr (TT::N1) r |= plane_bits<4 * I + Q, 4 * TT::N4 + 2 * TT::N2, 0x00010001u>(w.c);
    return r;
}

template <int BITS, int I>
__device__ __forceinline__ h8 wb_operand(const WbTile<BITS> &w, uint32_t magic)
{
    const u4 v = {wb_pair<BITS, I, 0>(w, magic), wb_pair<BITS, I, 1>(w, magic), wb_pair<BITS, I, 2>(w, magic),
                  wb_pair<BITS, I, 3>(w, magic)};
    return __builtin_bit_cast(h8, v);
}

// b = 3: the dword of block I (block 3's gathered from the spare nibble bits)
// -> 1024 + q at K offsets 0, 1, 4, 5 and 64 + q at 2, 3, 6, 7, the INT4
// offset-split form with a 3-bit mask (one shift and four mask-or operations)
template <int I>
__device__ __forceinline__ h8 wb3_operand(const WbTile<3> &w, uint32_t mlo, uint32_t mhi)
{
    uint32_t d;
    if constexpr (I == 0) d = w.b.x;
    else if constexpr (I == 1) d = w.b.y;
    else if constexpr (I == 2) d = w.c;
    else d = ((w.b.x >> 3) & 0x11111111u) | ((w.b.y >> 2) & 0x22222222u) | ((w.c >> 1) & 0x44444444u);
    const uint32_t d8 = d >> 8;
    const u4 v = {(d & 0x00070007u) | mlo, (d & 0x00700070u) | mhi, (d8 & 0x00070007u) | mlo,
                  (d8 & 0x00700070u) | mhi};
    return __builtin_bit_cast(h8, v);
}

// b = 8: block I's two dwords (a code per byte) -> 1024 + q at K offsets 0..7
template <int I>
__device__ __forceinline__ h8 wb8_operand(const WbTile<8> &w, uint32_t magic)
{
    const uint32_t d0 = w.a[I >> 1][2 * (I & 1)], d1 = w.a[I >> 1][2 * (I & 1) + 1];
    const u4 v = {(d0 & 0x00FF00FFu) | magic, ((d0 >> 8) & 0x00FF00FFu) | magic, (d1 & 0x00FF00FFu) | magic,
                  ((d1 >> 8) & 0x00FF00FFu) | magic};
    return __builtin_bit_cast(h8, v);
}

// the offset operand of zero point z in the slots of the operand above
__device__ __forceinline__ h8 wb3_offset(int z)
{
    const _Float16 lo = (_Float16)(1024.0f + (float)z);   // exact: integers below 2048
    const _Float16 hi = (_Float16)(64.0f + (float)z);
    return h8{lo, lo, hi, hi, lo, lo, hi, hi};
}

// offset operand of zero point z: 1024 + z in every half
__device__ __forceinline__ h8 wb_offset(int z)
{
    const _Float16 o = (_Float16)(1024.0f + (float)z);   // exact: integers below 2048
    return h8{o, o, o, o, o, o, o, o};
}

template <int BITS, int G, bool ASYM, int MR, int T, bool SINGLE = false>
__device__ __forceinline__ void wb_strip(const uint8_t *codes, const uint8_t *scales, const uint8_t *zeros,
                                         const _Float16 *xg, _Float16 *yp, int N, int K, int kt, int tw, int M, int W,
                                         int strip)
{
    using TT = WbTile<BITS>;
    constexpr int GPT = 128 / G;
    constexpr int MPG = G / 32;
    constexpr bool PRE = !ASYM && MR == 1;                  // shared offset chain (batch 1, symmetric)
    constexpr int TB = wb_tile_blocks(PRE);
    constexpr int TPS = 4 / GPT;                            // tiles per offset set
    constexpr int NLD = BITS == 3 ? 1 : TT::N4 + TT::N2 + TT::N1;   // code loads per tile (b = 8: 2)
    constexpr int NW = T * (NLD + (ASYM ? 2 : 1));           // weight + metadata loads per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, kq = lane >> 4;
    const int t0 = wave * tw;
    const int rowp = wb_rowp(kt, PRE);
    float *red = reinterpret_cast<float *>(smem + M * rowp * 16);

    // 1. x -> LDS: block bb < 16 of tile t of row m holds
    //    x[m][128 t + 8 (bb ^ (m & 15)) ..], blocks 16..TB-1 are zero padding
    {
        const auto xrs = buffer_rsrc(xg, (uint32_t)(M * K * 2));
        const int cpr = rowp >> 6;
        for (int m = 0; m < M; ++m)
            for (int cc = wave; cc < cpr; cc += W) {
                const int jj = cc * 64 + lane;
                const int t = jj / TB, bb = jj - t * TB;
                const int j = t * 16 + (bb ^ (m & 15));
                const bool ok = bb < 16 && j * 8 < K;
                lds_dma16(xrs, smem + (m * cpr + cc) * 1024, ok ? (uint32_t)((m * K + j * 8) * 2) : kBufferOob);
            }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. codes and metadata of this wave's tiles; 3. x in LDS everywhere,
    //    waited for after the first EARLY tiles' loads (eight tiles per wave:
    //    after the first, so the x reads do not land behind the compute
    //    unit's whole weight stream; a single-problem launch with four tiles
    //    per wave: after two)
    TT q[T];
    MetaRaw<G, ASYM> mr[T];
    constexpr int EARLY = T >= 8 ? 1 : (SINGLE && T == 4 ? 2 : T);
    constexpr int LPT = NLD + (ASYM ? 2 : 1);        // loads per tile (code planes, scales[, zeros])
    static_assert(NW == T * LPT, "load count");
    const int64_t tiles0 = (int64_t)strip * kt;
    const auto crs = buffer_rsrc(codes + tiles0 * 256 * BITS, (uint32_t)kt * 256 * BITS);
    const auto srs = buffer_rsrc(scales + tiles0 * 16 * GPT * 2, (uint32_t)kt * 16 * GPT * 2);
    const auto zrs = buffer_rsrc(ASYM ? zeros + tiles0 * 16 * GPT : scales, ASYM ? (uint32_t)kt * 16 * GPT : 0u);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u == EARLY) {
            wait_vm<EARLY * LPT>();                  // x has landed; tiles < EARLY may be in flight
            asm volatile("s_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        const int t = t0 + u;
        const bool ok = u < tw && t < kt;
        q[u] = load_wb<BITS>(crs, ok, (uint32_t)t * 256 * BITS, lane);
        mr[u] = load_meta<G, ASYM>(srs, zrs, ok ? t * 16 + r : -1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (EARLY == T) {
        wait_vm<NW>();
        asm volatile("s_barrier" ::: "memory");
    }

    // 4. products, tile by tile in load order
    uint32_t magic = 0x64006400u;                    // fp16 1024.0 in both halves
    uint32_t magic_hi = 0x54005400u;                 // fp16 64.0 (b = 3)
    asm volatile("" : "+v"(magic));
    if constexpr (BITS == 3) asm volatile("" : "+v"(magic_hi));
    h8 psym = BITS == 3 ? wb3_offset(1 << (BITS - 1)) : wb_offset(1 << (BITS - 1));
    {
        u4 pw = __builtin_bit_cast(u4, psym);
        asm volatile("" : "+v"(pw));
        psym = __builtin_bit_cast(h8, pw);
    }
    const int xr = a_token<MR>(r, M);
    const _Float16 *xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xa[i] = reinterpret_cast<const _Float16 *>(smem) + (xr * rowp + t0 * TB + ((i * 4 + kq) ^ (xr & 15))) * 8;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // batch 1, symmetric: x . p does not depend on the codes or the weight
    // row, so one MFMA chain computes it for several tiles, its A rows 0..3
    // carrying the K blocks of (tile u0 + j / GPT, group j % GPT); C row j is
    // exactly what a per-tile chain would give (same products, same order)
    f4 cps = zero4;
    const int tvalid = min(tw, kt - t0);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u < tvalid) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (PRE) {
                if (u % TPS == 0) {
                    const int rr = r < 4 ? r : 0;
                    const int tu = min(u + rr / GPT, tvalid - 1);
                    const int g = rr % GPT;
                    const _Float16 *xb = reinterpret_cast<const _Float16 *>(smem) + ((t0 + tu) * TB + g * MPG * 4 + kq) * 8;
#pragma unroll
                    for (int i = 0; i < MPG; ++i)
                        cps = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const h8 *>(xb + i * 32), psym,
                                                                     i == 0 ? zero4 : cps, 0, 0, 0);
                }
            }
            TT w = q[u];
            pin_wb<BITS>(w);
            MetaRaw<G, ASYM> mv = mr[u];
            pin_meta<G, ASYM>(mv);
            h8 vs[4];
            if constexpr (BITS == 8) {
                vs[0] = wb8_operand<0>(w, magic);
                vs[1] = wb8_operand<1>(w, magic);
                vs[2] = wb8_operand<2>(w, magic);
                vs[3] = wb8_operand<3>(w, magic);
            } else if constexpr (BITS == 3) {
                vs[0] = wb3_operand<0>(w, magic, magic_hi);
                vs[1] = wb3_operand<1>(w, magic, magic_hi);
                vs[2] = wb3_operand<2>(w, magic, magic_hi);
                vs[3] = wb3_operand<3>(w, magic, magic_hi);
            } else {
                vs[0] = wb_operand<BITS, 0>(w, magic);
                vs[1] = wb_operand<BITS, 1>(w, magic);
                vs[2] = wb_operand<BITS, 2>(w, magic);
                vs[3] = wb_operand<BITS, 3>(w, magic);
            }
            f4 cv = zero4, cp = zero4;
            h8 p = psym;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = i / MPG;
                if constexpr (ASYM) {
                    if (i % MPG == 0) {
                        uint32_t zb;
                        if constexpr (G == 128) zb = mv.z >> (8 * (r & 3));
                        else if constexpr (G == 64) zb = mv.z >> (16 * (r & 1) + 8 * g);
                        else zb = mv.z >> (8 * g);
                        p = BITS == 3 ? wb3_offset((int)(int8_t)(uint8_t)zb) : wb_offset((int)(int8_t)(uint8_t)zb);
                    }
                }
                const h8 a = *reinterpret_cast<const h8 *>(xa[i] + u * TB * 8);
                cv = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, vs[i], (i % MPG == 0) ? zero4 : cv, 0, 0, 0);
                if constexpr (!PRE) cp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p, (i % MPG == 0) ? zero4 : cp, 0, 0, 0);
                if (i % MPG == MPG - 1) {
                    uint16_t hb;
                    if constexpr (G == 128) hb = (uint16_t)(mv.s[0] >> (16 * (r & 1)));
                    else hb = (uint16_t)(mv.s[g / 2] >> (16 * (g & 1)));
                    const float sc = (float)__builtin_bit_cast(_Float16, hb);
                    if constexpr (PRE) {
                        acc[0] = __builtin_fmaf(sc, cv[0] - cps[(u % TPS) * GPT + g], acc[0]);
                    } else {
#pragma unroll
                        for (int j = 0; j < MR; ++j) acc[j] = __builtin_fmaf(sc, cv[j] - cp[j], acc[j]);
                    }
                }
            }
        }
    }

    // 5. fixed-order cross-wave sum (a balanced tree over the sixteen
    //    partial slots), fp16 RNE store
    if (W > 1) {
#pragma unroll
        for (int j = 0; j < MR; ++j) red_put(red + j * 64 + lane, MR * 64, wave, W, acc[j]);
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < MR; ++j) acc[j] = red_sum(red + j * 64 + lane, MR * 64);
        }
    }
    if (wave == 0) {
        const int n = strip * 16 + r;
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const int m = c_token<MR>(kq, j);
            if (m < M && n < N) yp[(int64_t)m * N + n] = (_Float16)acc[j];
        }
    }
}

template <int BITS, int G, bool ASYM, int MR, int T>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(T > 4 ? 4 : (!ASYM && MR == 1 && BITS <= 4) ? 8 : 6)))
void gemv_wb_single(const uint8_t *codes, const uint8_t *scales, const _Float16 *xg, _Float16 *yp, int N, int K,
                    int kt, int tw, int M, int W, const uint8_t *zeros)
{
    wb_strip<BITS, G, ASYM, MR, T, true>(codes, scales, zeros, xg, yp, N, K, kt, tw, M, W, (int)blockIdx.x);
}

// problems laid end to end over blockIdx.x (b.first[i] = first workgroup of
// problem i; unused entries hold INT_MAX)
template <int BITS, int G, bool ASYM, int MR, int T>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(T > 4 ? 4 : (!ASYM && MR == 1 && BITS <= 4) ? 8 : 6)))
void gemv_wb_batch(const GemvBatch b)
{
    const int bx = (int)blockIdx.x;
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGemvBatch; ++i) pi += bx >= b.first[i] ? 1 : 0;
    const GemvProblem &p = b.p[pi];
    wb_strip<BITS, G, ASYM, MR, T>(p.codes, p.scales, p.zeros, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W,
                                   bx - b.first[pi]);
}

inline hipError_t wb_lds_limit(const void *k, size_t lds, bool &raised)
{
    if (lds <= 64 * 1024 || raised) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kWbMaxLds);
    if (e == hipSuccess) raised = true;
    return e;
}

template <int BITS, int G, bool ASYM, int MR, int T>
hipError_t wb_launch_k(const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    if (b.count == 1) {
        static bool raised = false;
        auto k = gemv_wb_single<BITS, G, ASYM, MR, T>;
        const hipError_t e = wb_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        const GemvProblem &p = b.p[0];
        k<<<grid, block, lds, st>>>(p.codes, p.scales, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W, p.zeros);
    } else {
        static bool raised = false;
        auto k = gemv_wb_batch<BITS, G, ASYM, MR, T>;
        const hipError_t e = wb_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        k<<<grid, block, lds, st>>>(b);
    }
    return hipGetLastError();
}

template <int BITS, int G, bool ASYM>
hipError_t wb_launch_mt(int MR, int T, const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    if (MR == 1) return T <= 4 ? wb_launch_k<BITS, G, ASYM, 1, 4>(b, grid, block, lds, st)
                               : wb_launch_k<BITS, G, ASYM, 1, 8>(b, grid, block, lds, st);
    if (MR == 2) return T <= 4 ? wb_launch_k<BITS, G, ASYM, 2, 4>(b, grid, block, lds, st)
                               : wb_launch_k<BITS, G, ASYM, 2, 8>(b, grid, block, lds, st);
    return T <= 4 ? wb_launch_k<BITS, G, ASYM, 4, 4>(b, grid, block, lds, st)
                  : wb_launch_k<BITS, G, ASYM, 4, 8>(b, grid, block, lds, st);
}

template <int BITS>
hipError_t wb_launch_bits(int G, bool asym, int MR, int T, const GemvBatch &b, dim3 grid, dim3 block, size_t lds,
                          hipStream_t st)
{
    switch (G) {
    case 32: return asym ? wb_launch_mt<BITS, 32, true>(MR, T, b, grid, block, lds, st)
                         : wb_launch_mt<BITS, 32, false>(MR, T, b, grid, block, lds, st);
    case 64: return asym ? wb_launch_mt<BITS, 64, true>(MR, T, b, grid, block, lds, st)
                         : wb_launch_mt<BITS, 64, false>(MR, T, b, grid, block, lds, st);
    default: return asym ? wb_launch_mt<BITS, 128, true>(MR, T, b, grid, block, lds, st)
                         : wb_launch_mt<BITS, 128, false>(MR, T, b, grid, block, lds, st);
    }
}

}  // namespace

// LDS the b-bit GEMV needs for M rows over the widest problem (0 if it has
// no kernel for it: more than 8 tiles per wave or more than 160 KiB)
size_t gemv_wb_lds(int M, int64_t kt_max, bool asym)
{
    int W = (int)((kt_max + 3) / 4);
    W = W < 1 ? 1 : (W > 16 ? 16 : W);
    const int64_t T = (kt_max + W - 1) / W;
    const int MR = M == 1 ? 1 : (M <= 8 ? 2 : 4);     // accumulators per lane (see a_token)
    const int64_t lds = wb_lds(M, (int)kt_max, W, MR, !asym && MR == 1);
    return (T > 8 || lds > kWbMaxLds) ? 0 : (size_t)lds;
}

hipError_t launch_gemv_wb_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                const _Float16 *const *x, _Float16 *const *y, hipStream_t s)
{
    if (M == 0 || count == 0) return hipSuccess;
    GemvBatch b;
    int64_t strips = 0, kt = 0;
    for (int i = 0; i < count; ++i) kt = L[i].ktiles > kt ? L[i].ktiles : kt;
    int W = (int)((kt + 3) / 4);
    W = W < 1 ? 1 : (W > 16 ? 16 : W);
    const int T = (int)((kt + W - 1) / W);
    const int MR = M == 1 ? 1 : (M <= 8 ? 2 : 4);     // accumulators per lane (see a_token)
    const size_t lds = (size_t)wb_lds(M, (int)kt, W, MR, !L[0].asym && MR == 1);
    if (T > 8 || lds > (size_t)kWbMaxLds) return hipErrorInvalidValue;   // rejected by the caller first
    for (int i = 0; i < kMaxGemvBatch; ++i) b.first[i] = 0x7FFFFFFF;
    for (int i = 0; i < count; ++i) {
        GemvProblem &p = b.p[i];
        p.codes = packed[i] + L[i].codes_off;
        p.scales = packed[i] + L[i].scales_off;
        p.zeros = L[i].asym ? packed[i] + L[i].zeros_off : nullptr;
        p.x = x[i];
        p.y = y[i];
        p.N = (int)L[i].N;
        p.K = (int)L[i].K;
        p.ktiles = (int)L[i].ktiles;
        p.strips = (int)L[i].strips;
        p.tw = (int)((L[i].ktiles + W - 1) / W);
        p.pad = 0;
        b.first[i] = (int)strips;
        strips += L[i].strips;
    }
    b.count = count;
    b.M = M;
    b.ct = 0;
    b.W = W;
    if (strips == 0) return hipSuccess;
    const dim3 grid((unsigned)strips), block((unsigned)(W * 64));
    const int G = L[0].G;
    const bool asym = L[0].asym;
    switch (L[0].bits) {
    case 1: return wb_launch_bits<1>(G, asym, MR, T, b, grid, block, lds, s);
    case 2: return wb_launch_bits<2>(G, asym, MR, T, b, grid, block, lds, s);
    case 3: return wb_launch_bits<3>(G, asym, MR, T, b, grid, block, lds, s);
    case 4: return wb_launch_bits<4>(G, asym, MR, T, b, grid, block, lds, s);
    case 5: return wb_launch_bits<5>(G, asym, MR, T, b, grid, block, lds, s);
    case 6: return wb_launch_bits<6>(G, asym, MR, T, b, grid, block, lds, s);
    case 7: return wb_launch_bits<7>(G, asym, MR, T, b, grid, block, lds, s);
    default: return wb_launch_bits<8>(G, asym, MR, T, b, grid, block, lds, s);
    }
}

}  // namespace lowbit
