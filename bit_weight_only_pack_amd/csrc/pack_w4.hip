// pack_w4.hip -- offline re-pack of INT4 (and uniform b-bit) group-wise
// weights into the tiled device layout, its inverse, and the fp32 dequant
// test hook.
//
// Canonical input ("Low Bit Metal Kernels", int4_matmul step 2): row n of the
// weight holds K codes, two per byte, the low nibble being the even K index.
// The packed layout is described in lowbit_internal.hpp.  All three kernels
// are pure permutations / one exact product per weight, so they run once at
// load time and are not on the decode path.
#include "lowbit_internal.hpp"

namespace lowbit {

namespace {

constexpr int kThreads = 256;

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

// One thread per packed dword: gathers 8 codes of one row from the canonical
// bytes and places them in the interleaved nibble slots.
__global__ void w4_pack_codes(const uint8_t *__restrict__ codes, uint32_t *__restrict__ out,
                              int64_t N, int64_t K, int64_t ktiles, int64_t total)
{
    int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 8;          // 256 dwords per 1 KiB tile
    const int lane = (int)((d >> 2) & 63);
    const int i = (int)(d & 3);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + (lane & 15);
    const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
    uint32_t word = 0;
    if (n < N && kb < K) {
        // K % 32 == 0, so the 8 codes kb..kb+7 are all inside the row
        const uint8_t *row = codes + n * (K / 2) + kb / 2;
        const uint32_t src = (uint32_t)row[0] | ((uint32_t)row[1] << 8) | ((uint32_t)row[2] << 16) |
                             ((uint32_t)row[3] << 24);
        for (int j = 0; j < 8; ++j) {
            const uint32_t code = (src >> (4 * j)) & 0xF;   // byte j/2, nibble j%2 (low = even k)
            word |= code << (4 * w4_slot(j));
        }
    }
    out[d] = word;
}

// Inverse: one thread per packed dword writes the 4 canonical bytes.
__global__ void w4_unpack_codes(const uint32_t *__restrict__ in, uint8_t *__restrict__ codes,
                                int64_t N, int64_t K, int64_t ktiles, int64_t total)
{
    int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 8;
    const int lane = (int)((d >> 2) & 63);
    const int i = (int)(d & 3);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + (lane & 15);
    const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
    if (n >= N || kb >= K) return;
    const uint32_t word = in[d];
    uint32_t dst = 0;
    for (int j = 0; j < 8; ++j)
        dst |= ((word >> (4 * w4_slot(j))) & 0xF) << (4 * j);
    uint8_t *row = codes + n * (K / 2) + kb / 2;
    for (int b = 0; b < 4; ++b) row[b] = (uint8_t)(dst >> (8 * b));
}

// Group metadata (scales as 16-bit, zeros as 8-bit) in tile order.
// Packed index p -> (tile, row r, group-in-tile gi).
template <typename T>
__global__ void w4_pack_meta(const T *__restrict__ src, T *__restrict__ dst, int64_t N, int64_t K,
                             int G, int64_t ktiles, int64_t total)
{
    int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= total) return;
    const int gpt = 128 / G;
    const int gi = (int)(p % gpt);
    const int r = (int)((p / gpt) % 16);
    const int64_t tile = p / (gpt * 16);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + r;
    const int64_t g = t * gpt + gi;
    const int64_t groups = K / G;
    dst[p] = (n < N && g < groups) ? src[n * groups + g] : (T)0;
}

template <typename T>
__global__ void w4_unpack_meta(const T *__restrict__ src, T *__restrict__ dst, int64_t N, int64_t K,
                               int G, int64_t ktiles, int64_t total)
{
    int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= total) return;
    const int gpt = 128 / G;
    const int gi = (int)(p % gpt);
    const int r = (int)((p / gpt) % 16);
    const int64_t tile = p / (gpt * 16);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + r;
    const int64_t g = t * gpt + gi;
    const int64_t groups = K / G;
    if (n < N && g < groups) dst[n * groups + g] = src[p];
}

__global__ void fill_zero(uint8_t *__restrict__ p, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = 0;
}

// fp32 dequant: one thread per packed dword -> 8 weights of one row.
// w = (float)(q - z) * (float)s is exact in fp32 (<= 19 significant bits).
__global__ void w4_dequant_kernel(const uint32_t *__restrict__ codes, const _Float16 *__restrict__ scales,
                                  const int8_t *__restrict__ zeros, float *__restrict__ w,
                                  int64_t N, int64_t K, int G, int64_t ktiles, int64_t total)
{
    int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 8;
    const int lane = (int)((d >> 2) & 63);
    const int i = (int)(d & 3);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int r = lane & 15;
    const int64_t n = s * 16 + r;
    const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
    if (n >= N || kb >= K) return;
    const int gpt = 128 / G;
    const int gi = (i * 32) / G;                         // group of this 32-K sub-block inside the tile
    const int64_t meta = (tile * 16 + r) * gpt + gi;
    const float sc = (float)scales[meta];
    const int z = zeros ? (int)zeros[meta] : 8;
    const uint32_t word = codes[d];
    for (int j = 0; j < 8; ++j) {
        const int q = (int)((word >> (4 * w4_slot(j))) & 0xF);
        w[n * K + kb + j] = (float)(q - z) * sc;
    }
}

// ---- uniform b-bit codes: bit planes (layout in lowbit_internal.hpp) ----
struct WbPlanes {
    int n4, n2, n1;
};
__host__ __device__ inline WbPlanes wb_planes(int bits) { return WbPlanes{bits / 4, (bits % 4) >= 2 ? 1 : 0, bits & 1}; }

// position of code bit `plane bit` for (block i, K offset j) inside the lane's
// dwords: returns dword index and bit position
__device__ inline void wb_bit(const WbPlanes &P, int i, int j, int cb, int &dw, int &pos)
{
    const int q = j >> 1, h = (j & 1) * 16;
    if (P.n4 == 0 && P.n2 == 1 && P.n1 == 1) {             // b = 3: nibble-aligned dwords
        dw = i < 3 ? i : cb;
        pos = 4 * w4_slot(j) + (i < 3 ? cb : 3);
        return;
    }
    if (P.n4 == 2 && P.n2 == 0 && P.n1 == 0) {             // b = 8: a byte per code
        dw = 2 * i + (j >> 2);
        pos = 8 * (((j & 1) << 1) | ((j >> 1) & 1)) + cb;  // K offsets 4h, 4h+2, 4h+1, 4h+3 in bytes 0..3
        return;
    }
    if (cb < 4 * P.n4) {                                   // a 4-bit plane
        dw = (cb / 4) * 4 + i;
        pos = 4 * w4_slot(j) + (cb & 3);
    } else if (P.n2 && cb < 4 * P.n4 + 2) {                // the 2-bit plane
        dw = 4 * P.n4 + i / 2;
        pos = h + 2 * (4 * (i & 1) + q) + (cb - 4 * P.n4);
    } else {                                               // the 1-bit plane
        dw = 4 * P.n4 + 2 * P.n2;
        pos = h + 4 * i + q;
    }
}

// one thread per (tile, lane): its 32 codes -> `bits` dwords
__global__ void wb_pack_codes(const uint8_t *__restrict__ codes, uint32_t *__restrict__ out, int64_t N, int64_t K,
                              int64_t ktiles, int bits, int64_t total)
{
    const int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 6;
    const int lane = (int)(d & 63);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + (lane & 15);
    const WbPlanes P = wb_planes(bits);
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < 4; ++i) {
        const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
        if (n >= N || kb >= K) continue;                   // K % 32 == 0: the 8 codes are inside the row
        for (int j = 0; j < 8; ++j) {
            const uint32_t c = codes[n * K + kb + j];
            for (int cb = 0; cb < bits; ++cb) {
                int dw, pos;
                wb_bit(P, i, j, cb, dw, pos);
                w[dw] |= ((c >> cb) & 1u) << pos;
            }
        }
    }
    for (int k = 0; k < bits; ++k) out[tile * 64 * bits + wb_word(bits, lane, k)] = w[k];
}

__global__ void wb_unpack_codes(const uint32_t *__restrict__ in, uint8_t *__restrict__ codes, int64_t N, int64_t K,
                                int64_t ktiles, int bits, int64_t total)
{
    const int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 6;
    const int lane = (int)(d & 63);
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + (lane & 15);
    const WbPlanes P = wb_planes(bits);
    uint32_t w[8];
    for (int k = 0; k < bits; ++k) w[k] = in[tile * 64 * bits + wb_word(bits, lane, k)];
    for (int i = 0; i < 4; ++i) {
        const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
        if (n >= N || kb >= K) continue;
        for (int j = 0; j < 8; ++j) {
            uint32_t c = 0;
            for (int cb = 0; cb < bits; ++cb) {
                int dw, pos;
                wb_bit(P, i, j, cb, dw, pos);
                c |= ((w[dw] >> pos) & 1u) << cb;
            }
            codes[n * K + kb + j] = (uint8_t)c;
        }
    }
}

// fp32 dequant, one thread per (tile, lane): w = (q - z) * s exact in fp32
__global__ void wb_dequant_kernel(const uint32_t *__restrict__ in, const _Float16 *__restrict__ scales,
                                  const int8_t *__restrict__ zeros, float *__restrict__ wout, int64_t N, int64_t K,
                                  int G, int64_t ktiles, int bits, int64_t total)
{
    const int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (d >= total) return;
    const int64_t tile = d >> 6;
    const int lane = (int)(d & 63);
    const int r = lane & 15;
    const int64_t s = tile / ktiles, t = tile % ktiles;
    const int64_t n = s * 16 + r;
    const WbPlanes P = wb_planes(bits);
    const int gpt = 128 / G;
    uint32_t w[8];
    for (int k = 0; k < bits; ++k) w[k] = in[tile * 64 * bits + wb_word(bits, lane, k)];
    for (int i = 0; i < 4; ++i) {
        const int64_t kb = t * 128 + i * 32 + (lane >> 4) * 8;
        if (n >= N || kb >= K) continue;
        const int64_t meta = (tile * 16 + r) * gpt + (i * 32) / G;
        const float sc = (float)scales[meta];
        const int z = zeros ? (int)zeros[meta] : (1 << (bits - 1));
        for (int j = 0; j < 8; ++j) {
            int c = 0;
            for (int cb = 0; cb < bits; ++cb) {
                int dw, pos;
                wb_bit(P, i, j, cb, dw, pos);
                c |= (int)((w[dw] >> pos) & 1u) << cb;
            }
            wout[n * K + kb + j] = (float)(c - z) * sc;
        }
    }
}

// zero-fill of the alignment gaps between sections
void fill_gaps(const W4Layout &L, uint8_t *packed, hipStream_t s)
{
    const int64_t tiles = L.strips * L.ktiles;
    const int64_t gpt = 128 / L.G;
    const int64_t gaps[3][2] = {{L.codes_off + tiles * 256 * L.bits, L.scales_off},
                                {L.scales_off + tiles * 16 * gpt * 2, L.zeros_off},
                                {L.zeros_off + (L.asym ? tiles * 16 * gpt : 0), L.bytes}};
    for (auto &g : gaps)
        if (g[1] > g[0])
            fill_zero<<<blocks_for(g[1] - g[0]), kThreads, 0, s>>>(packed + g[0], g[1] - g[0]);
}

void pack_meta(const W4Layout &L, const uint16_t *scales, const int8_t *zeros, uint8_t *packed, hipStream_t s)
{
    const int64_t nm = L.strips * L.ktiles * 16 * (128 / L.G);
    if (nm == 0) return;
    w4_pack_meta<uint16_t><<<blocks_for(nm), kThreads, 0, s>>>(
        scales, reinterpret_cast<uint16_t *>(packed + L.scales_off), L.N, L.K, L.G, L.ktiles, nm);
    if (L.asym)
        w4_pack_meta<int8_t><<<blocks_for(nm), kThreads, 0, s>>>(
            zeros, reinterpret_cast<int8_t *>(packed + L.zeros_off), L.N, L.K, L.G, L.ktiles, nm);
}

void unpack_meta(const W4Layout &L, const uint8_t *packed, uint16_t *scales, int8_t *zeros, hipStream_t s)
{
    const int64_t nm = L.strips * L.ktiles * 16 * (128 / L.G);
    if (nm == 0) return;
    w4_unpack_meta<uint16_t><<<blocks_for(nm), kThreads, 0, s>>>(
        reinterpret_cast<const uint16_t *>(packed + L.scales_off), scales, L.N, L.K, L.G, L.ktiles, nm);
    if (L.asym)
        w4_unpack_meta<int8_t><<<blocks_for(nm), kThreads, 0, s>>>(
            reinterpret_cast<const int8_t *>(packed + L.zeros_off), zeros, L.N, L.K, L.G, L.ktiles, nm);
}

}  // namespace

hipError_t launch_wb_pack(const W4Layout &L, const uint8_t *codes, const uint16_t *scales, const int8_t *zeros,
                          uint8_t *packed, hipStream_t s)
{
    const int64_t nl = L.strips * L.ktiles * 64;
    if (nl > 0) {
        wb_pack_codes<<<blocks_for(nl), kThreads, 0, s>>>(codes, reinterpret_cast<uint32_t *>(packed + L.codes_off),
                                                          L.N, L.K, L.ktiles, L.bits, nl);
        pack_meta(L, scales, zeros, packed, s);
    }
    fill_gaps(L, packed, s);
    return hipGetLastError();
}

hipError_t launch_wb_unpack(const W4Layout &L, const uint8_t *packed, uint8_t *codes, uint16_t *scales,
                            int8_t *zeros, hipStream_t s)
{
    const int64_t nl = L.strips * L.ktiles * 64;
    if (nl == 0) return hipSuccess;
    wb_unpack_codes<<<blocks_for(nl), kThreads, 0, s>>>(reinterpret_cast<const uint32_t *>(packed + L.codes_off),
                                                        codes, L.N, L.K, L.ktiles, L.bits, nl);
    unpack_meta(L, packed, scales, zeros, s);
    return hipGetLastError();
}

hipError_t launch_wb_dequant(const W4Layout &L, const uint8_t *packed, float *w, hipStream_t s)
{
    const int64_t nl = L.strips * L.ktiles * 64;
    if (nl == 0) return hipSuccess;
    wb_dequant_kernel<<<blocks_for(nl), kThreads, 0, s>>>(
        reinterpret_cast<const uint32_t *>(packed + L.codes_off),
        reinterpret_cast<const _Float16 *>(packed + L.scales_off),
        L.asym ? reinterpret_cast<const int8_t *>(packed + L.zeros_off) : nullptr, w, L.N, L.K, L.G, L.ktiles,
        L.bits, nl);
    return hipGetLastError();
}

hipError_t launch_w4_pack(const W4Layout &L, const uint8_t *codes, const uint16_t *scales,
                          const int8_t *zeros, uint8_t *packed, hipStream_t s)
{
    const int64_t tiles = L.strips * L.ktiles;
    const int64_t gpt = 128 / L.G;
    if (tiles > 0) {
        const int64_t nd = tiles * 256;
        w4_pack_codes<<<blocks_for(nd), kThreads, 0, s>>>(codes, reinterpret_cast<uint32_t *>(packed + L.codes_off),
                                                          L.N, L.K, L.ktiles, nd);
        const int64_t nm = tiles * 16 * gpt;
        w4_pack_meta<uint16_t><<<blocks_for(nm), kThreads, 0, s>>>(
            scales, reinterpret_cast<uint16_t *>(packed + L.scales_off), L.N, L.K, L.G, L.ktiles, nm);
        if (L.asym)
            w4_pack_meta<int8_t><<<blocks_for(nm), kThreads, 0, s>>>(
                zeros, reinterpret_cast<int8_t *>(packed + L.zeros_off), L.N, L.K, L.G, L.ktiles, nm);
    }
    // the alignment gaps between sections are zero-filled so the blob is fully defined
    // (a fill kernel, not a memset node, so the call may be graph-captured)
    const int64_t gaps[3][2] = {{L.codes_off + tiles * 1024, L.scales_off},
                                {L.scales_off + tiles * 16 * gpt * 2, L.zeros_off},
                                {L.zeros_off + (L.asym ? tiles * 16 * gpt : 0), L.bytes}};
    for (auto &g : gaps)
        if (g[1] > g[0])
            fill_zero<<<blocks_for(g[1] - g[0]), kThreads, 0, s>>>(packed + g[0], g[1] - g[0]);
    return hipGetLastError();
}

hipError_t launch_w4_unpack(const W4Layout &L, const uint8_t *packed, uint8_t *codes,
                            uint16_t *scales, int8_t *zeros, hipStream_t s)
{
    const int64_t tiles = L.strips * L.ktiles;
    if (tiles == 0) return hipSuccess;
    const int64_t gpt = 128 / L.G;
    const int64_t nd = tiles * 256;
    w4_unpack_codes<<<blocks_for(nd), kThreads, 0, s>>>(reinterpret_cast<const uint32_t *>(packed + L.codes_off),
                                                        codes, L.N, L.K, L.ktiles, nd);
    const int64_t nm = tiles * 16 * gpt;
    w4_unpack_meta<uint16_t><<<blocks_for(nm), kThreads, 0, s>>>(
        reinterpret_cast<const uint16_t *>(packed + L.scales_off), scales, L.N, L.K, L.G, L.ktiles, nm);
    if (L.asym)
        w4_unpack_meta<int8_t><<<blocks_for(nm), kThreads, 0, s>>>(
            reinterpret_cast<const int8_t *>(packed + L.zeros_off), zeros, L.N, L.K, L.G, L.ktiles, nm);
    return hipGetLastError();
}

hipError_t launch_w4_dequant(const W4Layout &L, const uint8_t *packed, float *w, hipStream_t s)
{
    const int64_t tiles = L.strips * L.ktiles;
    if (tiles == 0) return hipSuccess;
    const int64_t nd = tiles * 256;
    w4_dequant_kernel<<<blocks_for(nd), kThreads, 0, s>>>(
        reinterpret_cast<const uint32_t *>(packed + L.codes_off),
        reinterpret_cast<const _Float16 *>(packed + L.scales_off),
        L.asym ? reinterpret_cast<const int8_t *>(packed + L.zeros_off) : nullptr,
        w, L.N, L.K, L.G, L.ktiles, nd);
    return hipGetLastError();
}

}  // namespace lowbit
