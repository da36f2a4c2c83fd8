// gemm_w4.hip -- prefill GEMM with packed INT4 weights on the matrix cores.
//
//   C[m][n] = sum_k A[m][k] * (q[n][k] - z) * s[n][k/G]      (fp32 accumulate)
//
// ("Low Bit ARM kernels": prefill is a GEMM over the same group-wise
// quantized weights; "Low Bit Metal Kernels", int4_matmul: an activation tile
// and a dequantized weight tile are staged in on-chip memory and multiplied.)
//
// MI355X design:
//   * Workgroup tile BM x BN, K in steps of 128 (one packed weight tile).  The
//     A tile (BM x 128, bf16 or fp16) is staged in LDS and shared by all
//     waves; each wave owns TN 16-column strips of the weight and reads its B
//     operands straight from the packed 16 x 128 tiles, already in the lane
//     order of v_mfma_f32_16x16x32_{bf16,f16}: no LDS traffic for B.
//   * Weights stay exact.  fp16 activations: B = q - z, formed exactly in
//     packed fp16 (as in the GEMV).  bf16 activations: gfx950 has no packed
//     bf16 add, so B = 128 + q (one mask+or with the bf16 constant 128.0, exact)
//     and the bias is removed with the row sums of the activations:
//       sum_k a (q - z) = sum_k a (128 + q) - (128 + z) * sum_k a
//     The row sums of each quantization group are taken (v_dot2_f32_bf16,
//     fp32) while the A tile is staged.
//   * Scales in fp32 with one accumulator set: before the MFMAs of group g
//     the accumulator (held in units of the previous group's scale) is
//     rescaled per column by s_prev / s_g and the group's bias correction is
//     added; the epilogue multiplies by the last scale.  A zero scale keeps
//     the unit and zeroes that column's operands for the group.
//   * Split-K over workgroups when the output tiles alone cannot fill the
//     256 CUs: fp32 partial tiles go to a workspace and a second kernel adds
//     them in a fixed order (deterministic) and rounds to the output type.
#include "lowbit_internal.hpp"

namespace lowbit {

namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

constexpr int kLdsRowHalfs = 128 + 8;             // A row in LDS: 128 K + 16 bytes of padding

template <typename T>
__device__ __forceinline__ T bitcast_u32(uint32_t v) { return __builtin_bit_cast(T, v); }

// 8 codes -> 8 exact fp16 values q - z (packed layout of lowbit_internal.hpp)
__device__ __forceinline__ h8 unpack_f16(uint32_t w, uint32_t magic, h2 blo, h2 bhi)
{
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    const h2 p0 = bitcast_u32<h2>((w & 0x000F000Fu) | magic) + blo;
    const h2 p1 = __builtin_elementwise_fma(bitcast_u32<h2>((w & 0x00F000F0u) | magic), sixteenth, bhi);
    const h2 p2 = bitcast_u32<h2>((w8 & 0x000F000Fu) | magic) + blo;
    const h2 p3 = __builtin_elementwise_fma(bitcast_u32<h2>((w8 & 0x00F000F0u) | magic), sixteenth, bhi);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 8 codes -> 8 exact bf16 values 128 + q (element j = K offset j)
__device__ __forceinline__ u4 unpack_bf16_biased(uint32_t w, uint32_t magic)
{
    u4 r;
    r.x = (w & 0x000F000Fu) | magic;                 // k+0, k+1
    r.y = ((w >> 4) & 0x000F000Fu) | magic;          // k+2, k+3
    r.z = ((w >> 8) & 0x000F000Fu) | magic;          // k+4, k+5
    r.w = ((w >> 12) & 0x000F000Fu) | magic;         // k+6, k+7
    return r;
}

template <int G, bool ASYM>
struct GemmMeta {
    uint32_t s[(128 / G + 1) / 2];
    uint32_t z;
};

template <int G, bool ASYM>
__device__ __forceinline__ GemmMeta<G, ASYM> gemm_load_meta(__amdgpu_buffer_rsrc_t srs, __amdgpu_buffer_rsrc_t zrs,
                                                            uint32_t idx, bool ok)
{
    constexpr int GPT = 128 / G;
    GemmMeta<G, ASYM> m;
    const uint32_t so = ok ? idx * GPT * 2 : kBufferOob;
    if constexpr (G == 128) m.s[0] = __builtin_amdgcn_raw_buffer_load_b16(srs, so, 0, 0);
    if constexpr (G == 64) m.s[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, 0);
    if constexpr (G == 32) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, so, 0, 0);
        m.s[0] = v[0];
        m.s[1] = v[1];
    }
    m.z = 0;
    if constexpr (ASYM) {
        const uint32_t zo = ok ? idx * GPT : kBufferOob;
        if constexpr (G == 128) m.z = __builtin_amdgcn_raw_buffer_load_b8(zrs, zo, 0, 0);
        if constexpr (G == 64) m.z = __builtin_amdgcn_raw_buffer_load_b16(zrs, zo, 0, 0);
        if constexpr (G == 32) m.z = __builtin_amdgcn_raw_buffer_load_b32(zrs, zo, 0, 0);
    }
    return m;
}

template <int G, bool ASYM>
__device__ __forceinline__ float meta_scale(const GemmMeta<G, ASYM> &m, int g)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(m.s[g / 2] >> (16 * (g & 1))));
}

template <int G, bool ASYM>
__device__ __forceinline__ int meta_zero(const GemmMeta<G, ASYM> &m, int g)
{
    if constexpr (ASYM) return (int)(int8_t)(uint8_t)(m.z >> (8 * g));
    return 8;
}

// Kernel parameters shared by the instantiations.
struct GemmArgs {
    const uint8_t *codes, *scales, *zeros;   // packed sections
    const uint16_t *a;                        // [M][K] bf16 or fp16 bits
    void *c;                                  // [M][N] output (bf16 / fp16), or fp32 partials when split
    float *part;                              // split-K partials [S][M][N]
    int M, N, K, ktiles, splits, c_bf16;
    int m_tiles, n_tiles;
};

// WM x WN waves; each wave owns TM x TN blocks of 16 x 16 outputs.
template <bool A_BF16, int G, bool ASYM, int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64, 2)
void gemm_w4_kernel(GemmArgs p)
{
    constexpr int NT = WM * WN * 64;                  // threads
    constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
    constexpr int GPT = 128 / G;
    constexpr int SPG = G / 32;                       // 32-K MFMA steps per group
    static_assert(NT == 2 * BM, "two staging threads per A row");
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsRowHalfs];
    __shared__ __attribute__((aligned(16))) float Rs[GPT][BM];   // activation row sums per group

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r16 = lane & 15, kq = lane >> 4;

    // tile coordinates; consecutive workgroups on one XCD (blockIdx % 8) walk
    // the N tiles of the same A rows so those rows stay in that XCD's L2
    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int split = lin % p.splits;
    const int tile = lin / p.splits;
    const int mt = tile / p.n_tiles, nt = tile % p.n_tiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const int kt0 = (int)((int64_t)p.ktiles * split / p.splits);
    const int kt1 = (int)((int64_t)p.ktiles * (split + 1) / p.splits);

    // A staging: thread -> row tid/2, 64 K (8 x 16 bytes) of the 128-K tile
    const int arow = tid >> 1, ahalf = tid & 1;
    const bool arow_ok = m0 + arow < p.M;
    const auto ars = buffer_rsrc(p.a, (uint32_t)((int64_t)p.M * p.K * 2));
    const uint32_t a_base = (uint32_t)(((int64_t)(m0 + arow) * p.K + ahalf * 64) * 2);

    // B: this wave's TN strips
    const int strip0 = n0 / 16 + wn * TN;
    const int strips_total = (p.N + 15) / 16;
    const auto crs = buffer_rsrc(p.codes, (uint32_t)((int64_t)strips_total * p.ktiles * 1024));
    const auto srs = buffer_rsrc(p.scales, (uint32_t)((int64_t)strips_total * p.ktiles * 16 * GPT * 2));
    const auto zrs = buffer_rsrc(ASYM ? p.zeros : p.scales, ASYM ? (uint32_t)((int64_t)strips_total * p.ktiles * 16 * GPT) : 0u);

    u4 areg[8];
    u4 bcur[TN], bnext[TN];
    GemmMeta<G, ASYM> mcur[TN], mnext[TN];

    auto load_a = [&](int kt) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // K % 32 == 0: an 8-element chunk is inside the row or wholly past K
            const bool ok = arow_ok && kt * 128 + ahalf * 64 + c * 8 < p.K;
            const uint32_t off = ok ? a_base + (uint32_t)kt * 256 + c * 16 : kBufferOob;
            areg[c] = __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0);
        }
    };
    auto load_b = [&](int kt, u4 *b, GemmMeta<G, ASYM> *m) {
#pragma unroll
        for (int nb = 0; nb < TN; ++nb) {
            const int s = strip0 + nb;
            const bool ok = s < strips_total;
            const uint32_t t = (uint32_t)s * p.ktiles + kt;
            b[nb] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? t * 1024 + lane * 16 : kBufferOob, 0, 0);
            m[nb] = gemm_load_meta<G, ASYM>(srs, zrs, t * 16 + r16, ok);
        }
    };

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    float unit[TN];                                   // current scale unit of each owned column
#pragma unroll
    for (int j = 0; j < TN; ++j) unit[j] = 1.0f;

    uint32_t magic = A_BF16 ? 0x43004300u : 0x64006400u;   // 128.0 (bf16) / 1024.0 (fp16)
    asm volatile("" : "+v"(magic));

    if (kt0 < kt1) {
        load_a(kt0);
        load_b(kt0, bcur, mcur);
    }
    for (int kt = kt0; kt < kt1; ++kt) {
        // 1. row sums of this thread's 64 activations, per quantization group
        //    (bf16 only), then the A tile and the sums go to LDS
        float rsum[2] = {0.f, 0.f};
        if constexpr (A_BF16) {
            const bf2v one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int h = (G == 32) ? (c >> 2) : 0;       // 32-K group within the 64-K half
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    rsum[h] = __builtin_amdgcn_fdot2_f32_bf16(bitcast_u32<bf2v>(areg[c][d]), one, rsum[h], false);
            }
        }
        __syncthreads();                              // previous tile fully consumed
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<u4 *>(&As[arow * kLdsRowHalfs + ahalf * 64 + c * 8]) = areg[c];
        if constexpr (A_BF16) {
            if constexpr (G == 128) {
                const float other = __shfl_xor(rsum[0], 1);
                if (ahalf == 0) Rs[0][arow] = rsum[0] + other;
            } else if constexpr (G == 64) {
                Rs[ahalf][arow] = rsum[0];
            } else {
                Rs[ahalf * 2][arow] = rsum[0];
                Rs[ahalf * 2 + 1][arow] = rsum[1];
            }
        }
        __syncthreads();

        // 2. prefetch the next K tile while this one is multiplied
        if (kt + 1 < kt1) {
            load_a(kt + 1);
            load_b(kt + 1, bnext, mnext);
        }

        // 3. per quantization group: rescale + bias correction, then MFMAs
#pragma unroll
        for (int g = 0; g < GPT; ++g) {
            float ratio[TN];
            float bz[TN];                              // -(128 + z) for the bf16 bias correction
            bool zcol[TN];
            bool anyzero = false;
#pragma unroll
            for (int nb = 0; nb < TN; ++nb) {
                const float s = meta_scale<G, ASYM>(mcur[nb], g);
                zcol[nb] = (s == 0.0f);
                anyzero |= zcol[nb];
                ratio[nb] = zcol[nb] ? 1.0f : unit[nb] * __builtin_amdgcn_rcpf(s);
                unit[nb] = zcol[nb] ? unit[nb] : s;
                bz[nb] = zcol[nb] ? 0.0f : -(128.0f + (float)meta_zero<G, ASYM>(mcur[nb], g));
            }
            // zero scales are rare: one wave-uniform test
            const bool wave_zero = __builtin_amdgcn_ballot_w64(anyzero) != 0;
            // acc <- acc * ratio (+ bias correction of this group, bf16 only)
#pragma unroll
            for (int mb = 0; mb < TM; ++mb) {
                f4 rrow = {0.f, 0.f, 0.f, 0.f};
                if constexpr (A_BF16) {
                    const int row = wm * TM * 16 + mb * 16 + kq * 4;
                    rrow = *reinterpret_cast<const f4 *>(&Rs[g][row]);
                }
#pragma unroll
                for (int nb = 0; nb < TN; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (A_BF16)
                            acc[mb][nb][i] = __builtin_fmaf(acc[mb][nb][i], ratio[nb], rrow[i] * bz[nb]);
                        else
                            acc[mb][nb][i] = acc[mb][nb][i] * ratio[nb];
                    }
            }
#pragma unroll
            for (int ss = 0; ss < SPG; ++ss) {
                const int ks = g * SPG + ss;           // 32-K step inside the tile
                u4 bops[TN];
#pragma unroll
                for (int nb = 0; nb < TN; ++nb) {
                    const uint32_t w = bcur[nb][ks];
                    if constexpr (A_BF16) {
                        bops[nb] = unpack_bf16_biased(w, magic);
                    } else {
                        const int z = meta_zero<G, ASYM>(mcur[nb], g);
                        const _Float16 lo = (_Float16)(-1024.0f - (float)z);
                        const _Float16 hi = (_Float16)(-64.0f - (float)z);
                        bops[nb] = __builtin_bit_cast(u4, unpack_f16(w, magic, h2{lo, lo}, h2{hi, hi}));
                    }
                    if (wave_zero && zcol[nb]) bops[nb] = u4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int mb = 0; mb < TM; ++mb) {
                    const int row = wm * TM * 16 + mb * 16 + r16;
                    const u4 av = *reinterpret_cast<const u4 *>(&As[row * kLdsRowHalfs + ks * 32 + kq * 8]);
#pragma unroll
                    for (int nb = 0; nb < TN; ++nb) {
                        if constexpr (A_BF16)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf8v, av), __builtin_bit_cast(bf8v, bops[nb]), acc[mb][nb], 0, 0, 0);
                        else
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(h8, av), __builtin_bit_cast(h8, bops[nb]), acc[mb][nb], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int nb = 0; nb < TN; ++nb) {
            bcur[nb] = bnext[nb];
            mcur[nb] = mnext[nb];
        }
    }

    // 4. epilogue: back to real units; C layout of the 16x16 MFMA: lane holds
    //    column (lane % 16) and rows 4*(lane / 16) + i of each block
#pragma unroll
    for (int mb = 0; mb < TM; ++mb)
#pragma unroll
        for (int nb = 0; nb < TN; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * TM * 16 + mb * 16 + kq * 4 + i;
                const int n = n0 + wn * TN * 16 + nb * 16 + r16;
                if (m < p.M && n < p.N) {
                    const float v = acc[mb][nb][i] * unit[nb];
                    const int64_t o = (int64_t)m * p.N + n;
                    if (p.splits > 1)
                        p.part[(int64_t)split * p.M * p.N + o] = v;
                    else if (p.c_bf16)
                        reinterpret_cast<__bf16 *>(p.c)[o] = (__bf16)v;
                    else
                        reinterpret_cast<_Float16 *>(p.c)[o] = (_Float16)v;
                }
            }
}

// Split-K reduction: C = round(sum_{s=0}^{S-1} part[s]) in a fixed order.
__global__ void gemm_splitk_reduce(const float *__restrict__ part, void *__restrict__ c, int64_t MN, int S,
                                   int c_bf16)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(int64_t)s * MN + i];
    if (c_bf16)
        reinterpret_cast<__bf16 *>(c)[i] = (__bf16)v;
    else
        reinterpret_cast<_Float16 *>(c)[i] = (_Float16)v;
}

struct GemmPlan {
    int splits;
    int m_tiles, n_tiles;
};

// 128 x 128 output tiles (4 waves of 64 x 64); split K over workgroups while
// the tiles alone give fewer than 256 work units and each split keeps >= 8
// K tiles.
GemmPlan plan_gemm(int M, int N, int K)
{
    const int ktiles = (K + 127) / 128;
    GemmPlan pl;
    pl.m_tiles = (M + 127) / 128;
    pl.n_tiles = (N + 127) / 128;
    const int64_t tiles = (int64_t)pl.m_tiles * pl.n_tiles;
    pl.splits = 1;
    while (tiles * pl.splits < 256 && ktiles / (pl.splits * 2) >= 8) pl.splits *= 2;
    return pl;
}

template <bool A_BF16, int G, bool ASYM>
hipError_t launch_cfg(const GemmPlan &pl, const GemmArgs &a, hipStream_t s)
{
    const unsigned blocks = (unsigned)((int64_t)pl.m_tiles * pl.n_tiles * pl.splits);
    gemm_w4_kernel<A_BF16, G, ASYM, 2, 2, 4, 4><<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <bool A_BF16>
hipError_t launch_dtype(const GemmPlan &pl, const W4Layout &L, const GemmArgs &a, hipStream_t s)
{
    switch (L.G) {
    case 32: return L.asym ? launch_cfg<A_BF16, 32, true>(pl, a, s) : launch_cfg<A_BF16, 32, false>(pl, a, s);
    case 64: return L.asym ? launch_cfg<A_BF16, 64, true>(pl, a, s) : launch_cfg<A_BF16, 64, false>(pl, a, s);
    default: return L.asym ? launch_cfg<A_BF16, 128, true>(pl, a, s) : launch_cfg<A_BF16, 128, false>(pl, a, s);
    }
}

}  // namespace

size_t gemm_w4_workspace(int M, int64_t N, int64_t K, int)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const GemmPlan pl = plan_gemm(M, (int)N, (int)K);
    if (pl.splits <= 1) return 0;
    return (size_t)pl.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_gemm_w4(const W4Layout &L, int M, const uint8_t *packed, const void *a, int a_bf16, void *c,
                          int c_bf16, void *ws, size_t ws_bytes, hipStream_t s)
{
    if (M == 0 || L.N == 0) return hipSuccess;
    const int N = (int)L.N, K = (int)L.K;
    const GemmPlan pl = plan_gemm(M, N, K);
    GemmArgs ga;
    ga.codes = packed + L.codes_off;
    ga.scales = packed + L.scales_off;
    ga.zeros = L.asym ? packed + L.zeros_off : nullptr;
    ga.a = static_cast<const uint16_t *>(a);
    ga.c = c;
    ga.part = static_cast<float *>(ws);
    ga.M = M;
    ga.N = N;
    ga.K = K;
    ga.ktiles = (int)L.ktiles;
    ga.splits = pl.splits;
    ga.c_bf16 = c_bf16;
    ga.m_tiles = pl.m_tiles;
    ga.n_tiles = pl.n_tiles;
    if (pl.splits > 1 && (ws == nullptr || ws_bytes < gemm_w4_workspace(M, N, K, L.G)))
        return hipErrorInvalidValue;
    hipError_t e = a_bf16 ? launch_dtype<true>(pl, L, ga, s) : launch_dtype<false>(pl, L, ga, s);
    if (e != hipSuccess || pl.splits == 1) return e;
    const int64_t MN = (int64_t)M * N;
    gemm_splitk_reduce<<<(unsigned)((MN + 255) / 256), 256, 0, s>>>(ga.part, c, MN, pl.splits, c_bf16);
    return hipGetLastError();
}

}  // namespace lowbit
