// gemv_w4.hip -- decode GEMV / small-batch product with packed INT4 weights.
//
// Computes y[m][n] = sum_k x[m][k] * (q[n][k] - z) * s[n][k/G] for M <= 16
// ("Low Bit Metal Kernels", int4_matmul: dequantize each nibble with its
// group's scale just before the multiply-add; "Low Bit ARM kernels": decode at
// batch 1 is a GEMV bound by the weight bytes, group-wise scales with an
// optional int8 zero point).
//
// MI355X design (not the pages' Metal/NEON tiling):
//   * The weight streams from HBM exactly once, as one coalesced 16-byte load
//     per lane per 1 KiB tile (16 rows x 128 K), in the packed layout of
//     lowbit_internal.hpp.
//   * Unpack in registers: a mask+or of the packed dword with 0x6400 (fp16
//     1024.0) gives 1024 + q in each fp16 half; one packed fp16 add (or fma
//     by 1/16 for the nibbles that sit 4 bits higher) subtracts 1024 + z.
//     The result q - z is an exact small integer in fp16.
//   * The dot product runs on the matrix cores: v_mfma_f32_16x16x32_f16 with
//     the activations as A (M <= 16 rows, padded) and q - z as B; each MFMA
//     covers 32 K of 16 rows.  MFMAs of one quantization group chain in fp32,
//     then the group's fp32 scale multiplies the chain into the running sum,
//     so no weight is ever rounded (the scale is applied in fp32, not folded
//     into a 16-bit operand).
//   * The waves of a workgroup split one 16-row strip along K; their fp32
//     partial sums are added through LDS in a fixed order (deterministic),
//     then rounded to fp16 (RNE).
#include "lowbit_internal.hpp"

namespace lowbit {

namespace {

constexpr int kMaxWaves = 8;
constexpr int kUnroll = 4;

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

// per-tile group metadata of one lane's row: GPT scales (and zero points)
template <int G, bool ASYM> struct MetaRaw;
template <> struct MetaRaw<128, false> { uint16_t s; };
template <> struct MetaRaw<64, false> { uint32_t s; };
template <> struct MetaRaw<32, false> { uint2 s; };
template <> struct MetaRaw<128, true> { uint16_t s; uint8_t z; };
template <> struct MetaRaw<64, true> { uint32_t s; uint16_t z; };
template <> struct MetaRaw<32, true> { uint2 s; uint32_t z; };

template <int G, bool ASYM>
__device__ __forceinline__ MetaRaw<G, ASYM> load_meta(const uint8_t *scales, const uint8_t *zeros, int64_t idx)
{
    // idx = (tile * 16 + row) ; GPT entries per row
    constexpr int GPT = 128 / G;
    MetaRaw<G, ASYM> m;
    if constexpr (G == 128) m.s = reinterpret_cast<const uint16_t *>(scales)[idx];
    if constexpr (G == 64) m.s = reinterpret_cast<const uint32_t *>(scales)[idx];
    if constexpr (G == 32) m.s = reinterpret_cast<const uint2 *>(scales)[idx];
    if constexpr (ASYM) {
        if constexpr (G == 128) m.z = zeros[idx];
        if constexpr (G == 64) m.z = reinterpret_cast<const uint16_t *>(zeros)[idx];
        if constexpr (G == 32) m.z = reinterpret_cast<const uint32_t *>(zeros)[idx];
    }
    (void)GPT;
    return m;
}

template <int G, bool ASYM>
__device__ __forceinline__ void decode_meta(const MetaRaw<G, ASYM> &m, float *sc, h2 *blo, h2 *bhi)
{
    constexpr int GPT = 128 / G;
    uint32_t sw[2];
    if constexpr (G == 128) { sw[0] = m.s; }
    if constexpr (G == 64) { sw[0] = m.s; }
    if constexpr (G == 32) { sw[0] = m.s.x; sw[1] = m.s.y; }
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
        const uint16_t hb = (uint16_t)(sw[g / 2] >> (16 * (g & 1)));
        sc[g] = (float)__builtin_bit_cast(_Float16, hb);
        int z = 8;
        if constexpr (ASYM) z = (int)(int8_t)(uint8_t)(m.z >> (8 * g));
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
    decode_meta<G, ASYM>(mr, sc, blo, bhi);
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

template <int G, bool ASYM, int MR>
__global__ __launch_bounds__(kMaxWaves * 64)
void gemv_w4_kernel(const u4 *__restrict__ codes, const uint8_t *__restrict__ scales,
                    const uint8_t *__restrict__ zeros, const _Float16 *__restrict__ x,
                    _Float16 *__restrict__ y, int M, int N, int K, int ktiles)
{
    __shared__ float red[kMaxWaves][MR][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int W = blockDim.x >> 6;
    const int strip = blockIdx.x;
    const int r = lane & 15;                         // B column (weight row) and A row (token)
    const int kq = lane >> 4;                        // 8-K slice inside each 32-K MFMA block
    // A row r only feeds C row r, so lanes past M read a valid row (M - 1) and
    // their results are never stored: the activation loads need no mask.
    const _Float16 *xr = x + (int64_t)(r < M ? r : M - 1) * K + kq * 8;
    const u4 *cw = codes + (int64_t)strip * ktiles * 64 + lane;
    const int64_t meta0 = (int64_t)strip * ktiles * 16 + r;
    const int full = K / 128;                        // tiles with all 128 K inside the matrix

    uint32_t magic = 0x64006400u;                    // fp16 1024.0 in both halves
    asm volatile("" : "+v"(magic));                  // keep it in a register: mask+or becomes one op

    f4 acc = {0.f, 0.f, 0.f, 0.f};

    for (int t0 = wave; t0 < full; t0 += W * kUnroll) {
        u4 q[kUnroll];
        MetaRaw<G, ASYM> mr[kUnroll];
        h8 a[kUnroll][4];
        // issue every load of the unrolled tiles before any arithmetic
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = t0 + u * W;
            if (t < full) {
                q[u] = __builtin_nontemporal_load(cw + (int64_t)t * 64);
                mr[u] = load_meta<G, ASYM>(scales, zeros, meta0 + (int64_t)t * 16);
                const _Float16 *xt = xr + t * 128;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[u][i] = *reinterpret_cast<const h8 *>(xt + i * 32);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = t0 + u * W;
            if (t < full) tile_product<G, ASYM, MR>(q[u], mr[u], a[u], magic, acc);
        }
    }
    // ragged last tile (K % 128 != 0): its 32-K blocks past K read zeros
    if (full < ktiles && wave == full % W) {
        const int t = full;
        const u4 q = cw[(int64_t)t * 64];
        const MetaRaw<G, ASYM> mr = load_meta<G, ASYM>(scales, zeros, meta0 + (int64_t)t * 16);
        h8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = t * 128 + i * 32;
            a[i] = h8{};
            if (k < K) a[i] = *reinterpret_cast<const h8 *>(xr + k);
        }
        tile_product<G, ASYM, MR>(q, mr, a, magic, acc);
    }

    if (W > 1) {
#pragma unroll
        for (int j = 0; j < MR; ++j) red[wave][j][lane] = acc[j];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                float s = red[0][j][lane];
                for (int w = 1; w < W; ++w) s += red[w][j][lane];
                acc[j] = s;
            }
        }
    }
    if (wave == 0) {
        // C layout of the 16x16 MFMA: lane holds column (lane % 16), rows 4*(lane / 16) + j
        const int n = strip * 16 + r;
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const int m = kq * 4 + j;
            if (m < M && n < N) y[(int64_t)m * N + n] = (_Float16)acc[j];
        }
    }
}

template <int G, bool ASYM>
hipError_t launch_gm(int MR, dim3 grid, dim3 block, hipStream_t s, const u4 *codes, const uint8_t *scales,
                     const uint8_t *zeros, const _Float16 *x, _Float16 *y, int M, int N, int K, int ktiles)
{
    if (MR == 1)
        gemv_w4_kernel<G, ASYM, 1><<<grid, block, 0, s>>>(codes, scales, zeros, x, y, M, N, K, ktiles);
    else if (MR == 2)
        gemv_w4_kernel<G, ASYM, 2><<<grid, block, 0, s>>>(codes, scales, zeros, x, y, M, N, K, ktiles);
    else
        gemv_w4_kernel<G, ASYM, 4><<<grid, block, 0, s>>>(codes, scales, zeros, x, y, M, N, K, ktiles);
    return hipGetLastError();
}

}  // namespace

size_t gemv_w4_workspace(int, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemv_w4(const W4Layout &L, int M, const uint8_t *packed, const _Float16 *x,
                          _Float16 *y, void *, size_t, hipStream_t s)
{
    if (M == 0 || L.N == 0) return hipSuccess;
    // waves per workgroup: about four 1 KiB tiles per wave along the strip's K
    const int64_t kt = L.ktiles;
    int W = (int)((kt + kUnroll - 1) / kUnroll);
    if (W < 1) W = 1;
    if (W > kMaxWaves) W = kMaxWaves;
    const dim3 grid((unsigned)L.strips), block((unsigned)(W * 64));
    const int MR = M == 1 ? 1 : (M == 2 ? 2 : 4);
    const u4 *codes = reinterpret_cast<const u4 *>(packed + L.codes_off);
    const uint8_t *scales = packed + L.scales_off;
    const uint8_t *zeros = L.asym ? packed + L.zeros_off : nullptr;
    const int N = (int)L.N, K = (int)L.K, ktiles = (int)L.ktiles;
    switch (L.G) {
    case 32:
        return L.asym ? launch_gm<32, true>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles)
                      : launch_gm<32, false>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles);
    case 64:
        return L.asym ? launch_gm<64, true>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles)
                      : launch_gm<64, false>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles);
    default:
        return L.asym ? launch_gm<128, true>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles)
                      : launch_gm<128, false>(MR, grid, block, s, codes, scales, zeros, x, y, M, N, K, ktiles);
    }
}

}  // namespace lowbit
