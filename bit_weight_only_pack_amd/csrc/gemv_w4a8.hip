// gemv_w4a8.hip -- W4A8: packed INT4 weights against dynamically quantized
// INT8 activations, on the int8 matrix cores.
//
// What is computed ("Low Bit ARM kernels", measurements section: 4-bit weights
// with dynamic INT8 activations at group size 32; NEON/I8MM section: the
// unpacked weights stay int8 and feed int8 matrix-multiply instructions that
// accumulate in int32).  Per token row m:
//   amax = max_k |x[m][k]|,  inv = fl32(127 / amax),  s[m] = fl32(amax / 127)
//   xq[m][k] = rint(fl32(x[m][k] * inv))                  (0 for a zero row)
//   y[m][n]  = s[m] * sum_g sw[n][g] * ( sum_{k in g} xq[m][k] q[n][k]
//                                        - z[n][g] sum_{k in g} xq[m][k] )
// The bracket is an exact int32; the scales are applied in fp32 and y is
// rounded to nearest even into fp16.
//
// MI355X design:
//   * Weights: the packed blob of lowbit_pack_weights, unchanged.  One dword
//     of a lane holds 8 codes of one weight row; masking it with 0x0F0F0F0F
//     before and after a 4-bit shift gives them as unsigned bytes, which is
//     the B operand of v_mfma_i32_16x16x32_i8 (3 operations per 8 weights,
//     and no per-weight zero-point arithmetic: z enters once per group).
//   * Activations: an "activation block" holds, per 8-K block kb and token m,
//     the 8 codes in the byte order of the unpacked weights (K offsets 0 4 1 5
//     2 6 3 7), then the code sums per (group, token), then the per-token
//     scales.  The tile loop reads only this block, from LDS.
//   * Fused form (one token): each workgroup stages its problem's fp16 x in
//     LDS and builds the block itself (every workgroup computes the same
//     codes), so a projection costs one launch.  From two tokens on,
//     quant_act_kernel writes the block to a workspace once and the GEMV
//     copies it into LDS (cheaper than re-quantizing in every workgroup).
//   * Schedule of the W4A16 streaming GEMV: one workgroup per 16-row strip,
//     waves split K into runs of at most 8 tiles, every weight load issued up
//     front with the non-temporal hint, fixed-order cross-wave sum.
#include <mutex>

#include "lowbit_internal.hpp"
#include "gemv_tile.hpp"

namespace lowbit {

// Scratch for the entry point that allocates nothing
// (lowbit_gemv_w4a8_batched_noalloc): the activation blocks of up to eight
// problems, written by quant_act_kernel and read by the GEMV of the same
// call.  Each GPU the library runs on holds one copy until the process ends.
// In host code `scratch` is only a stand-in for the symbol; kernels receive
// the device address that w4a8_scratch() looked up for the current device.
static __device__ __align__(256) uint8_t scratch[kW4a8ScratchBytes];

hipError_t w4a8_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // once per device, with that device current: each GPU has its own copy
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

using namespace tile;

typedef int i4v __attribute__((ext_vector_type(4)));

constexpr int kA8FusedMaxLds = 80 * 1024;        // two workgroups per compute unit
constexpr int kA8MaxLds = 160 * 1024;            // one workgroup per compute unit

// slots per group in the code-sum table: M rounded up to a power of two
__host__ __device__ inline int a8_ms(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// Activation block of M tokens over kt K tiles: codes, code sums, scales.
// Offsets are bytes from the block start; the size is a whole number of KiB.
struct A8Block {
    int img, xs, sx, bytes;
};
__host__ __device__ inline A8Block a8_block(int M, int kt, int G)
{
    A8Block b;
    b.img = 0;
    b.xs = kt * 128 * M;
    b.sx = b.xs + (kt * 128 / G) * a8_ms(M) * 4;
    b.bytes = (int)round_up(b.sx + 16 * 4, 1024);
    return b;
}

// LDS of the GEMV: the block, the cross-wave sums, then (fused) 1 KiB of
// per-wave maxima and the fp16 staging of x.  The sums do not share the
// staging: a wave that has finished its tiles writes its partial sums while
// slower waves may still be quantizing from the staging.
struct A8Lds {
    int red, amx, xf, total;
};
__host__ __device__ inline A8Lds a8_lds(int M, int K, int kt, int G, int W, int MR, bool fused)
{
    const A8Block b = a8_block(M, kt, G);
    A8Lds l;
    l.red = b.bytes;
    l.amx = l.red + (W > 1 ? kRedSlots * MR * 64 * 4 : 0);
    l.xf = fused ? l.amx + 1024 : l.amx;
    l.total = l.xf + (fused ? M * (int)round_up(K, 512) * 2 : 0);
    return l;
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// workgroup barrier without the vmcnt(0) of __syncthreads
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// this wave's LDS writes done, then a workgroup barrier (weight loads stay in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Codes of 8 activations, as the low bytes of fl32(fl32(x * inv) + 1.5 * 2^23):
// the product is rounded to binary32 first (as the definition does), then the
// add rounds it to an integer, ties to even, in the unit place of [2^23, 2^24);
// |x * inv| <= 127.00002, so the integer is the code and no clamp is needed
// (its bits are 0x4B400000 + code, whose low byte is the code's byte).
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
constexpr float kRoundMagic = 12582912.0f;           // 1.5 * 2^23
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

__device__ __forceinline__ void a8_codes8(h8 v, float inv, uint32_t *bits)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float t = __fmul_rn((float)v[i], inv);
        asm volatile("" : "+v"(t));                   // two roundings: no fused multiply-add
        bits[i] = __builtin_bit_cast(uint32_t, t + kRoundMagic);
    }
}

// the block's two dwords of 8 codes: bytes ordered by K offsets 0 4 1 5 | 2 6 3 7
// (the byte order of the unpacked weight dword); v_perm_b32 picks byte 0 of
// two sources per half-word
__device__ __forceinline__ uint2 a8_pack(const uint32_t *b)
{
    // selector bytes: 0 = byte 0 of the second operand, 4 = byte 0 of the first
    const uint32_t p04 = __builtin_amdgcn_perm(b[4], b[0], 0x0C0C0400u);   // [c0, c4, 0, 0]
    const uint32_t p15 = __builtin_amdgcn_perm(b[5], b[1], 0x04000C0Cu);   // [0, 0, c1, c5]
    const uint32_t p26 = __builtin_amdgcn_perm(b[6], b[2], 0x0C0C0400u);
    const uint32_t p37 = __builtin_amdgcn_perm(b[7], b[3], 0x04000C0Cu);
    return make_uint2(p04 | p15, p26 | p37);
}

// largest magnitude of 8 fp16 values as fp16 bits (non-negative fp16 bit
// patterns order as unsigned integers), folded into m
__device__ __forceinline__ us2 a8_absmax8(h8 v, us2 m)
{
    const u4 w = __builtin_bit_cast(u4, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu));
    return m;
}

// Cross-lane steps on the DPP path (no LDS round trip): swap lanes within
// pairs and within halves of each quad, mirror each half-row (8 lanes) and
// each row (16 lanes).
__device__ __forceinline__ int dpp_pair(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_quad(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_half_mirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); }

// Sum of v over aligned groups of `n` lanes (n = 4, 8 or 16); every lane of
// a group must be active.  After each step every lane of the combined span
// holds the span's sum.
template <int n>
__device__ __forceinline__ int seg_sum(int v)
{
    static_assert(n == 4 || n == 8 || n == 16, "group of 4, 8 or 16 lanes");
    v += dpp_pair(v);
    v += dpp_quad(v);
    if constexpr (n >= 8) v += dpp_half_mirror(v);
    if constexpr (n >= 16) v += dpp_mirror(v);
    return v;
}

// Maximum of a non-negative float over the wave (all lanes active): the bit
// patterns of non-negative floats order as integers.
__device__ __forceinline__ float wave_max_nonneg(float a)
{
    int v = __builtin_bit_cast(int, a);
    v = max(v, dpp_pair(v));
    v = max(v, dpp_quad(v));
    v = max(v, dpp_half_mirror(v));
    v = max(v, dpp_mirror(v));
    const int r = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                      max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
    return __builtin_bit_cast(float, r);
}

// Quantizes 8-K blocks kb of token m into the activation block `blk`
// (generic address space: LDS or global).  Lanes of a wave must hold
// consecutive kb of one token, in whole groups of G/8.
template <int G>
__device__ __forceinline__ void a8_put(uint8_t *blk, const A8Block &B, int M, int m, int kb, h8 v, float inv)
{
    uint32_t c[8];
    a8_codes8(v, inv, c);
    uint32_t usum = 0u - 8u * kRoundMagicBits;       // sum of codes = sum of bits - 8 * magic (mod 2^32)
#pragma unroll
    for (int i = 0; i < 8; ++i) usum += c[i];
    int sum = (int)usum;
    *reinterpret_cast<uint2 *>(blk + B.img + ((int64_t)kb * M + m) * 8) = a8_pack(c);
    sum = seg_sum<G / 8>(sum);
    if ((threadIdx.x & (G / 8 - 1)) == 0)
        reinterpret_cast<int *>(blk + B.xs)[(kb / (G / 8)) * a8_ms(M) + m] = sum;
}

// The GEMV's work for one strip.  xin: fp16 x [M][K] (FUSED) or the
// problem's activation block in the workspace.
template <int G, bool ASYM, int MR, int T, bool FUSED>
__device__ __forceinline__ void a8_strip(const uint8_t *codes, const uint8_t *scales, const uint8_t *zeros,
                                         const void *xin, _Float16 *yp, int N, int K, int kt, int tw, int M, int W,
                                         int strip)
{
    constexpr int GPT = 128 / G;
    constexpr int MPG = G / 32;                      // MFMAs per group
    constexpr int NW = T * (ASYM ? 3 : 2);           // weight + metadata loads per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, kq = lane >> 4;
    const int t0 = wave * tw;
    const A8Block B = a8_block(M, kt, G);
    const A8Lds L = a8_lds(M, K, kt, G, W, MR, FUSED);

    // 1. activations -> LDS (fused: fp16 x, rows padded to whole KiB; else
    //    the prepared block), by LDS-direct loads issued before the weights
    if constexpr (FUSED) {
        const auto xrs = buffer_rsrc(xin, (uint32_t)(M * K * 2));
        const int cpr = (int)(round_up(K, 512) >> 9);
        for (int m = 0; m < M; ++m)
            for (int cc = wave; cc < cpr; cc += W) {
                const int k = cc * 512 + lane * 8;
                lds_dma16(xrs, smem + L.xf + (m * cpr + cc) * 1024, k < K ? (uint32_t)((m * K + k) * 2) : kBufferOob);
            }
    } else {
        const auto brs = buffer_rsrc(xin, (uint32_t)B.bytes);
        for (int cc = wave; cc < (B.bytes >> 10); cc += W)
            lds_dma16(brs, smem + cc * 1024, (uint32_t)(cc * 1024 + lane * 16));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. weights and metadata of this wave's tiles, tile by tile; 3. the
    //    activation loads landed (issued first; loads retire in order),
    //    waited for after the first EARLY tiles' loads (eight tiles per wave:
    //    after the first, so they do not land behind the compute unit's whole
    //    weight stream)
    u4 q[T];
    MetaRaw<G, ASYM> mr[T];
    constexpr int EARLY = T >= 8 ? 1 : T;
    constexpr int LPT = ASYM ? 3 : 2;                // loads per tile (codes, scales[, zeros])
    static_assert(NW == T * LPT, "load count");
    const int64_t tiles0 = (int64_t)strip * kt;
    const auto crs = buffer_rsrc(codes + tiles0 * 1024, (uint32_t)kt * 1024);
    const auto srs = buffer_rsrc(scales + tiles0 * 16 * GPT * 2, (uint32_t)kt * 16 * GPT * 2);
    const auto zrs = buffer_rsrc(ASYM ? zeros + tiles0 * 16 * GPT : scales, ASYM ? (uint32_t)kt * 16 * GPT : 0u);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u == EARLY) {
            wait_vm<EARLY * LPT>();
            wg_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        const int t = t0 + u;
        const bool ok = u < tw && t < kt;
        q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (uint32_t)t * 1024 + lane * 16 : kBufferOob, 0,
                                                     kStreamLoad);
        mr[u] = load_meta<G, ASYM>(srs, zrs, ok ? t * 16 + r : -1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (EARLY == T) {
        wait_vm<NW>();
        wg_barrier();
    }

    if constexpr (FUSED) {
        // 4. per-token maximum magnitude: each wave over the 8-K blocks of its
        //    own tiles (zero padding past K included), then across waves
        float *amx = reinterpret_cast<float *>(smem + L.amx);
        const int xrow = (int)round_up(K, 512) * 2;
        const int kb0 = t0 * 16, kb1 = (t0 + max(min(tw, kt - t0), 0)) * 16;
        for (int m = 0; m < M; ++m) {
            us2 mm = {0, 0};
            for (int kb = kb0 + lane; kb < kb1; kb += 64)
                mm = a8_absmax8(*reinterpret_cast<const h8 *>(smem + L.xf + m * xrow + kb * 16), mm);
            const unsigned short mh = mm.x > mm.y ? mm.x : mm.y;
            float a = (float)__builtin_bit_cast(_Float16, mh);
            a = wave_max_nonneg(a);
            if (lane == 0) amx[wave * 16 + m] = a;
        }
        lds_barrier();
        // 5. each wave writes the codes and code sums its own tiles read (its
        //    LDS writes precede its reads: a wave's LDS instructions execute
        //    in order), wave 0 the scales it applies at the end
        for (int m = 0; m < M; ++m) {
            float a = amx[m];
            for (int w = 1; w < W; ++w) a = __builtin_fmaxf(a, amx[w * 16 + m]);
            const float inv = a > 0.f ? __fdiv_rn(127.f, a) : 0.f;
            for (int kb = kb0 + lane; kb < kb1; kb += 64) {
                const h8 v = *reinterpret_cast<const h8 *>(smem + L.xf + m * xrow + kb * 16);
                a8_put<G>(smem, B, M, m, kb, v, inv);
            }
            if (wave == 0 && lane == 0) reinterpret_cast<float *>(smem + B.sx)[m] = __fdiv_rn(a, 127.f);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // 6. products, tile by tile in load order
    const int xr = a_token<MR>(r, M);
    const int MS = a8_ms(M);
    const int row0 = min(c_token<MR>(kq, 0), MS - MR);   // first token of this lane's C elements
    const uint8_t *img = smem + B.img + xr * 8;
    const int *xsum = reinterpret_cast<const int *>(smem + B.xs) + row0;
    const i4v zero4 = {0, 0, 0, 0};
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const int tvalid = min(tw, kt - t0);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u < tvalid) {
            __builtin_amdgcn_sched_barrier(0);
            const int t = t0 + u;
            u4 qv = q[u];
            asm volatile("" : "+v"(qv));
            MetaRaw<G, ASYM> mv = mr[u];
            pin_meta<G, ASYM>(mv);
            const uint32_t wd[4] = {qv.x, qv.y, qv.z, qv.w};
            int xs1[GPT];                            // MR == 1: the tile's GPT code sums, one read
            if constexpr (MR == 1) {
                const int *xs = xsum + t * GPT * MS;
                if constexpr (GPT == 4) {
                    if (MS == 1) {
                        const i4v v4 = *reinterpret_cast<const i4v *>(xs);
                        xs1[0] = v4.x; xs1[1] = v4.y; xs1[2] = v4.z; xs1[3] = v4.w;
                    } else {
#pragma unroll
                        for (int g = 0; g < GPT; ++g) xs1[g] = xs[g * MS];
                    }
                } else {
#pragma unroll
                    for (int g = 0; g < GPT; ++g) xs1[g] = xs[g * MS];
                }
            }
            i4v c = zero4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long a = *reinterpret_cast<const long *>(img + (int64_t)((t * 16 + i * 4 + kq) * M) * 8);
                const uint32_t lo = wd[i] & 0x0F0F0F0Fu, hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
                const long b = (long)(((uint64_t)hi << 32) | lo);
                c = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (i % MPG == 0) ? zero4 : c, 0, 0, 0);
                if (i % MPG == MPG - 1) {
                    const int g = i / MPG;
                    const int *xs = xsum + (t * GPT + g) * MS;
                    int xv[MR];
                    if constexpr (MR == 1) {
                        xv[0] = xs1[g];
                    } else if constexpr (MR == 4) {
                        const i4v v4 = *reinterpret_cast<const i4v *>(xs);
                        xv[0] = v4.x; xv[1] = v4.y; xv[2] = v4.z; xv[3] = v4.w;
                    } else {
#pragma unroll
                        for (int j = 0; j < MR; ++j) xv[j] = xs[j];
                    }
                    uint16_t hb;
                    if constexpr (G == 128) hb = (uint16_t)(mv.s[0] >> (16 * (r & 1)));
                    else hb = (uint16_t)(mv.s[g / 2] >> (16 * (g & 1)));
                    const float sc = (float)__builtin_bit_cast(_Float16, hb);
                    int z = 8;
                    if constexpr (ASYM) {
                        uint32_t zb;
                        if constexpr (G == 128) zb = mv.z >> (8 * (r & 3));
                        else if constexpr (G == 64) zb = mv.z >> (16 * (r & 1) + 8 * g);
                        else zb = mv.z >> (8 * g);
                        z = (int)(int8_t)(uint8_t)zb;
                    }
#pragma unroll
                    for (int j = 0; j < MR; ++j) acc[j] = __builtin_fmaf(sc, (float)(c[j] - z * xv[j]), acc[j]);
                }
            }
        }
    }

    // 7. fixed-order cross-wave sum (a balanced tree over the sixteen
    //    partial slots), y = fp16(s[m] * sum)
    float *red = reinterpret_cast<float *>(smem + L.red);
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
        const float *sxv = reinterpret_cast<const float *>(smem + B.sx);
        const int n = strip * 16 + r;
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const int m = c_token<MR>(kq, j);
            if (m < M && n < N) yp[(int64_t)m * N + n] = (_Float16)(sxv[m] * acc[j]);
        }
    }
}

// One problem: scalar kernel arguments only (preloaded into SGPRs).
template <int G, bool ASYM, int MR, int T, bool FUSED>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(T > 4 ? 4 : 6)))
void gemv_w4a8_single(const uint8_t *codes, const uint8_t *scales, const void *xin, _Float16 *yp, int N, int K,
                      int kt, int tw, int M, int W, const uint8_t *zeros)
{
    a8_strip<G, ASYM, MR, T, FUSED>(codes, scales, zeros, xin, yp, N, K, kt, tw, M, W, (int)blockIdx.x);
}

// Problems laid end to end over blockIdx.x (b.first[i] = first workgroup of
// problem i; unused entries hold INT_MAX).  NP = 4: every field of the four
// problems is read in one round of scalar loads and selected afterwards (a
// dependent second round would delay the first HBM load); NP = 8: the
// problem is found first, then its fields are read.
template <int G, bool ASYM, int MR, int T, bool FUSED, int NP>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(T > 4 ? 4 : 6)))
void gemv_w4a8_batch(const GemvBatch b)
{
    const int bx = (int)blockIdx.x;
    if constexpr (NP == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const GemvProblem &q = b.p[i];
            asm volatile("" ::"s"(q.codes), "s"(q.scales), "s"(q.zeros), "s"(q.x), "s"(q.y), "s"(q.N), "s"(q.K),
                         "s"(q.ktiles), "s"(q.tw));
        }
        asm volatile("" ::"s"(b.first[1]), "s"(b.first[2]), "s"(b.first[3]), "s"(b.M), "s"(b.W));
        const int f1 = b.first[1], f2 = b.first[2], f3 = b.first[3];
        const int pi = (bx >= f1 ? 1 : 0) + (bx >= f2 ? 1 : 0) + (bx >= f3 ? 1 : 0);
        auto field = [&](auto get) {
            const auto v0 = get(b.p[0]), v1 = get(b.p[1]), v2 = get(b.p[2]), v3 = get(b.p[3]);
            return pi == 0 ? v0 : pi == 1 ? v1 : pi == 2 ? v2 : v3;
        };
        const int strip = bx - (pi == 0 ? 0 : pi == 1 ? f1 : pi == 2 ? f2 : f3);
        a8_strip<G, ASYM, MR, T, FUSED>(field([](const GemvProblem &q) { return q.codes; }),
                                         field([](const GemvProblem &q) { return q.scales; }),
                                         field([](const GemvProblem &q) { return q.zeros; }),
                                         field([](const GemvProblem &q) { return (const void *)q.x; }),
                                         field([](const GemvProblem &q) { return q.y; }),
                                         field([](const GemvProblem &q) { return q.N; }),
                                         field([](const GemvProblem &q) { return q.K; }),
                                         field([](const GemvProblem &q) { return q.ktiles; }),
                                         field([](const GemvProblem &q) { return q.tw; }), b.M, b.W, strip);
    } else {
        int pi = 0;
#pragma unroll
        for (int i = 1; i < kMaxGemvBatch; ++i) pi += bx >= b.first[i] ? 1 : 0;
        const GemvProblem &p = b.p[pi];
        a8_strip<G, ASYM, MR, T, FUSED>(p.codes, p.scales, p.zeros, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W,
                                         bx - b.first[pi]);
    }
}

// Writes activation blocks (IMAGE) or canonical codes [M][K] + scales [M].
// One workgroup of 256 threads per (token row, problem).
struct A8QuantBatch {
    const _Float16 *x[kMaxGemvBatch];
    uint8_t *out[kMaxGemvBatch];     // IMAGE: block; else int8 codes [M][K]
    float *sx[kMaxGemvBatch];        // canonical scales (unused for IMAGE)
    int K[kMaxGemvBatch], kt[kMaxGemvBatch];
    int M;
};

// One 256-thread workgroup per token row m of one problem: the row's
// maximum magnitude, then its codes (IMAGE: into the GEMV's prepared block;
// else int8 [M][K] and the canonical scale).
template <int G, bool IMAGE>
__device__ __forceinline__ void quant_act_row(const _Float16 *x, uint8_t *out, float *sx, int K, int kt, int M, int m)
{
    __shared__ float wmax[4];
    const _Float16 *xr = x + (int64_t)m * K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    us2 mm = {0, 0};
    for (int c = threadIdx.x; c < K / 8; c += 256) mm = a8_absmax8(*reinterpret_cast<const h8 *>(xr + c * 8), mm);
    float a = (float)__builtin_bit_cast(_Float16, (unsigned short)(mm.x > mm.y ? mm.x : mm.y));
    a = wave_max_nonneg(a);
    if (lane == 0) wmax[wave] = a;
    __syncthreads();
    a = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    const float inv = a > 0.f ? __fdiv_rn(127.f, a) : 0.f;
    const float s = __fdiv_rn(a, 127.f);
    if constexpr (IMAGE) {
        const A8Block B = a8_block(M, kt, G);
        uint8_t *blk = out;
        for (int kb = threadIdx.x; kb < kt * 16; kb += 256) {
            h8 v = {};
            if (kb * 8 < K) v = *reinterpret_cast<const h8 *>(xr + kb * 8);
            a8_put<G>(blk, B, M, m, kb, v, inv);
        }
        if (threadIdx.x == 0) reinterpret_cast<float *>(blk + B.sx)[m] = s;
    } else {
        uint8_t *o = out + (int64_t)m * K;
        for (int c = threadIdx.x; c < K / 8; c += 256) {
            const h8 v = *reinterpret_cast<const h8 *>(xr + c * 8);
            uint32_t b[8];
            a8_codes8(v, inv, b);
            // natural K order: bytes 0..3 and 4..7
            const uint32_t d0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
            const uint32_t d1 = __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[6], 0x04000C0Cu);
            *reinterpret_cast<uint2 *>(o + c * 8) = make_uint2(d0, d1);
        }
        if (threadIdx.x == 0) sx[m] = s;
    }
}

// batch: blockIdx.y = problem
template <int G, bool IMAGE>
__global__ __launch_bounds__(256) void quant_act_kernel(const A8QuantBatch qb)
{
    const int pi = (int)blockIdx.y;
    quant_act_row<G, IMAGE>(qb.x[pi], qb.out[pi], qb.sx[pi], qb.K[pi], qb.kt[pi], qb.M, (int)blockIdx.x);
}

// one problem: its fields as scalar kernel arguments, preloaded into scalar
// registers (no kernel-argument round trip before the first load)
template <int G, bool IMAGE>
__global__ __launch_bounds__(256) void quant_act_single(const _Float16 *x, uint8_t *out, float *sx, int K, int kt,
                                                        int M)
{
    quant_act_row<G, IMAGE>(x, out, sx, K, kt, M, (int)blockIdx.x);
}

// Launch plan shared by the workspace query and the launcher.
struct A8Plan {
    int mode;                        // 0 fused, 1 workspace, -1 unsupported
    int W, T, MR;
    int64_t kt;
    size_t lds, ws;
    int64_t ws_off[kMaxGemvBatch];
};

A8Plan a8_plan(const W4Layout *L, int count, int M)
{
    A8Plan p;
    p.mode = -1;
    p.ws = 0;
    p.lds = 0;
    p.MR = M == 1 ? 1 : (M <= 8 ? 2 : 4);          // accumulators per lane (see a_token)
    int64_t kt = 0;
    for (int i = 0; i < count; ++i) kt = L[i].ktiles > kt ? L[i].ktiles : kt;
    p.kt = kt;
    int W = (int)((kt + 3) / 4);
    if (W < 1) W = 1;
    if (W > 16) W = 16;
    p.W = W;
    p.T = (int)((kt + W - 1) / W);
    if (M < 1 || M > 16 || p.T > 8 || count < 1) return p;
    int fused = 0, split = 0;
    int64_t off = 0;
    for (int i = 0; i < count; ++i) {
        const int f = a8_lds(M, (int)L[i].K, (int)L[i].ktiles, L[i].G, W, p.MR, true).total;
        const int s = a8_lds(M, (int)L[i].K, (int)L[i].ktiles, L[i].G, W, p.MR, false).total;
        fused = f > fused ? f : fused;
        split = s > split ? s : split;
        p.ws_off[i] = off;
        off += align256(a8_block(M, (int)L[i].ktiles, L[i].G).bytes);
    }
    // The fused form pays the quantization once per workgroup (a launch has
    // hundreds to thousands): worth it at M = 1, where a separate launch costs
    // more; from M = 2 one quantization kernel plus a block copy is faster.
    if (M == 1 && fused <= kA8FusedMaxLds) {
        p.mode = 0;
        p.lds = (size_t)fused;
    } else if (split <= kA8MaxLds) {
        p.mode = 1;
        p.lds = (size_t)split;
        p.ws = (size_t)off;
    }
    return p;
}

// raises a kernel's dynamic LDS limit when a launch needs more than 64 KiB
// (`raised` belongs to the caller's instantiation)
inline hipError_t a8_lds_limit(const void *k, size_t lds, bool &raised)
{
    if (lds <= 64 * 1024 || raised) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kA8MaxLds);
    if (e == hipSuccess) raised = true;
    return e;
}

template <int G, bool ASYM, int MR, int T, bool FUSED>
hipError_t a8_launch_k(const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    if (b.count == 1) {
        static bool raised = false;
        auto k = gemv_w4a8_single<G, ASYM, MR, T, FUSED>;
        const hipError_t e = a8_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        const GemvProblem &p = b.p[0];
        k<<<grid, block, lds, st>>>(p.codes, p.scales, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W, p.zeros);
    } else if (b.count <= 4) {
        static bool raised = false;
        auto k = gemv_w4a8_batch<G, ASYM, MR, T, FUSED, 4>;
        const hipError_t e = a8_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        k<<<grid, block, lds, st>>>(b);
    } else {
        static bool raised = false;
        auto k = gemv_w4a8_batch<G, ASYM, MR, T, FUSED, 8>;
        const hipError_t e = a8_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        k<<<grid, block, lds, st>>>(b);
    }
    return hipGetLastError();
}

template <int G, bool ASYM, int MR, bool FUSED>
hipError_t a8_launch_t(int T, const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    if (T <= 2) return a8_launch_k<G, ASYM, MR, 2, FUSED>(b, grid, block, lds, st);
    if (T <= 4) return a8_launch_k<G, ASYM, MR, 4, FUSED>(b, grid, block, lds, st);
    return a8_launch_k<G, ASYM, MR, 8, FUSED>(b, grid, block, lds, st);
}

template <int G, bool ASYM, bool FUSED>
hipError_t a8_launch_m(int MR, int T, const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    if (MR == 1) return a8_launch_t<G, ASYM, 1, FUSED>(T, b, grid, block, lds, st);
    if (MR == 2) return a8_launch_t<G, ASYM, 2, FUSED>(T, b, grid, block, lds, st);
    return a8_launch_t<G, ASYM, 4, FUSED>(T, b, grid, block, lds, st);
}

template <int G, bool ASYM>
hipError_t a8_launch(bool fused, int MR, int T, const GemvBatch &b, dim3 grid, dim3 block, size_t lds, hipStream_t st)
{
    return fused ? a8_launch_m<G, ASYM, true>(MR, T, b, grid, block, lds, st)
                 : a8_launch_m<G, ASYM, false>(MR, T, b, grid, block, lds, st);
}

template <int G>
hipError_t quant_launch(bool image, const A8QuantBatch &qb, int count, hipStream_t st)
{
    const dim3 grid((unsigned)qb.M, (unsigned)count);
    if (count == 1) {
        if (image)
            quant_act_single<G, true><<<grid, 256, 0, st>>>(qb.x[0], qb.out[0], qb.sx[0], qb.K[0], qb.kt[0], qb.M);
        else
            quant_act_single<G, false><<<grid, 256, 0, st>>>(qb.x[0], qb.out[0], qb.sx[0], qb.K[0], qb.kt[0], qb.M);
    } else if (image) {
        quant_act_kernel<G, true><<<grid, 256, 0, st>>>(qb);
    } else {
        quant_act_kernel<G, false><<<grid, 256, 0, st>>>(qb);
    }
    return hipGetLastError();
}

}  // namespace

int gemv_w4a8_plan(const W4Layout *L, int count, int M, size_t *ws_bytes)
{
    const A8Plan p = a8_plan(L, count, M);
    if (ws_bytes) *ws_bytes = p.ws;
    return p.mode;
}

hipError_t launch_gemv_w4a8_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                  const _Float16 *const *x, _Float16 *const *y, void *ws, hipStream_t s)
{
    if (M == 0 || count == 0) return hipSuccess;
    const A8Plan plan = a8_plan(L, count, M);
    if (plan.mode < 0) return hipErrorInvalidValue;    // rejected by the caller's validation first
    const bool fused = plan.mode == 0;
    const int G = L[0].G;
    const bool asym = L[0].asym;
    if (!fused) {
        A8QuantBatch qb;
        for (int i = 0; i < count; ++i) {
            qb.x[i] = x[i];
            qb.out[i] = static_cast<uint8_t *>(ws) + plan.ws_off[i];
            qb.sx[i] = nullptr;
            qb.K[i] = (int)L[i].K;
            qb.kt[i] = (int)L[i].ktiles;
        }
        qb.M = M;
        hipError_t e;
        switch (G) {
        case 32: e = quant_launch<32>(true, qb, count, s); break;
        case 64: e = quant_launch<64>(true, qb, count, s); break;
        default: e = quant_launch<128>(true, qb, count, s); break;
        }
        if (e != hipSuccess) return e;
    }
    GemvBatch b;
    int64_t strips = 0;
    for (int i = 0; i < kMaxGemvBatch; ++i) b.first[i] = 0x7FFFFFFF;
    for (int i = 0; i < count; ++i) {
        GemvProblem &p = b.p[i];
        p.codes = packed[i] + L[i].codes_off;
        p.scales = packed[i] + L[i].scales_off;
        p.zeros = L[i].asym ? packed[i] + L[i].zeros_off : nullptr;
        p.x = fused ? x[i] : reinterpret_cast<const _Float16 *>(static_cast<uint8_t *>(ws) + plan.ws_off[i]);
        p.y = y[i];
        p.N = (int)L[i].N;
        p.K = (int)L[i].K;
        p.ktiles = (int)L[i].ktiles;
        p.strips = (int)L[i].strips;
        p.tw = (int)((L[i].ktiles + plan.W - 1) / plan.W);
        p.pad = 0;
        b.first[i] = (int)strips;
        strips += L[i].strips;
    }
    b.count = count;
    b.M = M;
    b.ct = 0;
    b.W = plan.W;
    if (strips == 0) return hipSuccess;
    const dim3 grid((unsigned)strips), block((unsigned)(plan.W * 64));
    switch (G) {
    case 32: return asym ? a8_launch<32, true>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s)
                         : a8_launch<32, false>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s);
    case 64: return asym ? a8_launch<64, true>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s)
                         : a8_launch<64, false>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s);
    default: return asym ? a8_launch<128, true>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s)
                         : a8_launch<128, false>(fused, plan.MR, plan.T, b, grid, block, plan.lds, s);
    }
}

hipError_t launch_quant_act_i8(int M, int K, const _Float16 *x, int8_t *xq, float *sx, hipStream_t s)
{
    if (M == 0) return hipSuccess;
    A8QuantBatch qb;
    qb.x[0] = x;
    qb.out[0] = reinterpret_cast<uint8_t *>(xq);
    qb.sx[0] = sx;
    qb.K[0] = K;
    qb.kt[0] = (K + 127) / 128;
    qb.M = M;
    return quant_launch<32>(false, qb, 1, s);
}

}  // namespace lowbit
