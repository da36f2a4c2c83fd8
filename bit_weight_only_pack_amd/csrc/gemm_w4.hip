// gemm_w4.hip -- prefill GEMM with packed INT4 weights on the matrix cores.
//
//   C[m][n] = sum_k A[m][k] * (q[n][k] - z) * s[n][k/G]      (fp32 accumulate)
//
// ("Low Bit ARM kernels": prefill is a GEMM over the same group-wise
// quantized weights; "Low Bit Metal Kernels", int4_matmul: an activation tile
// and a dequantized weight tile are staged in on-chip memory and multiplied.)
//
// MI355X design:
//   * Workgroup tile 128 x 256, K in steps of 128 (one packed weight tile),
//     8 waves of 64 x 64.  The A tile (128 x 128, bf16 or fp16), the
//     workgroup's 16 packed 16 x 128 weight tiles (already in the lane order
//     of v_mfma_f32_16x16x32_{bf16,f16}) and their scales move to LDS by
//     LDS-direct loads in a 3-stage ring; each wave reads its operands from
//     there.  With one quantization group per K tile the two wave groups run
//     a phase apart (one wave of each SIMD unpacks while the other issues
//     MFMAs); see the kernel for the schedule.
//   * Weights stay exact, in offset form.  The B operand holds each code
//     plus a constant, made by masking it into the mantissa of a power of
//     two: bf16 activations 128 + q (mask-or with bf16 128.0); fp16
//     activations 1024 + q and 64 + q (fp16 1024.0 and 64.0, one unit 1/16
//     there, as in the GEMV).  The zero point enters as an operand p of the
//     same shape (128 + z, or 1024 + z / 64 + z), and per group
//       sum_k a (q - z) = sum_k a v  -  sum_k a p
//     is one MFMA chain over v started from the chain of a against -p (one
//     chain per row block for symmetric weights, where p is a constant; one
//     per column block for asymmetric ones).
//   * Scales in fp32: each group's chain starts fresh and is added to the
//     accumulator with one FMA by the column's scale (a zero scale adds 0).
//   * Split-K over workgroups when the output tiles alone cannot fill the
//     256 CUs: fp32 partial tiles go to a workspace and a second kernel adds
//     them in a fixed order (deterministic) and rounds to the output type.
#include "lowbit_internal.hpp"

namespace lowbit {

namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

// 8 codes -> exact fp16 offset values: 1024 + q at K offsets 0, 1, 4, 5 (mask
// into 1024.0) and 64 + q at 2, 3, 6, 7 (mask into 64.0, where one unit is 1/16)
__device__ __forceinline__ u4 unpack_f16_split(uint32_t w, uint32_t mlo, uint32_t mhi)
{
    const uint32_t w8 = w >> 8;
    return u4{(w & 0x000F000Fu) | mlo, (w & 0x00F000F0u) | mhi, (w8 & 0x000F000Fu) | mlo, (w8 & 0x00F000F0u) | mhi};
}

// the negated offset operand of zero point z, same slots as the unpack
__device__ __forceinline__ u4 neg_offset(bool bf16, int z)
{
    if (bf16) {
        const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)(-128.0f - (float)z));   // exact: |128 + z| < 256
        const uint32_t d = h | (h << 16);
        return u4{d, d, d, d};
    }
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(-1024.0f - (float)z));
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(-64.0f - (float)z));
    return u4{lo | (lo << 16), hi | (hi << 16), lo | (lo << 16), hi | (hi << 16)};
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

// Kernel parameters shared by the instantiations.
struct GemmArgs {
    const uint8_t *codes, *scales, *zeros;   // packed sections
    const uint16_t *a;                        // [M][K] bf16 or fp16 bits
    void *c;                                  // [M][N] output (bf16 / fp16), or fp32 partials when split
    float *part;                              // split-K partials [S][M][N]
    int M, N, K, ktiles, splits, c_bf16;
    int m_tiles, n_tiles;
};

// ---------------------------------------------------------------- pipelined GEMM
// Workgroup tile 128 x 256 (8 waves as 2 x 4, each 64 x 64 = 4 x 4 MFMA
// blocks), K in steps of one packed 128-K tile.  Every operand moves from
// memory to LDS with LDS-direct loads (no registers), kV2Stages - 1 K steps
// ahead of the MFMAs, in a ring of kV2Stages LDS stages:
//   A : 128 rows x 128 K, rows of 256 bytes whose 16-byte chunks are XOR-
//       swizzled by the row (chunk c of row r stored at c ^ (r % 16)), so the
//       16 rows of an MFMA operand read 16 different bank groups;
//   B : the 16 packed 1 KiB tiles of the workgroup's columns, as stored;
//   scale / zero-point blocks of those tiles.
// Each wave issues the same fixed set of load instructions per stage, so
// "stage k has landed" is a vmcnt count; a barrier then publishes it.
constexpr int kV2Waves = 8;
constexpr int kV2BM = 128, kV2BN = 256;
constexpr int kV2Stages = 3;
constexpr int kV2AStage = kV2BM * 256;                 // bytes
constexpr int kV2BStage = (kV2BN / 16) * 1024;         // 16 strips
constexpr int kV2MStage = kV2Waves * 256;              // per-wave 256-byte metadata slots
template <bool ASYM> constexpr int v2_stage_bytes() { return kV2AStage + kV2BStage + kV2MStage * (ASYM ? 2 : 1); }
template <bool ASYM> constexpr int v2_dma_per_stage() { return 4 + 2 + 1 + (ASYM ? 1 : 0); }

template <int BYTES>
__device__ __forceinline__ void v2_dma(__amdgpu_buffer_rsrc_t rs, uint8_t *lds, uint32_t off)
{
    static_assert(BYTES == 16 || BYTES == 4, "LDS-direct load size");
    auto *l = (__attribute__((address_space(3))) void *)lds;
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 4, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void v2_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void v2_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <bool A_BF16, int G, bool ASYM>
__global__ __launch_bounds__(kV2Waves * 64, 1)
void gemm_w4_v2_kernel(GemmArgs p)
{
    constexpr int GPT = 128 / G;
    constexpr int SPG = G / 32;                       // 32-K MFMA steps per group
    constexpr int TM = 4, TN = 4;
    constexpr int SB = v2_stage_bytes<ASYM>();
    constexpr int NDMA = v2_dma_per_stage<ASYM>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int r16 = lane & 15, kq = lane >> 4;

    // tile coordinates (XCD-aware: consecutive workgroups on one XCD share A rows)
    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int split = lin % p.splits;
    const int tile = lin / p.splits;
    const int mt = tile / p.n_tiles, nt = tile % p.n_tiles;
    const int m0 = mt * kV2BM, n0 = nt * kV2BN;
    const int kt0 = (int)((int64_t)p.ktiles * split / p.splits);
    const int kt1 = (int)((int64_t)p.ktiles * (split + 1) / p.splits);

    const int strips_total = (p.N + 15) / 16;
    const auto ars = buffer_rsrc(p.a, (uint32_t)((int64_t)p.M * p.K * 2));
    const auto crs = buffer_rsrc(p.codes, (uint32_t)((int64_t)strips_total * p.ktiles * 1024));
    const auto srs = buffer_rsrc(p.scales, (uint32_t)((int64_t)strips_total * p.ktiles * 16 * GPT * 2));
    const auto zrs = buffer_rsrc(ASYM ? p.zeros : p.scales,
                                 ASYM ? (uint32_t)((int64_t)strips_total * p.ktiles * 16 * GPT) : 0u);

    // load `part` of K tile kt into stage st (a tile past kt1 loads zeros):
    // parts 0-3 the A rows, 4-5 the B strips, 6 the scales, 7 the zero points
    auto issue_part = [&](int kt, int st, int part) __attribute__((always_inline)) {
        uint8_t *sa = smem + st * SB;
        uint8_t *sb = sa + kV2AStage;
        uint8_t *sm = sb + kV2BStage;
        const bool live = kt < kt1;
        if (part < 4) {
            // A: instruction i of wave w fills LDS rows 4(4w + i) .. +3, lane -> (row, stored chunk)
            const int i = part;
            const int row = (wave * 4 + i) * 4 + (lane >> 4);
            const int pos = lane & 15;
            const int chunk = pos ^ (row & 15);
            const int k = kt * 128 + chunk * 8;
            const bool ok = live && m0 + row < p.M && k < p.K;
            v2_dma<16>(ars, sa + (wave * 4 + i) * 1024,
                       ok ? (uint32_t)(((int64_t)(m0 + row) * p.K + k) * 2) : kBufferOob);
        } else if (part < 6) {
            // B: wave w loads strips 2w, 2w + 1 of the tile's 16
            const int j = part - 4;
            const int s = n0 / 16 + wave * 2 + j;
            const bool ok = live && s < strips_total;
            v2_dma<16>(crs, sb + (wave * 2 + j) * 1024,
                       ok ? (uint32_t)(((int64_t)s * p.ktiles + kt) * 1024 + lane * 16) : kBufferOob);
        } else if (part == 6) {
            // scales of those two strips: 2 x 32*GPT bytes, 4 bytes per lane
            const int b = lane * 4, j = b / (32 * GPT), off = b - j * 32 * GPT;
            const int s = n0 / 16 + wave * 2 + j;
            const bool ok = live && j < 2 && s < strips_total;
            v2_dma<4>(srs, sm + wave * 256,
                      ok ? (uint32_t)(((int64_t)s * p.ktiles + kt) * 32 * GPT + off) : kBufferOob);
        } else if constexpr (ASYM) {
            const int b = lane * 4, j = b / (16 * GPT), off = b - j * 16 * GPT;
            const int s = n0 / 16 + wave * 2 + j;
            const bool ok = live && j < 2 && s < strips_total;
            v2_dma<4>(zrs, sm + kV2MStage + wave * 256,
                      ok ? (uint32_t)(((int64_t)s * p.ktiles + kt) * 16 * GPT + off) : kBufferOob);
        }
    };
    auto issue = [&](int kt, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int part = 0; part < NDMA; ++part) issue_part(kt, st, part);
    };

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    uint32_t mlo = A_BF16 ? 0x43004300u : 0x64006400u;   // 128.0 (bf16) / 1024.0 (fp16)
    uint32_t mhi = 0x54005400u;                          // 64.0 (fp16)
    asm volatile("" : "+v"(mlo), "+v"(mhi));             // in registers: each mask-or is one operation
    u4 psym = neg_offset(A_BF16, 8);
    asm volatile("" : "+v"(psym));

    auto mfma = [&](const u4 &a, const u4 &b, const f4 &c) __attribute__((always_inline)) {
        if constexpr (A_BF16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c,
                                                          0, 0, 0);
    };

    if constexpr (G == 128) {
        // Two phases per K tile.  Memory phase: start the loads of the tile two
        // steps ahead, read this tile's B codes, scales and A operands from LDS
        // and unpack B.  Compute phase: the tile's MFMAs, then the blocks' scale
        // FMAs (written beside the next block's run; the compiler gathers them at
        // the end of the phase).  The wave group wm = 1 runs one phase behind
        // wm = 0, and waves w and w + 4 share a SIMD, so on every SIMD one wave
        // reads and unpacks while the other keeps the matrix core busy; a
        // barrier closes every phase, and the compute phase runs at raised wave
        // priority.
        // Stage (kt + 2) % 3 is refilled in tile kt's memory phase: group 0 read
        // it two phases earlier, group 1 one phase earlier (its LDS reads
        // complete before that barrier).  Tile kt + 1 must have landed before
        // the barrier that opens group 0's next memory phase: group 0 waits for
        // its loads at the end of its compute phase, group 1 at the end of its
        // memory phase, each with one tile's loads still in flight.
        static_assert(kV2Stages == 3, "the phase schedule refills stage (kt + 2) % 3");
        const int grp = wm;
        issue(kt0, 0);
        issue(kt0 + 1, 1);
        v2_wait_vm<NDMA>();
        v2_barrier();
        if (grp == 1) v2_barrier();

        for (int kt = kt0; kt < kt1; ++kt) {
            const int st = (kt - kt0) % kV2Stages;
            issue(kt + 2, (st + 2) % kV2Stages);
            const uint8_t *sa = smem + st * SB;
            const uint8_t *sb = sa + kV2AStage;
            const uint8_t *sm = sb + kV2BStage;
            u4 bq[TN];
#pragma unroll
            for (int nb = 0; nb < TN; ++nb) bq[nb] = *reinterpret_cast<const u4 *>(sb + (wn * 4 + nb) * 1024 + lane * 16);
            float sc[TN];
            u4 pn[TN];                                 // asymmetric: negated offset operands
#pragma unroll
            for (int nb = 0; nb < TN; ++nb) {
                const int s = wn * 4 + nb;             // strip in the tile; its loader wave = s / 2
                const uint8_t *ms = sm + (s >> 1) * 256 + (s & 1) * 32;
                sc[nb] = (float)*reinterpret_cast<const _Float16 *>(ms + r16 * 2);
                if constexpr (ASYM) {
                    const uint8_t *mz = sm + kV2MStage + (s >> 1) * 256 + (s & 1) * 16;
                    pn[nb] = neg_offset(A_BF16, (int)*reinterpret_cast<const int8_t *>(mz + r16));
                }
            }
            u4 av[TM][4];
#pragma unroll
            for (int mb = 0; mb < TM; ++mb) {
                const int row = wm * 64 + mb * 16 + r16;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int chunk = (j * 4 + kq) ^ (row & 15);
                    av[mb][j] = *reinterpret_cast<const u4 *>(sa + row * 256 + chunk * 16);
                }
            }
            // B operands of the tile's four 32-K steps in offset form
            u4 bv[4][TN];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < TN; ++nb)
                    bv[j][nb] = A_BF16 ? unpack_bf16_biased(bq[nb][j], mlo) : unpack_f16_split(bq[nb][j], mlo, mhi);
            if (grp == 1) v2_wait_vm<NDMA>();
            __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0): this phase's LDS reads are done
            __builtin_amdgcn_sched_barrier(0);
            v2_barrier();
            __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);

            // The matrix core runs at full rate from one wave only on back-to-back
            // accumulation into the same registers: each 16x16 block's chain over
            // the tile is one uninterrupted run (sched_barrier keeps the runs
            // apart).  Symmetric weights: the four row blocks' offset chains go
            // first, so every block chain starts from a value finished long before.
            f4 offs[TM];
#pragma unroll
            for (int mb = 0; mb < TM; ++mb) {
                offs[mb] = f4{0.f, 0.f, 0.f, 0.f};
                if constexpr (!ASYM) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) offs[mb] = mfma(av[mb][j], psym, offs[mb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            f4 prev = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = 0; blk < TM * TN; ++blk) {
                const int mb = blk / TN, nb = blk % TN;
                f4 c = offs[mb];
                if constexpr (ASYM) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) c = mfma(av[mb][j], pn[nb], j == 0 ? f4{0.f, 0.f, 0.f, 0.f} : c);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) c = mfma(av[mb][j], bv[j][nb], c);
                __builtin_amdgcn_sched_barrier(0);
                if (blk > 0) {
                    const int pm = (blk - 1) / TN, pnb = (blk - 1) % TN;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[pm][pnb][i] = __builtin_fmaf(sc[pnb], prev[i], acc[pm][pnb][i]);
                }
                prev = c;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[TM - 1][TN - 1][i] = __builtin_fmaf(sc[TN - 1], prev[i], acc[TM - 1][TN - 1][i]);
            if (grp == 0) v2_wait_vm<NDMA>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            v2_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        if (grp == 0) v2_barrier();
    } else {
        // groups of 32 or 64 K: operands for a whole K tile do not fit beside
        // the per-group metadata in 256 registers; one barrier per K tile
        // prologue: stages 0 .. kV2Stages-2
#pragma unroll
        for (int s = 0; s < kV2Stages - 1; ++s) issue(kt0 + s, s);

        for (int kt = kt0; kt < kt1; ++kt) {
            const int st = (kt - kt0) % kV2Stages;
            v2_wait_vm<NDMA * (kV2Stages - 2)>();          // this wave's loads of stage st landed
            v2_barrier();                                  // every wave's; stage (st + 2) % 3 free
            issue(kt + kV2Stages - 1, (st + kV2Stages - 1) % kV2Stages);

            const uint8_t *sa = smem + st * SB;
            const uint8_t *sb = sa + kV2AStage;
            const uint8_t *sm = sb + kV2BStage;
            // this wave's B strips (wn * 4 + nb) and their metadata
            u4 bq[TN];
#pragma unroll
            for (int nb = 0; nb < TN; ++nb) bq[nb] = *reinterpret_cast<const u4 *>(sb + (wn * 4 + nb) * 1024 + lane * 16);

#pragma unroll
            for (int g = 0; g < GPT; ++g) {
                float sc[TN];
                u4 pneg[TN];
#pragma unroll
                for (int nb = 0; nb < TN; ++nb) {
                    const int s = wn * 4 + nb;             // strip in the tile; its loader wave = s / 2
                    const uint8_t *ms = sm + (s >> 1) * 256 + (s & 1) * 32 * GPT;
                    sc[nb] = (float)*reinterpret_cast<const _Float16 *>(ms + (r16 * GPT + g) * 2);
                    if constexpr (ASYM) {
                        const uint8_t *mz = sm + kV2MStage + (s >> 1) * 256 + (s & 1) * 16 * GPT;
                        pneg[nb] = neg_offset(A_BF16, (int)*reinterpret_cast<const int8_t *>(mz + r16 * GPT + g));
                    }
                }
                // the group's B operands in offset form
                u4 bv[SPG][TN];
#pragma unroll
                for (int ss = 0; ss < SPG; ++ss)
#pragma unroll
                    for (int nb = 0; nb < TN; ++nb) {
                        const uint32_t w = bq[nb][g * SPG + ss];
                        bv[ss][nb] = A_BF16 ? unpack_bf16_biased(w, mlo) : unpack_f16_split(w, mlo, mhi);
                    }
#pragma unroll
                for (int mb = 0; mb < TM; ++mb) {
                    const int row = wm * 64 + mb * 16 + r16;
                    u4 av[SPG];
#pragma unroll
                    for (int ss = 0; ss < SPG; ++ss) {
                        const int chunk = ((g * SPG + ss) * 4 + kq) ^ (row & 15);
                        av[ss] = *reinterpret_cast<const u4 *>(sa + row * 256 + chunk * 16);
                    }
                    // - sum_k a p over the group: shared by the row block (symmetric)
                    f4 off = f4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (!ASYM) {
#pragma unroll
                        for (int ss = 0; ss < SPG; ++ss) off = mfma(av[ss], psym, off);
                    }
#pragma unroll
                    for (int nb = 0; nb < TN; ++nb) {
                        f4 c = off;
                        if constexpr (ASYM) {
#pragma unroll
                            for (int ss = 0; ss < SPG; ++ss) c = mfma(av[ss], pneg[nb], ss == 0 ? f4{0.f, 0.f, 0.f, 0.f} : c);
                        }
#pragma unroll
                        for (int ss = 0; ss < SPG; ++ss) c = mfma(av[ss], bv[ss][nb], c);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[mb][nb][i] = __builtin_fmaf(sc[nb], c[i], acc[mb][nb][i]);
                    }
                }
            }
        }
    }

    // the loads issued for stages past the end write LDS too: let them land
    // before this workgroup's LDS can be handed to another one
    v2_wait_vm<0>();

    // epilogue; C layout of the 16x16 MFMA: lane holds column (lane % 16) and
    // rows 4*(lane / 16) + i of each block
#pragma unroll
    for (int mb = 0; mb < TM; ++mb)
#pragma unroll
        for (int nb = 0; nb < TN; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 64 + mb * 16 + kq * 4 + i;
                const int n = n0 + wn * 64 + nb * 16 + r16;
                if (m < p.M && n < p.N) {
                    const float v = acc[mb][nb][i];
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

// 128 x 256 output tiles (8 waves of 64 x 64), one workgroup per compute
// unit at a time.  Split K over workgroups by the estimated makespan: rounds
// of 256 workgroups x K tiles per workgroup, plus, when split, the reduce
// pass's bytes (S fp32 partials read, the output written) in units of one
// workgroup's K tile (about 12 MB of HBM traffic in the time one K tile
// takes); each split keeps >= 8 K tiles.  (224 tiles of 32 K tiles: two
// splits give 448 workgroups, two rounds of 16, the same makespan as one
// round of 32, so the reduce pass would be pure cost.)
GemmPlan plan_gemm(int M, int N, int K)
{
    const int ktiles = (K + 127) / 128;
    GemmPlan pl;
    pl.m_tiles = (M + kV2BM - 1) / kV2BM;
    pl.n_tiles = (N + kV2BN - 1) / kV2BN;
    const int64_t tiles = (int64_t)pl.m_tiles * pl.n_tiles;
    pl.splits = 1;
    double best = -1.0;
    for (int s = 1;; s *= 2) {
        const int64_t rounds = (tiles * s + 255) / 256;
        const double reduce = s == 1 ? 0.0 : ((double)s * M * N * 4 + (double)M * N * 2) / 12e6;
        const double cost = (double)rounds * ((ktiles + s - 1) / s) + reduce;
        if (best < 0.0 || cost < best - 1e-9) {
            best = cost;
            pl.splits = s;
        }
        if (ktiles / (s * 2) < 8) break;
    }
    return pl;
}

template <bool A_BF16, int G, bool ASYM>
hipError_t launch_cfg(const GemmPlan &pl, const GemmArgs &a, hipStream_t s)
{
    const unsigned blocks = (unsigned)((int64_t)pl.m_tiles * pl.n_tiles * pl.splits);
    constexpr int lds = kV2Stages * v2_stage_bytes<ASYM>();
    auto k = gemm_w4_v2_kernel<A_BF16, G, ASYM>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    k<<<blocks, kV2Waves * 64, lds, s>>>(a);
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
