// gemv_chain.hip -- a chain of dependent W4 GEMV stages (a whole decode step)
// run by one persistent launch.
//
// At batch 1 every projection of a decoder layer is a small, bandwidth-bound
// GEMV, and a step is a long sequence of them; paying a kernel launch, a
// ramp-up and a drain for each one costs as much as the weight traffic of the
// smaller ones ("BaseRT" wiki chapter, limitations and approach: per-command
// submission overhead dominates batch-1 decode, so many small operations are
// encoded into one submission).  Here the whole sequence is one launch.
//
// Semantics: problems are grouped into stages 0..S-1 (consecutive, in order).
// Every problem of stage s+1 reads its x only after every problem of stage s
// has stored its y, so y of one stage may be x of the next.  Each y has
// exactly the value lowbit_gemv gives for the same problem (same per-tile
// arithmetic, same fixed-order reduction).
//
// MI355X design:
//   * Grid = one workgroup per compute unit, all resident at once (a
//     cooperative launch: the runtime guarantees it or refuses).  Each
//     workgroup has 9 waves: waves 0..7 ("compute waves") stream weights and
//     run the MFMAs; wave 8 (the "control wave") never loads weights.  It
//     waits for the previous stage, stages activations into LDS with
//     LDS-direct loads, sums the compute waves' partials, stores y and signals
//     completion.  Keeping weight loads out of the control wave matters:
//     vector loads and stores retire in order, so a wave with weight loads in
//     flight could not see its own stores complete until those loads landed.
//   * Work items are (problem, 16-row strip) pairs numbered across the chain
//     in stage order; workgroup w takes items w, w + grid, w + 2 grid, ...
//     An item is processed in rounds of 32 K tiles (4 per compute wave).
//   * Weight loads run several rounds ahead of the MFMAs, across item and
//     stage boundaries (a ring of register slots, unrolled so that no slot is
//     ever copied while its loads are in flight): while the control wave
//     waits for stage s, the weights of the next rounds are already streaming.
//   * Stage completion: a workgroup signals once per stage in which it had
//     items (after its last one), by a relaxed atomic add on one of 32
//     counters of that stage (one per 128-byte line, picked by workgroup
//     index); a waiter sums the 32 counters.  y is written with
//     device-coherent stores and the control wave waits for their completion
//     before it signals; x is read with device-coherent loads after the wait
//     has seen the count.  That orders the data without an L2 write-back or
//     invalidate, which on this chip cost more than the wait itself.
//   * Counters accumulate across runs: a run reads the epoch (runs completed
//     on this buffer) and waits for (epoch + 1) * arrivals; the last
//     workgroup to finish bumps the epoch.  Nothing is cleared between runs,
//     so a run can be replayed from a graph.
//   * Every wait is bounded: past `spin_limit` polls the wait gives up, sets
//     bit 0 of the error word and goes on (results of that run are then
//     undefined, the launch still ends).  A timed-out run still signals every
//     stage it took part in, so the counters stay consistent for later runs.
#include "lowbit_internal.hpp"
#include "gemv_tile.hpp"

namespace lowbit {

namespace {

using namespace tile;

constexpr int kComputeWaves = 8;
constexpr int kChainThreads = (kComputeWaves + 1) * 64;
constexpr int kTilesPerWave = 4;
constexpr int kRoundTiles = kComputeWaves * kTilesPerWave;   // 32 K tiles = 4096 K per round
static_assert(kRoundTiles == kChainRoundTiles, "round size shared with the planner");
constexpr uint32_t kCoherent = 16;                            // cache policy: device-coherent (sc1)

// counter words: [0] error bits, [1] epoch, [32] finished workgroups, then per
// stage kChainSlots counters kChainSlotStride words apart
constexpr int kCtrDone = 32;
constexpr int kCtrHeader = kChainCtrHeader;

__device__ __forceinline__ uint32_t ld_coherent(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The plan is read-only for the whole launch: reading it through the
// constant address space makes every uniform access a scalar load, which
// waits on its own counter instead of behind the weight stream.
typedef const __attribute__((address_space(4))) ChainProb CProb;
typedef const __attribute__((address_space(4))) int CInt;

struct Cursor {
    int pi, item, rr;   // problem, global item index, round inside the item
};

__device__ __forceinline__ void seek(Cursor &c, CProb *P, int nprob)
{
    while (c.pi < nprob && c.item >= P[c.pi].item_end) ++c.pi;
}

__device__ __forceinline__ void advance(Cursor &c, CProb *P, int nprob, int nwg)
{
    if (c.pi >= nprob) return;
    if (++c.rr < P[c.pi].rounds) return;
    c.rr = 0;
    c.item += nwg;
    seek(c, P, nprob);
}

template <int G, bool ASYM> struct Slot {
    u4 q[kTilesPerWave];
    MetaRaw<G, ASYM> m[kTilesPerWave];
};

// Weight and metadata loads of one round of one compute wave (branch-free:
// a finished cursor or a tile past the strip's end reads zeros).
template <int G, bool ASYM>
__device__ __forceinline__ void load_round(Slot<G, ASYM> &s, const Cursor &p, CProb *P, int nprob, int wave,
                                           int lane)
{
    constexpr int GPT = 128 / G;
    const bool live = p.pi < nprob;
    CProb &pr = P[live ? p.pi : 0];
    const int kt = live ? pr.ktiles : 0;
    const int64_t tiles0 = live ? (int64_t)(p.item - pr.item_begin) * pr.ktiles : 0;
    const auto crs = buffer_rsrc(pr.codes + tiles0 * 1024, (uint32_t)kt * 1024);
    const auto srs = buffer_rsrc(pr.scales + tiles0 * 16 * GPT * 2, (uint32_t)kt * 16 * GPT * 2);
    const auto zrs = buffer_rsrc(ASYM ? pr.zeros + tiles0 * 16 * GPT : pr.scales, ASYM ? (uint32_t)kt * 16 * GPT : 0u);
    const int r = lane & 15;
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
        const int t = p.rr * kRoundTiles + wave + u * kComputeWaves;
        const bool ok = t < kt;
        s.q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (uint32_t)t * 1024 + lane * 16 : kBufferOob, 0, kStreamLoad);
        s.m[u] = load_meta<G, ASYM>(srs, zrs, ok ? t * 16 + r : -1);
    }
}

// Constants of the offset-split product (gemv_tile.hpp), kept in registers.
struct SplitConst {
    uint32_t mlo, mhi;
    h8 psym;
};

// Branch-free: a tile past the strip's end has zero codes and zero scales
// (its loads read out of range), so its product adds exactly zero; its
// activation address is clamped to the last real tile so it only reads
// finite values.  The product is the offset-split one of the streaming GEMV
// (gemv_tile.hpp): one MFMA chain over the codes and, for batch-1 symmetric
// weights, the offset terms of up to four tiles from one shared chain whose
// A rows carry the K blocks of different (tile, group) pairs; otherwise a
// second chain per tile over the zero-point operand.
template <int G, bool ASYM, int MR>
__device__ __forceinline__ void compute_round(const Slot<G, ASYM> &s, const Cursor &c, CProb *P,
                                              const _Float16 *xs, const _Float16 *xa, int wave, int lane,
                                              const SplitConst &k, f4 &acc)
{
    constexpr int GPT = 128 / G;
    constexpr int MPG = G / 32;
    constexpr bool PRE = !ASYM && MR == 1;
    constexpr int TPS = 4 / GPT;                     // tiles per shared offset chain
    const int kt = P[c.pi].ktiles;
    const int r = lane & 15, kq = lane >> 4;
    f4 cps = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
        const int t = c.rr * kRoundTiles + wave + u * kComputeWaves;
        const int tx = t < kt ? t : kt - 1;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PRE) {
            if (u % TPS == 0) {
                // A row j < 4: tile u + j / GPT, group j % GPT (C row j = its offset term)
                const int rr = r < 4 ? r : 0;
                const int tu = c.rr * kRoundTiles + wave + (u + rr / GPT) * kComputeWaves;
                const int txu = tu < kt ? tu : kt - 1;
                const _Float16 *xb = xs + txu * 128 + (rr % GPT) * G + kq * 8;
#pragma unroll
                for (int b = 0; b < MPG; ++b) {
                    const h8 ab = *reinterpret_cast<const h8 *>(xb + b * 32);
                    cps = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, k.psym, b == 0 ? f4{0.f, 0.f, 0.f, 0.f} : cps, 0,
                                                                 0, 0);
                }
            }
        }
        u4 qv = s.q[u];
        asm volatile("" : "+v"(qv));
        MetaRaw<G, ASYM> mv = s.m[u];
        pin_meta<G, ASYM>(mv);
        h8 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const h8 *>(xa + tx * 128 + i * 32);
        if constexpr (PRE) {
            float off[GPT];
#pragma unroll
            for (int g = 0; g < GPT; ++g) off[g] = cps[(u % TPS) * GPT + g];
            tile_product_pre<G>(qv, mv, av, off, k.mlo, k.mhi, acc);
        } else {
            tile_product_split<G, ASYM, MR>(qv, mv, av, k.psym, k.mlo, k.mhi, acc);
        }
    }
}

// Control wave: poll the counters of `stage` until they reach the target.
__device__ __forceinline__ void wait_stage(const ChainArgs &a, CInt *arrivals, uint32_t epoch, int stage, int lane)
{
    const uint32_t target = (epoch + 1u) * (uint32_t)arrivals[stage];
    const uint32_t *ctr = a.ctr + kCtrHeader + (int64_t)stage * kChainSlots * kChainSlotStride;
    uint32_t n = 0;
    for (;;) {
        uint32_t v = lane < kChainSlots ? ld_coherent(ctr + lane * kChainSlotStride) : 0u;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if ((int32_t)(v - target) >= 0) break;
        if (++n > a.spin_limit) {
            if (lane == 0) __hip_atomic_fetch_or(a.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Control wave: x[0..M)[0..K) -> LDS rows of `xrow` halfs with LDS-direct
// 16-byte loads (1 KiB per instruction, no registers involved); K past the
// end reads zeros.
__device__ __forceinline__ void stage_x(CProb &pr, int M, int xrow, _Float16 *xs, int lane)
{
    const auto xrs = buffer_rsrc(pr.x, (uint32_t)((int64_t)M * pr.K * 2));
    const int row_chunks = (pr.ktiles * 128 + 511) / 512;        // 512 halfs per instruction
    for (int m = 0; m < M; ++m) {
        for (int c = 0; c < row_chunks; ++c) {
            const int k = c * 512 + lane * 8;
            const uint32_t off = k < pr.K ? (uint32_t)(((int64_t)m * pr.K + k) * 2) : kBufferOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void *)(xs + m * xrow + c * 512),
                                                 16, off, 0, 0, kCoherent);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// Compute waves: stream weights two rounds ahead and run the MFMAs.  This
// loop holds no other vector memory traffic, so the compiler's wait before
// each tile counts only the weight loads issued after it.
// Register slots of weight loads in flight: D - 1 rounds ahead of the MFMAs.
template <int G, bool ASYM> struct ChainDepth { static constexpr int D = (ASYM && G == 32) ? 4 : 5; };

// Compute waves: stream weights D - 1 rounds ahead and run the MFMAs.  This
// loop holds no other vector memory traffic and no data-dependent branch
// around a load or a use, so the compiler's wait before each tile counts
// exactly the weight loads issued after it.
template <int G, bool ASYM, int MR>
__device__ __forceinline__ void compute_loop(const ChainArgs &a, CProb *P, const _Float16 *xs, float *red, int wave,
                                             int lane)
{
    constexpr int D = ChainDepth<G, ASYM>::D;
    const int nprob = a.nprob, nwg = gridDim.x;
    const int r = lane & 15, kq = lane >> 4;
    const _Float16 *xa = xs + (r < a.M ? r : a.M - 1) * a.xrow + kq * 8;
    SplitConst kc;
    kc.mlo = kMagicLo;
    kc.mhi = kMagicHi;
    asm volatile("" : "+v"(kc.mlo), "+v"(kc.mhi));   // in registers: each mask-or is one operation
    {
        u4 pw = __builtin_bit_cast(u4, offset8(8));
        asm volatile("" : "+v"(pw));
        kc.psym = __builtin_bit_cast(h8, pw);
    }

    Slot<G, ASYM> s[D];
    Cursor c = {0, (int)blockIdx.x, 0};
    seek(c, P, nprob);
    Cursor p = c;
#pragma unroll
    for (int k = 0; k < D - 1; ++k) {
        load_round<G, ASYM>(s[k], p, P, nprob, wave, lane);
        advance(p, P, nprob, nwg);
    }

    int x_pi = -1, rb = 0;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    // One round.  Past the last item the step still runs (its loads read
    // nothing, its products are discarded); only the barrier bookkeeping is
    // guarded, and that branch holds no vector memory operation, so every
    // step has the same load/wait structure.
    auto step = [&](Slot<G, ASYM> &cur, Slot<G, ASYM> &pf) {
        const bool alive = c.pi < nprob;
        const Cursor cc = {alive ? c.pi : nprob - 1, c.item, c.rr};
        load_round<G, ASYM>(pf, p, P, nprob, wave, lane);
        if (alive && c.rr == 0 && c.pi != x_pi) {
            x_pi = c.pi;
            __syncthreads();                                   // (A) control wave: dependency met, x staged
        }
        compute_round<G, ASYM, MR>(cur, cc, P, xs, xa, wave, lane, kc, acc);
        if (alive && c.rr == P[cc.pi].rounds - 1) {
            float *rbuf = red + rb * (kComputeWaves * MR * 64);
#pragma unroll
            for (int j = 0; j < MR; ++j) rbuf[(wave * MR + j) * 64 + lane] = acc[j];
            acc = f4{0.f, 0.f, 0.f, 0.f};
            __syncthreads();                                   // (B) partials of this item in LDS
            rb ^= 1;
        }
        advance(c, P, nprob, nwg);
        advance(p, P, nprob, nwg);
    };
    while (c.pi < nprob) {
#pragma unroll
        for (int k = 0; k < D; ++k) step(s[k], s[(k + D - 1) % D]);
    }
}

// Control wave: stage dependencies, activations, reduction, y, signals.  It
// walks the same items and meets the compute waves at the same barriers.
template <int MR>
__device__ __forceinline__ void control_loop(const ChainArgs &a, CProb *P, CInt *arrivals, _Float16 *xs, float *red,
                                             int lane)
{
    const int nprob = a.nprob, nwg = gridDim.x, M = a.M;
    const int r = lane & 15, kq = lane >> 4;
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(ld_coherent(a.ctr + 1));

    Cursor c = {0, (int)blockIdx.x, 0};
    seek(c, P, nprob);
    int x_pi = -1, ready = 0, rb = 0, x_K = -1;
    const _Float16 *x_loaded = nullptr;
    while (c.pi < nprob) {
        CProb &pr = P[c.pi];
        if (c.rr == 0 && c.pi != x_pi) {
            if (pr.stage > ready) {
                wait_stage(a, arrivals, epoch, pr.stage - 1, lane);
                ready = pr.stage;
            }
            if (pr.x != x_loaded || pr.K != x_K) {
                stage_x(pr, M, a.xrow, xs, lane);
                x_loaded = pr.x;
                x_K = pr.K;
            }
            x_pi = c.pi;
            __syncthreads();                                   // (A)
        }
        if (c.rr == pr.rounds - 1) {
            __syncthreads();                                   // (B)
            const float *rbuf = red + rb * (kComputeWaves * MR * 64);
            float sum[MR];
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                float v = rbuf[j * 64 + lane];
                for (int w = 1; w < kComputeWaves; ++w) v += rbuf[(w * MR + j) * 64 + lane];
                sum[j] = v;
            }
            const int n = (c.item - pr.item_begin) * 16 + r;
            const auto yrs = buffer_rsrc(pr.y, (uint32_t)((int64_t)M * pr.N * 2));
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const int m = kq * 4 + j;
                const uint32_t off = (m < M && n < pr.N) ? (uint32_t)(((int64_t)m * pr.N + n) * 2) : kBufferOob;
                const _Float16 hv = (_Float16)sum[j];
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hv), yrs, off, 0, kCoherent);
            }
            // signal the stage after this workgroup's last item in it
            Cursor nx = {c.pi, c.item + nwg, 0};
            seek(nx, P, nprob);
            if (nx.pi >= nprob || P[nx.pi].stage != pr.stage) {
                __builtin_amdgcn_s_waitcnt(0);                 // y stores complete
                if (lane == 0)
                    __hip_atomic_fetch_add(a.ctr + kCtrHeader +
                                               ((int64_t)pr.stage * kChainSlots + (int)blockIdx.x % kChainSlots) *
                                                   kChainSlotStride,
                                           1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            rb ^= 1;
        }
        advance(c, P, nprob, nwg);
    }
    if (lane == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.ctr + kCtrDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1u == (epoch + 1u) * (uint32_t)nwg)
            __hip_atomic_store(a.ctr + 1, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int G, bool ASYM, int MR>
__global__ __launch_bounds__(kChainThreads, 1)
void gemv_chain_kernel(const ChainArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (int64_t)a.M * a.xrow * 2);   // [2][8 waves][MR][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    CProb *P = (CProb *)a.probs;
    if (wave == kComputeWaves)
        control_loop<MR>(a, P, (CInt *)a.arrivals, xs, red, lane);
    else
        compute_loop<G, ASYM, MR>(a, P, xs, red, wave, lane);
}

template <int G, bool ASYM, int MR>
hipError_t launch_chain_t(const ChainArgs &a, int grid, size_t lds, hipStream_t s)
{
    auto k = gemv_chain_kernel<G, ASYM, MR>;
    hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // a cooperative launch: the runtime starts every workgroup at once or
    // refuses the launch (hipErrorCooperativeLaunchTooLarge), so the waits
    // never depend on a workgroup that is not running; it can be captured
    // in a graph
    ChainArgs args = a;
    void *kargs[] = {&args};
    return hipLaunchCooperativeKernel((const void *)k, dim3(grid), dim3(kChainThreads), kargs, (unsigned)lds, s);
}

template <int G, bool ASYM, int MR>
int occupancy_t(size_t lds)
{
    int n = 0;
    auto k = gemv_chain_kernel<G, ASYM, MR>;
    if (hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kChainThreads, lds) != hipSuccess) return 0;
    return n;
}

template <int G, bool ASYM>
hipError_t launch_chain_g(const ChainArgs &a, int grid, size_t lds, hipStream_t s)
{
    if (a.M == 1) return launch_chain_t<G, ASYM, 1>(a, grid, lds, s);
    if (a.M == 2) return launch_chain_t<G, ASYM, 2>(a, grid, lds, s);
    return launch_chain_t<G, ASYM, 4>(a, grid, lds, s);
}

template <int G, bool ASYM>
int occupancy_g(int M, size_t lds)
{
    if (M == 1) return occupancy_t<G, ASYM, 1>(lds);
    if (M == 2) return occupancy_t<G, ASYM, 2>(lds);
    return occupancy_t<G, ASYM, 4>(lds);
}

}  // namespace

size_t gemv_chain_lds_bytes(int M, int xrow)
{
    const int MR = M == 1 ? 1 : (M == 2 ? 2 : 4);
    return (size_t)M * xrow * 2 + (size_t)2 * kComputeWaves * MR * 64 * 4;
}

int gemv_chain_occupancy(int G, bool asym, int M, size_t lds)
{
    switch (G) {
    case 32: return asym ? occupancy_g<32, true>(M, lds) : occupancy_g<32, false>(M, lds);
    case 64: return asym ? occupancy_g<64, true>(M, lds) : occupancy_g<64, false>(M, lds);
    default: return asym ? occupancy_g<128, true>(M, lds) : occupancy_g<128, false>(M, lds);
    }
}

hipError_t launch_gemv_chain(int G, bool asym, const ChainArgs &a, int grid, hipStream_t s)
{
    const size_t lds = gemv_chain_lds_bytes(a.M, a.xrow);
    switch (G) {
    case 32: return asym ? launch_chain_g<32, true>(a, grid, lds, s) : launch_chain_g<32, false>(a, grid, lds, s);
    case 64: return asym ? launch_chain_g<64, true>(a, grid, lds, s) : launch_chain_g<64, false>(a, grid, lds, s);
    default: return asym ? launch_chain_g<128, true>(a, grid, lds, s) : launch_chain_g<128, false>(a, grid, lds, s);
    }
}

}  // namespace lowbit
