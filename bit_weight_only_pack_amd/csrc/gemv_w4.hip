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
#include "gemv_tile.hpp"

namespace lowbit {

namespace {

using namespace tile;

constexpr size_t kMaxLds = 64 * 1024;

// Dynamic LDS of one workgroup: a chunk of `ct` K tiles of every activation
// row, each row padded by 16 bytes (so the 16 A rows of an MFMA operand fall
// in different banks), followed by the cross-wave reduction buffer.
__host__ __device__ inline int x_row_halfs(int ct) { return ct * 128 + 8; }
__host__ __device__ inline int64_t gemv_lds_bytes(int M, int ct, int W, int MR)
{
    return (int64_t)M * x_row_halfs(ct) * 2 + (int64_t)kRedSlots * MR * 64 * 4;
}

// One workgroup = one 16-row strip (all of K) of one problem of the batch
// (problems are laid end to end over blockIdx.x).  The strip's K tiles are
// taken in rounds of W*P: in a round, wave w owns tiles round + w + u*W
// (u < P) and issues all of their weight loads before any arithmetic
// (branch-free buffer loads; slots past the last tile read zeros and are
// skipped).  The activations of the round are staged in LDS `ct` tiles at a
// time (all at once whenever they fit, which covers every decode shape).
template <int G, bool ASYM, int MR, int P>
// min waves per SIMD (VGPR budget 512 / waves): 8 (64) for 4 tiles in flight,
// 6 (85) for 8; asymmetric G=32 carries three metadata words per tile
__global__ __launch_bounds__(1024, (P <= 4 ? (ASYM && G == 32 ? 7 : 8) : (ASYM ? 5 : 6)))
void gemv_w4_kernel(const GemvBatch b)
{
    constexpr int GPT = 128 / G;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // the problem of this workgroup is blockIdx.y; strips past its end exit
    const GemvProblem &pr = b.p[blockIdx.y];
    if ((int)blockIdx.x >= pr.strips) return;
    const uint8_t *codes = pr.codes, *scales = pr.scales, *zeros = pr.zeros;
    const _Float16 *x = pr.x;
    _Float16 *y = pr.y;
    const int M = b.M, N = pr.N, K = pr.K, ktiles = pr.ktiles, ct = b.ct;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int strip = (int)blockIdx.x;
    const int r = lane & 15;                         // B column (weight row) and A row (token)
    const int kq = lane >> 4;                        // 8-K slice inside each 32-K MFMA block
    const int xrow = x_row_halfs(ct);
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (int64_t)M * xrow * 2);

    // descriptors over this strip's codes / scales / zero points and over x
    const int64_t tiles0 = (int64_t)strip * ktiles;
    const auto crs = buffer_rsrc(codes + tiles0 * 1024, (uint32_t)ktiles * 1024);
    const auto srs = buffer_rsrc(scales + tiles0 * 16 * GPT * 2, (uint32_t)ktiles * 16 * GPT * 2);
    const auto zrs = buffer_rsrc(ASYM ? zeros + tiles0 * 16 * GPT : scales, ASYM ? (uint32_t)ktiles * 16 * GPT : 0u);
    const auto xrs = buffer_rsrc(x, (uint32_t)((int64_t)M * K * 2));
    const _Float16 *xa = xs + a_token<MR>(r, M) * xrow + kq * 8;

    uint32_t magic = 0x64006400u;                    // fp16 1024.0 in both halves
    asm volatile("" : "+v"(magic));                  // keep it in a register: mask+or becomes one op

    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < ktiles; b0 += W * P) {
        // 1. weight and group-metadata loads of this wave's tiles in the round
        u4 q[P];
        MetaRaw<G, ASYM> mr[P];
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int t = b0 + wave + u * W;
            const bool ok = t < ktiles;
            q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (uint32_t)t * 1024 + lane * 16 : kBufferOob, 0, kStreamLoad);
            mr[u] = load_meta<G, ASYM>(srs, zrs, ok ? t * 16 + r : -1);
        }
        const int rend = min(b0 + W * P, ktiles);
        for (int c0 = b0; c0 < rend; c0 += ct) {
            const int cend = min(c0 + ct, rend);
            // 2. stage x[0..M)[128*c0, 128*cend) into LDS, 8 halfs per thread and
            //    step; K % 32 == 0, so a chunk is inside the row or wholly padding
            if (c0 > 0) __syncthreads();                 // previous chunk fully read
            const int cpr = (cend - c0) * 16;            // 8-half chunks per row
            for (int j = threadIdx.x; j < M * cpr; j += blockDim.x) {
                const int m = j / cpr;
                const int kl = (j - m * cpr) * 8;
                const int k = c0 * 128 + kl;
                const uint32_t off = k < K ? (uint32_t)(((int64_t)m * K + k) * 2) : kBufferOob;
                const u4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
                *reinterpret_cast<u4 *>(xs + m * xrow + kl) = v;
            }
            __syncthreads();
            // 3. products of the tiles of this chunk
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int t = b0 + wave + u * W;
                if (t >= c0 && t < cend) {
                    // keep each tile's operands live only for that tile: the
                    // empty asm stops the compiler from unpacking every tile
                    // ahead of the activation staging
                    __builtin_amdgcn_sched_barrier(0);
                    u4 qv = q[u];
                    asm volatile("" : "+v"(qv));
                    MetaRaw<G, ASYM> mv = mr[u];
                    pin_meta<G, ASYM>(mv);
                    h8 a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a[i] = *reinterpret_cast<const h8 *>(xa + (t - c0) * 128 + i * 32);
                    tile_product<G, ASYM, MR>(qv, mv, a, magic, acc);
                }
            }
        }
    }

    // 4. fixed-order cross-wave sum, fp16 RNE store
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
        // C layout of the 16x16 MFMA: lane holds column (lane % 16), rows 4*(lane / 16) + j
        const int n = strip * 16 + r;
#pragma unroll
        for (int j = 0; j < MR; ++j) {
            const int m = c_token<MR>(kq, j);
            if (m < M && n < N) y[(int64_t)m * N + n] = (_Float16)acc[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel (every decode shape): the workgroup's whole activation
// block sits in LDS, so nothing waits behind the weight stream.
//   1. x goes to LDS first, by LDS-direct loads (1 KiB per wave instruction).
//      Rows are padded to whole 1 KiB chunks, so every chunk lies in one row,
//      and the 16-byte blocks of row m are XOR-swizzled by m & 15 so the up
//      to 16 A rows of an MFMA operand fall in different banks.
//   2. Each wave then issues the weight and metadata loads of its K tiles (a
//      contiguous run of the strip), tile by tile.
//   3. A wait for the x part only (issued first; vector loads retire in
//      order) and one barrier.  With eight tiles per wave (16-wave
//      workgroups, one per compute unit) the wait and barrier come after the
//      first tile's loads and before the other seven: x reads issued ahead of
//      a whole compute unit's weight stream still land behind much of it
//      (measured 3.4-4.8 us into the down projection's launch, against
//      0.7-1.1 us this way), and every tile product waits for x.  A
//      single-problem launch with four tiles per wave (the o projection)
//      waits after two tiles; the batched four-tile launches after all four
//      (an earlier wait measured slower there).
//   4. Tiles in issue order, each waiting only for its own loads; the
//      offset-split product (two MFMA chains per group, see gemv_tile.hpp).
//   5. Fixed-order cross-wave sum through LDS, fp16 RNE store.
// ---------------------------------------------------------------------------
constexpr int kV2MaxLds = 80 * 1024;               // two workgroups still fit a compute unit's 160 KiB
constexpr int64_t kNs2MinStrips = 1024;             // launches of at least this many strips take two per workgroup
constexpr int kNs2MinM = 5;                         // ... with at least this many tokens

struct V2Lds {
    int rowp;                                        // 16-byte blocks per LDS row of x
    int red, total;
};
// 16-byte blocks per K tile in LDS: 16, or 20 for the batch-1 symmetric form,
// whose shared offset chain reads the same block of four consecutive tiles at
// once (the 64-byte pad puts those reads in different banks)
__host__ __device__ constexpr int v2_tile_blocks(bool asym, int MR) { return !asym && MR == 1 ? 20 : 16; }
__host__ __device__ inline V2Lds v2_lds(int M, int kt, int W, int MR, bool asym, int NS = 1)
{
    V2Lds l;
    l.rowp = (int)round_up((int64_t)kt * v2_tile_blocks(asym, MR), 64);
    l.red = M * l.rowp * 16;
    l.total = l.red + (W > 1 ? NS * kRedSlots * MR * 64 * 4 : 0);
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
// a workgroup barrier without the vmcnt(0) that __syncthreads implies
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Occupancy targets: batch-1 symmetric with up to 4 tiles per wave keeps 8
// waves per SIMD (64 VGPRs), so four 8-wave workgroups share a compute unit;
// other forms with up to 4 tiles per wave 6; 8 tiles per wave (16-wave
// workgroups, one per compute unit), or two strips of 4 tiles, 4.
// The streaming kernel's work for NS consecutive strips strip0 .. strip0 +
// NS - 1 (those below nst), once their problem's fields are known (in scalar
// registers).  NS = 2 (several tokens, launches of many strips): the two
// strips share one staged activation block, whose LDS-direct copy is the
// larger part of a workgroup's vector-memory traffic at M = 8, and each tile's
// A fragments are read from LDS once for both.
template <int G, bool ASYM, int MR, int T, bool SINGLE = false, int NS = 1>
__device__ __forceinline__ void gemv_v2_strip(const uint8_t *codes, const uint8_t *scales, const uint8_t *zeros,
                                              const _Float16 *xg, _Float16 *yp, int N, int K, int kt, int tw, int M,
                                              int W, int strip0, int nst = 0x7FFFFFFF)
{
    static_assert(NS == 1 || (NS == 2 && !(!ASYM && MR == 1)), "two strips: the general product only");
    constexpr int GPT = 128 / G;
    constexpr int NW = T * (ASYM ? 3 : 2);          // weight + metadata loads per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, kq = lane >> 4;
    const int t0 = wave * tw;
    constexpr int TB = v2_tile_blocks(ASYM, MR);
    const V2Lds L = v2_lds(M, kt, W, MR, ASYM, NS);
    float *red = reinterpret_cast<float *>(smem + L.red);     // [NS][kRedSlots][MR][64]

    // 1. activations -> LDS: chunk cc of row m holds blocks 64 cc .. 64 cc + 63
    //    of the row; block b < 16 of tile t of row m holds
    //    x[m][128 t + 8 (b ^ (m & 15)) ..], blocks 16..TB-1 are zero padding
    {
        const auto xrs = buffer_rsrc(xg, (uint32_t)(M * K * 2));
        const int cpr = L.rowp >> 6;
        for (int m = 0; m < M; ++m) {
            for (int cc = wave; cc < cpr; cc += W) {
                const int jj = cc * 64 + lane;
                const int t = jj / TB, bb = jj - t * TB;
                const int j = t * 16 + (bb ^ (m & 15));
                const bool ok = bb < 16 && j * 8 < K;
                lds_dma16(xrs, smem + (m * cpr + cc) * 1024, ok ? (uint32_t)((m * K + j * 8) * 2) : kBufferOob);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. weights and metadata of this wave's tiles, in tile order; 3. x in
    //    LDS everywhere, waited for after the first EARLY tiles' loads
    u4 q[NS][T];
    MetaRaw<G, ASYM> mr[NS][T];
    constexpr int EARLY = T >= 8 ? 1 : (SINGLE && NS == 1 && T == 4 ? 2 : T);
    constexpr int LPT = ASYM ? 3 : 2;                // loads per tile (codes, scales[, zeros])
    static_assert(NW == T * LPT, "load count");
    __amdgpu_buffer_rsrc_t crs[NS], srs[NS], zrs[NS];
#pragma unroll
    for (int sj = 0; sj < NS; ++sj) {
        // (a strip past the problem's end reads zeros and stores nothing; with
        // one strip the caller has already checked it)
        const bool live = NS == 1 || strip0 + sj < nst;
        const int64_t tiles0 = (int64_t)(live ? strip0 + sj : 0) * kt;
        crs[sj] = buffer_rsrc(codes + tiles0 * 1024, live ? (uint32_t)kt * 1024 : 0u);
        srs[sj] = buffer_rsrc(scales + tiles0 * 16 * GPT * 2, live ? (uint32_t)kt * 16 * GPT * 2 : 0u);
        zrs[sj] = buffer_rsrc(ASYM ? zeros + tiles0 * 16 * GPT : scales, ASYM && live ? (uint32_t)kt * 16 * GPT : 0u);
    }
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u == EARLY) {
            wait_vm<EARLY * LPT * NS>();             // x has landed; tiles < EARLY may be in flight
            wg_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        const int t = t0 + u;
        const bool ok = u < tw && t < kt;
#pragma unroll
        for (int sj = 0; sj < NS; ++sj) {
            q[sj][u] = __builtin_amdgcn_raw_buffer_load_b128(crs[sj], ok ? (uint32_t)t * 1024 + lane * 16 : kBufferOob,
                                                             0, kStreamLoad);
            mr[sj][u] = load_meta<G, ASYM>(srs[sj], zrs[sj], ok ? t * 16 + r : -1);
        }
        __builtin_amdgcn_sched_barrier(0);           // keep the loads in tile order
    }
    if constexpr (EARLY == T) {
        wait_vm<NW * NS>();
        wg_barrier();
    }

    // 4. products, tile by tile in load order
    uint32_t mlo = kMagicLo, mhi = kMagicHi, m1152 = kMagic1152;
    asm volatile("" : "+v"(mlo), "+v"(mhi), "+v"(m1152));   // in registers: each mask-or is one operation
    uint32_t zsel[4];
    zp32_selectors(zsel);
    if constexpr (ASYM && G == 32) asm volatile("" : "+v"(zsel[0]), "+v"(zsel[1]), "+v"(zsel[2]), "+v"(zsel[3]));
    h8 psym = offset8(8);
    {
        u4 pw = __builtin_bit_cast(u4, psym);
        asm volatile("" : "+v"(pw));                 // materialised once, outside the tile loop
        psym = __builtin_bit_cast(h8, pw);
    }
    const int xr = a_token<MR>(r, M);
    const _Float16 *xa[4];                           // A fragment i of this wave's first tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xa[i] = reinterpret_cast<const _Float16 *>(smem) + (xr * L.rowp + t0 * TB + ((i * 4 + kq) ^ (xr & 15))) * 8;
    f4 acc[NS];
#pragma unroll
    for (int sj = 0; sj < NS; ++sj) acc[sj] = f4{0.f, 0.f, 0.f, 0.f};
    // Batch-1 symmetric weights: the offset chain x . p does not depend on
    // the codes or the weight row, so one MFMA chain serves several tiles.
    // Its A rows 0..3 carry K blocks of different (tile, group) pairs
    // instead of copies of the one token: row j = (tile u0 + j / GPT, group
    // j % GPT), and C row j (lane / 16 == 0, element j) is that group's offset
    // term, computed exactly as the per-tile chain would compute it.
    constexpr bool PRE = !ASYM && MR == 1;
    constexpr int TPS = 4 / GPT;                     // tiles per offset set
    constexpr int MPG = G / 32;
    f4 cps = {0.f, 0.f, 0.f, 0.f};
    const int tvalid = min(tw, kt - t0);             // this wave's real tiles (>= 1 when it has work)
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
                    for (int i = 0; i < MPG; ++i) {
                        const h8 ab = *reinterpret_cast<const h8 *>(xb + i * 32);
                        cps = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, psym, i == 0 ? f4{0.f, 0.f, 0.f, 0.f} : cps,
                                                                     0, 0, 0);
                    }
                }
            }
            h8 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const h8 *>(xa[i] + u * TB * 8);
#pragma unroll
            for (int sj = 0; sj < NS; ++sj) {
                u4 qv = q[sj][u];
                asm volatile("" : "+v"(qv));
                MetaRaw<G, ASYM> mv = mr[sj][u];
                pin_meta<G, ASYM>(mv);
                if constexpr (PRE) {
                    float off[GPT];
#pragma unroll
                    for (int g = 0; g < GPT; ++g) off[g] = cps[(u % TPS) * GPT + g];
                    tile_product_pre<G>(qv, mv, a, off, mlo, mhi, acc[sj]);
                } else if constexpr (ASYM && G == 32) {
                    tile_product_zp32<MR>(qv, mv, a, m1152, mhi, zsel, acc[sj]);
                } else {
                    tile_product_split<G, ASYM, MR>(qv, mv, a, psym, mlo, mhi, acc[sj]);
                }
            }
        }
    }

    // 5. fixed-order cross-wave sum (a balanced tree over the sixteen
    //    partial slots), fp16 RNE store; wave sj sums and stores strip sj
    //    (wave 0 both when the workgroup has one wave)
    if (W > 1) {
#pragma unroll
        for (int sj = 0; sj < NS; ++sj)
#pragma unroll
            for (int j = 0; j < MR; ++j)
                red_put(red + (sj * kRedSlots * MR + j) * 64 + lane, MR * 64, wave, W, acc[sj][j]);
        __syncthreads();
#pragma unroll
        for (int sj = 0; sj < NS; ++sj) {
            if (wave == sj) {
#pragma unroll
                for (int j = 0; j < MR; ++j) acc[sj][j] = red_sum(red + (sj * kRedSlots * MR + j) * 64 + lane, MR * 64);
            }
        }
    }
#pragma unroll
    for (int sj = 0; sj < NS; ++sj) {
        if (wave == (W > 1 ? sj : 0) && (NS == 1 || strip0 + sj < nst)) {
            const int n = (strip0 + sj) * 16 + r;
#pragma unroll
            for (int j = 0; j < MR; ++j) {
                const int m = c_token<MR>(kq, j);
                if (m < M && n < N) yp[(int64_t)m * N + n] = (_Float16)acc[sj][j];
            }
        }
    }
}

template <int G, bool ASYM, int MR, int T, int NP, int NS = 1>
__global__ __launch_bounds__(1024)
__attribute__((amdgpu_waves_per_eu(T > 4 || NS > 1 ? 4 : (!ASYM && MR == 1) ? 8 : 6)))
void gemv_w4_v2_kernel(const GemvBatch b)
{
    // One round of kernel-argument reads.  NP = 4:
    // the problems' strips are laid end to end over blockIdx.x and the fields
    // of all four are read at once, then selected.  NP = 8: blockIdx.y is the
    // problem and strips past its end exit.  Every field is made live right
    // away (empty asm), so the scalar loads go out together.
    if constexpr (NP == 4) {
        // all four problems' pointers and sizes live before the selection
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const GemvProblem &q = b.p[i];
            asm volatile("" ::"s"(q.codes), "s"(q.scales), "s"(q.zeros), "s"(q.x), "s"(q.y), "s"(q.N), "s"(q.K),
                         "s"(q.ktiles), "s"(q.strips), "s"(q.tw));
        }
        asm volatile("" ::"s"(b.first[1]), "s"(b.first[2]), "s"(b.first[3]), "s"(b.M), "s"(b.W));
    }
    int pi, strip;
    if constexpr (NP == 4) {
        const int bx = (int)blockIdx.x, f1 = b.first[1], f2 = b.first[2], f3 = b.first[3];
        pi = (bx >= f1 ? 1 : 0) + (bx >= f2 ? 1 : 0) + (bx >= f3 ? 1 : 0);
        strip = bx - (pi == 0 ? 0 : pi == 1 ? f1 : pi == 2 ? f2 : f3);
    } else {
        pi = (int)blockIdx.y;
        strip = (int)blockIdx.x;
    }
    auto field = [&](auto get) {
        if constexpr (NP == 4) {
            const auto v0 = get(b.p[0]), v1 = get(b.p[1]), v2 = get(b.p[2]), v3 = get(b.p[3]);
            return pi == 0 ? v0 : pi == 1 ? v1 : pi == 2 ? v2 : v3;
        } else {
            return get(b.p[pi]);
        }
    };
    const uint8_t *codes = field([](const GemvProblem &q) { return q.codes; });
    const uint8_t *scales = field([](const GemvProblem &q) { return q.scales; });
    const uint8_t *zeros = field([](const GemvProblem &q) { return q.zeros; });
    const _Float16 *xg = field([](const GemvProblem &q) { return q.x; });
    _Float16 *yp = field([](const GemvProblem &q) { return q.y; });
    int N = field([](const GemvProblem &q) { return q.N; });
    int K = field([](const GemvProblem &q) { return q.K; });
    int kt = field([](const GemvProblem &q) { return q.ktiles; });
    int nst = field([](const GemvProblem &q) { return q.strips; });
    int tw = field([](const GemvProblem &q) { return q.tw; });
    int M = b.M, W = b.W;
    asm volatile("" : "+s"(codes), "+s"(scales), "+s"(xg), "+s"(yp), "+s"(N), "+s"(K), "+s"(kt), "+s"(nst),
                 "+s"(tw), "+s"(M), "+s"(W));
    if constexpr (ASYM) asm volatile("" : "+s"(zeros));
    // (strip counts workgroups: NS row strips each)
    if (strip * NS >= nst) return;
    gemv_v2_strip<G, ASYM, MR, T, false, NS>(codes, scales, zeros, xg, yp, N, K, kt, tw, M, W, strip * NS, nst);
}

// One problem: every field is a kernel argument of its own (16 dwords), so
// the hardware preloads them into scalar registers before the first
// instruction and the first load needs no kernel-argument read.
// NS = 2: two strips per workgroup (the problem's strip count follows from N).
template <int G, bool ASYM, int MR, int T, int NS = 1>
__global__ __launch_bounds__(1024)
__attribute__((amdgpu_waves_per_eu(T > 4 || NS > 1 ? 4 : (!ASYM && MR == 1) ? 8 : 6)))
void gemv_w4_v2_single(const uint8_t *codes, const uint8_t *scales, const _Float16 *xg, _Float16 *yp, int N, int K,
                       int kt, int tw, int M, int W, const uint8_t *zeros)
{
    gemv_v2_strip<G, ASYM, MR, T, true, NS>(codes, scales, zeros, xg, yp, N, K, kt, tw, M, W, (int)blockIdx.x * NS,
                                           (N + 15) / 16);
}

// ---------------------------------------------------------------------------
// Streaming kernel with a per-wave activation ring (M >= 2 when the whole
// activation block does not fit in LDS, e.g. M = 8 with K = 14336: 229 KB).
// A wave only ever reads the activations of its own tiles, so instead of the
// workgroup's whole block each wave keeps a ring of NC tile slots (M rows x
// 128 K each) in its own part of LDS, filled by LDS-direct loads: the slots of
// its first NC tiles go out first, then all its weight loads, and after each
// tile's product the slot just read is refilled with the tile NC ahead.  No
// barrier is needed until the cross-wave sum; the wave waits only on its own
// load counter (explicit vmcnt counts: the compiler does not track what
// LDS-direct loads write).
// ---------------------------------------------------------------------------
constexpr int kXrSlots = 4;                         // activation slots per wave
constexpr int kXrMaxLds = 160 * 1024;

// rows staged per tile: 4, 8 or 16 (one LDS-direct load moves 4 rows of
// 128 K), at least M; the kernels are instantiated for these three
__host__ __device__ inline int xr_rows(int M) { return M <= 4 ? 4 : (M <= 8 ? 8 : 16); }
__host__ __device__ inline int xr_lds(int M, int W, int MR)
{
    return W * kXrSlots * xr_rows(M) * 256 + kRedSlots * MR * 64 * 4;
}

// s_waitcnt vmcnt(n) for an n the optimizer folds to a constant (unrolled loops)
__device__ __forceinline__ void vm_wait_n(int n)
{
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(3952); break;
    case 1: __builtin_amdgcn_s_waitcnt(3953); break;
    case 2: __builtin_amdgcn_s_waitcnt(3954); break;
    case 3: __builtin_amdgcn_s_waitcnt(3955); break;
    case 4: __builtin_amdgcn_s_waitcnt(3956); break;
    case 5: __builtin_amdgcn_s_waitcnt(3957); break;
    case 6: __builtin_amdgcn_s_waitcnt(3958); break;
    case 7: __builtin_amdgcn_s_waitcnt(3959); break;
    case 8: __builtin_amdgcn_s_waitcnt(3960); break;
    case 9: __builtin_amdgcn_s_waitcnt(3961); break;
    case 10: __builtin_amdgcn_s_waitcnt(3962); break;
    case 11: __builtin_amdgcn_s_waitcnt(3963); break;
    case 12: __builtin_amdgcn_s_waitcnt(3964); break;
    case 13: __builtin_amdgcn_s_waitcnt(3965); break;
    case 14: __builtin_amdgcn_s_waitcnt(3966); break;
    case 15: __builtin_amdgcn_s_waitcnt(3967); break;
    case 16: __builtin_amdgcn_s_waitcnt(20336); break;
    case 17: __builtin_amdgcn_s_waitcnt(20337); break;
    case 18: __builtin_amdgcn_s_waitcnt(20338); break;
    case 19: __builtin_amdgcn_s_waitcnt(20339); break;
    case 20: __builtin_amdgcn_s_waitcnt(20340); break;
    case 21: __builtin_amdgcn_s_waitcnt(20341); break;
    case 22: __builtin_amdgcn_s_waitcnt(20342); break;
    case 23: __builtin_amdgcn_s_waitcnt(20343); break;
    case 24: __builtin_amdgcn_s_waitcnt(20344); break;
    case 25: __builtin_amdgcn_s_waitcnt(20345); break;
    case 26: __builtin_amdgcn_s_waitcnt(20346); break;
    case 27: __builtin_amdgcn_s_waitcnt(20347); break;
    case 28: __builtin_amdgcn_s_waitcnt(20348); break;
    case 29: __builtin_amdgcn_s_waitcnt(20349); break;
    case 30: __builtin_amdgcn_s_waitcnt(20350); break;
    case 31: __builtin_amdgcn_s_waitcnt(20351); break;
    case 32: __builtin_amdgcn_s_waitcnt(36720); break;
    case 33: __builtin_amdgcn_s_waitcnt(36721); break;
    case 34: __builtin_amdgcn_s_waitcnt(36722); break;
    case 35: __builtin_amdgcn_s_waitcnt(36723); break;
    case 36: __builtin_amdgcn_s_waitcnt(36724); break;
    case 37: __builtin_amdgcn_s_waitcnt(36725); break;
    case 38: __builtin_amdgcn_s_waitcnt(36726); break;
    case 39: __builtin_amdgcn_s_waitcnt(36727); break;
    case 40: __builtin_amdgcn_s_waitcnt(36728); break;
    case 41: __builtin_amdgcn_s_waitcnt(36729); break;
    case 42: __builtin_amdgcn_s_waitcnt(36730); break;
    case 43: __builtin_amdgcn_s_waitcnt(36731); break;
    case 44: __builtin_amdgcn_s_waitcnt(36732); break;
    case 45: __builtin_amdgcn_s_waitcnt(36733); break;
    case 46: __builtin_amdgcn_s_waitcnt(36734); break;
    case 47: __builtin_amdgcn_s_waitcnt(36735); break;
    case 48: __builtin_amdgcn_s_waitcnt(53104); break;
    case 49: __builtin_amdgcn_s_waitcnt(53105); break;
    case 50: __builtin_amdgcn_s_waitcnt(53106); break;
    case 51: __builtin_amdgcn_s_waitcnt(53107); break;
    case 52: __builtin_amdgcn_s_waitcnt(53108); break;
    case 53: __builtin_amdgcn_s_waitcnt(53109); break;
    case 54: __builtin_amdgcn_s_waitcnt(53110); break;
    case 55: __builtin_amdgcn_s_waitcnt(53111); break;
    case 56: __builtin_amdgcn_s_waitcnt(53112); break;
    case 57: __builtin_amdgcn_s_waitcnt(53113); break;
    case 58: __builtin_amdgcn_s_waitcnt(53114); break;
    case 59: __builtin_amdgcn_s_waitcnt(53115); break;
    case 60: __builtin_amdgcn_s_waitcnt(53116); break;
    case 61: __builtin_amdgcn_s_waitcnt(53117); break;
    case 62: __builtin_amdgcn_s_waitcnt(53118); break;
    case 63: __builtin_amdgcn_s_waitcnt(53119); break;
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
    }
}

template <int G, bool ASYM, int MR, int T, int XI>
__device__ __forceinline__ void gemv_xr_strip(const uint8_t *codes, const uint8_t *scales, const uint8_t *zeros,
                                              const _Float16 *xg, _Float16 *yp, int N, int K, int kt, int tw, int M,
                                              int W, int strip)
{
    constexpr int GPT = 128 / G;
    constexpr int NC = kXrSlots;
    constexpr int LPT = ASYM ? 3 : 2;                // weight loads per tile (codes, scales[, zeros])
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, kq = lane >> 4;
    const int t0 = wave * tw;
    const int XS = XI * 1024;                        // bytes of one slot: 4 XI rows x 256 bytes
    uint8_t *ring = smem + wave * NC * XS;
    float *red = reinterpret_cast<float *>(smem + W * NC * XS);
    const auto xrs = buffer_rsrc(xg, (uint32_t)(M * K * 2));

    // slot of tile u: row m (0 .. 4 XI - 1) at m * 256 bytes; 16-byte block b
    // of row m holds K offsets 8 (b ^ (m & 15)) .. + 7 of the tile
    auto stage = [&](int u) __attribute__((always_inline)) {
        const int t = t0 + u;
        const bool live = u < tw && t < kt;
        uint8_t *slot = ring + (u % NC) * XS;
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int m = 4 * i + (lane >> 4), b = lane & 15;
            const int k = t * 128 + 8 * (b ^ (m & 15));
            const bool ok = live && m < M && k < K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void *)(slot + i * 1024),
                                                     16, ok ? (uint32_t)((m * K + k) * 2) : kBufferOob, 0, 0, 0);
        }
    };
#pragma unroll
    for (int u = 0; u < NC && u < T; ++u) stage(u);

    u4 q[T];
    MetaRaw<G, ASYM> mr[T];
    const int64_t tiles0 = (int64_t)strip * kt;
    const auto crs = buffer_rsrc(codes + tiles0 * 1024, (uint32_t)kt * 1024);
    const auto srs = buffer_rsrc(scales + tiles0 * 16 * GPT * 2, (uint32_t)kt * 16 * GPT * 2);
    const auto zrs = buffer_rsrc(ASYM ? zeros + tiles0 * 16 * GPT : scales, ASYM ? (uint32_t)kt * 16 * GPT : 0u);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        const int t = t0 + u;
        const bool ok = u < tw && t < kt;
        q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (uint32_t)t * 1024 + lane * 16 : kBufferOob, 0,
                                                     kStreamLoad);
        mr[u] = load_meta<G, ASYM>(srs, zrs, ok ? t * 16 + r : -1);
        __builtin_amdgcn_sched_barrier(0);           // keep the loads in tile order
    }

    uint32_t mlo = kMagicLo, mhi = kMagicHi, m1152 = kMagic1152;
    asm volatile("" : "+v"(mlo), "+v"(mhi), "+v"(m1152));
    uint32_t zsel[4];
    zp32_selectors(zsel);
    if constexpr (ASYM && G == 32) asm volatile("" : "+v"(zsel[0]), "+v"(zsel[1]), "+v"(zsel[2]), "+v"(zsel[3]));
    h8 psym = offset8(8);
    {
        u4 pw = __builtin_bit_cast(u4, psym);
        asm volatile("" : "+v"(pw));
        psym = __builtin_bit_cast(h8, pw);
    }
    const int xr = a_token<MR>(r, M);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const int tvalid = min(tw, kt - t0);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        if (u < tvalid) {
            __builtin_amdgcn_sched_barrier(0);
            // wait until slot u has landed: count the loads issued after it.
            // A first slot (u < NC) is followed by the later first slots, all
            // T tiles' weight loads and the slots refilled at steps before u;
            // a refilled slot (issued after tile u - NC) by the slots refilled
            // at the steps since.
            const int after = u < NC ? (NC - 1 - u) * XI + T * LPT + min(u, T - NC > 0 ? T - NC : 0) * XI
                                     : min(NC - 1, T - 1 - u) * XI;
            vm_wait_n(after);
            asm volatile("" ::: "memory");
            const uint8_t *slot = ring + (u % NC) * XS + xr * 256;
            h8 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const h8 *>(slot + (((i * 4 + kq) ^ (xr & 15)) * 16));
            u4 qv = q[u];
            asm volatile("" : "+v"(qv));
            MetaRaw<G, ASYM> mv = mr[u];
            pin_meta<G, ASYM>(mv);
            if constexpr (ASYM && G == 32)
                tile_product_zp32<MR>(qv, mv, a, m1152, mhi, zsel, acc);
            else
                tile_product_split<G, ASYM, MR>(qv, mv, a, psym, mlo, mhi, acc);
        }
        if (u + NC < T) {
            // the slot's reads have returned; refill it with tile u + NC
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stage(u + NC);
        }
    }

    // fixed-order cross-wave sum (a balanced tree over the sixteen partial
    // slots), fp16 RNE store
    if (W > 1) {
#pragma unroll
        for (int j = 0; j < MR; ++j) red_put(red + j * 64 + lane, MR * 64, wave, W, acc[j]);
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < MR; ++j) acc[j] = red_sum(red + j * 64 + lane, MR * 64);
        }
    } else {
        __builtin_amdgcn_s_waitcnt(0);
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

template <int G, bool ASYM, int MR, int T, int XI>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_xr_single(const uint8_t *codes, const uint8_t *scales, const _Float16 *xg, _Float16 *yp, int N, int K,
                    int kt, int tw, int M, int W, const uint8_t *zeros)
{
    gemv_xr_strip<G, ASYM, MR, T, XI>(codes, scales, zeros, xg, yp, N, K, kt, tw, M, W, (int)blockIdx.x);
}

// batched form: blockIdx.y = problem, strips past its end exit
template <int G, bool ASYM, int MR, int T, int XI>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_xr_batch(const GemvBatch b)
{
    const GemvProblem &p = b.p[blockIdx.y];
    if ((int)blockIdx.x >= p.strips) return;
    gemv_xr_strip<G, ASYM, MR, T, XI>(p.codes, p.scales, p.zeros, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W,
                                      (int)blockIdx.x);
}

// raises a kernel's dynamic LDS limit when a launch needs more than the default
// (`raised` belongs to the caller's instantiation, i.e. to one kernel)
inline hipError_t v2_lds_limit(const void *k, size_t lds, bool &raised)
{
    if (lds <= 64 * 1024 || raised) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kV2MaxLds);
    if (e == hipSuccess) raised = true;
    return e;
}

template <int G, bool ASYM, int MR, int T, int NP>
hipError_t launch_v2_np(dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    static bool raised = false;
    if constexpr (NP == 1) {
        auto k = gemv_w4_v2_single<G, ASYM, MR, T>;
        const hipError_t e = v2_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        const GemvProblem &p = b.p[0];
        k<<<grid, block, lds, st>>>(p.codes, p.scales, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W, p.zeros);
    } else {
        auto k = gemv_w4_v2_kernel<G, ASYM, MR, T, NP>;
        const hipError_t e = v2_lds_limit((const void *)k, lds, raised);
        if (e != hipSuccess) return e;
        k<<<grid, block, lds, st>>>(b);
    }
    return hipGetLastError();
}

template <int G, bool ASYM, int MR, int T>
hipError_t launch_v2_k(dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    if (b.count == 1) return launch_v2_np<G, ASYM, MR, T, 1>(grid, block, lds, st, b);
    if (b.count <= 4) return launch_v2_np<G, ASYM, MR, T, 4>(grid, block, lds, st, b);
    return launch_v2_np<G, ASYM, MR, T, 8>(grid, block, lds, st, b);
}

template <int G, bool ASYM, int MR>
hipError_t launch_v2_t(int T, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    if (T <= 2) return launch_v2_k<G, ASYM, MR, 2>(grid, block, lds, st, b);
    if (T <= 4) return launch_v2_k<G, ASYM, MR, 4>(grid, block, lds, st, b);
    return launch_v2_k<G, ASYM, MR, 8>(grid, block, lds, st, b);
}

// two strips per workgroup, several tokens: one problem (its fields as kernel
// arguments) or 2-4 laid end to end
template <int G, bool ASYM, int MR>
hipError_t launch_v2_ns2_m(int T, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    if (b.count == 1) {
        static bool raised2s = false, raised4s = false;
        auto k = T <= 2 ? gemv_w4_v2_single<G, ASYM, MR, 2, 2> : gemv_w4_v2_single<G, ASYM, MR, 4, 2>;
        const hipError_t e = v2_lds_limit((const void *)k, lds, T <= 2 ? raised2s : raised4s);
        if (e != hipSuccess) return e;
        const GemvProblem &p = b.p[0];
        k<<<grid, block, lds, st>>>(p.codes, p.scales, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W, p.zeros);
        return hipGetLastError();
    }
    static bool raised2 = false, raised4 = false;
    auto k = T <= 2 ? gemv_w4_v2_kernel<G, ASYM, MR, 2, 4, 2> : gemv_w4_v2_kernel<G, ASYM, MR, 4, 4, 2>;
    const hipError_t e = v2_lds_limit((const void *)k, lds, T <= 2 ? raised2 : raised4);
    if (e != hipSuccess) return e;
    k<<<grid, block, lds, st>>>(b);
    return hipGetLastError();
}
template <int G, bool ASYM>
hipError_t launch_v2_ns2(int MR, int T, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    return MR == 2 ? launch_v2_ns2_m<G, ASYM, 2>(T, grid, block, lds, st, b)
                   : launch_v2_ns2_m<G, ASYM, 4>(T, grid, block, lds, st, b);
}

template <int G, bool ASYM>
hipError_t launch_v2(int MR, int T, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    if (MR == 1) return launch_v2_t<G, ASYM, 1>(T, grid, block, lds, st, b);
    if (MR == 2) return launch_v2_t<G, ASYM, 2>(T, grid, block, lds, st, b);
    return launch_v2_t<G, ASYM, 4>(T, grid, block, lds, st, b);
}

// XI = staged rows / 4: up to 8 tokens (XI <= 2) take two accumulators per
// lane, up to 16 four
template <int G, bool ASYM, int T, int XI>
hipError_t launch_xr_k(dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    constexpr int MR = XI <= 2 ? 2 : 4;
    if (b.count == 1) {
        static bool raised = false;
        auto k = gemv_xr_single<G, ASYM, MR, T, XI>;
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kXrMaxLds);
            if (e != hipSuccess) return e;
            raised = true;
        }
        const GemvProblem &p = b.p[0];
        k<<<grid, block, lds, st>>>(p.codes, p.scales, p.x, p.y, p.N, p.K, p.ktiles, p.tw, b.M, b.W, p.zeros);
    } else {
        static bool raised = false;
        auto k = gemv_xr_batch<G, ASYM, MR, T, XI>;
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kXrMaxLds);
            if (e != hipSuccess) return e;
            raised = true;
        }
        k<<<grid, block, lds, st>>>(b);
    }
    return hipGetLastError();
}

template <int G, bool ASYM>
hipError_t launch_xr(int T, int XI, dim3 grid, dim3 block, size_t lds, hipStream_t st, const GemvBatch &b)
{
    if (T <= 4) {
        if (XI == 1) return launch_xr_k<G, ASYM, 4, 1>(grid, block, lds, st, b);
        if (XI == 2) return launch_xr_k<G, ASYM, 4, 2>(grid, block, lds, st, b);
        return launch_xr_k<G, ASYM, 4, 4>(grid, block, lds, st, b);
    }
    if (XI == 1) return launch_xr_k<G, ASYM, 8, 1>(grid, block, lds, st, b);
    if (XI == 2) return launch_xr_k<G, ASYM, 8, 2>(grid, block, lds, st, b);
    return launch_xr_k<G, ASYM, 8, 4>(grid, block, lds, st, b);
}

template <int G, bool ASYM, int MR>
hipError_t launch_p(int P, dim3 grid, dim3 block, size_t lds, hipStream_t s, const GemvBatch &b)
{
    if (P <= 4)
        gemv_w4_kernel<G, ASYM, MR, 4><<<grid, block, lds, s>>>(b);
    else
        gemv_w4_kernel<G, ASYM, MR, 8><<<grid, block, lds, s>>>(b);
    return hipGetLastError();
}

template <int G, bool ASYM>
hipError_t launch_gm(int MR, int P, dim3 grid, dim3 block, size_t lds, hipStream_t s, const GemvBatch &b)
{
    if (MR == 1) return launch_p<G, ASYM, 1>(P, grid, block, lds, s, b);
    if (MR == 2) return launch_p<G, ASYM, 2>(P, grid, block, lds, s, b);
    return launch_p<G, ASYM, 4>(P, grid, block, lds, s, b);
}

}  // namespace

size_t gemv_w4_workspace(int, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemv_w4_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                const _Float16 *const *x, _Float16 *const *y, hipStream_t s)
{
    if (M == 0 || count == 0) return hipSuccess;
    GemvBatch b;
    int64_t strips = 0, kt = 0;
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
        strips += L[i].strips;
        if (L[i].ktiles > kt) kt = L[i].ktiles;
    }
    b.count = count;
    b.M = M;
    b.W = 0;
    if (strips == 0) return hipSuccess;
    const int MR = M == 1 ? 1 : (M <= 8 ? 2 : 4);     // accumulators per lane (see a_token)
    const int G = L[0].G;
    const bool asym = L[0].asym;
    // waves per workgroup: enough that each wave holds at most 4 tiles (8 for
    // long K), capped at 16 waves
    int W = (int)((kt + 3) / 4);
    if (W < 1) W = 1;
    if (W > 16) W = 16;
    const int64_t T = (kt + W - 1) / W;
    int64_t max_strips = 0;
    for (int i = 0; i < kMaxGemvBatch; ++i) b.first[i] = 0x7FFFFFFF;
    for (int i = 0, f = 0; i < count; ++i) {
        b.p[i].tw = (int)((L[i].ktiles + W - 1) / W);
        b.first[i] = f;
        f += (int)L[i].strips;
        if (L[i].strips > max_strips) max_strips = L[i].strips;
    }
    b.W = W;
    // one workgroup per strip.  The streaming kernel lays up to 4 problems end
    // to end over blockIdx.x; otherwise (and in the round-based kernel)
    // blockIdx.x = strip and blockIdx.y = problem.
    const dim3 grid((unsigned)max_strips, (unsigned)count), block((unsigned)(W * 64));
    const dim3 grid_flat((unsigned)strips);

    // streaming kernel whenever the x block fits.  Two strips per workgroup
    // for 5 or more tokens and up to four tiles per wave when the launch has at
    // least 1024 strips (512 workgroups: two per compute unit) and the two
    // strips' partial sums fit beside x.  (Measured on the 8B gate+up launch,
    // asymmetric G=32: 25.4 -> 23.4 us at M = 8, but 20.1 -> 21.6 us at M = 4,
    // where one-strip workgroups still fit three to a compute unit.)
    if (T <= 4 && MR >= 2 && M >= kNs2MinM && count <= 4 && strips >= kNs2MinStrips &&
        v2_lds(M, (int)kt, W, MR, asym, 2).total <= kV2MaxLds) {
        b.ct = 0;
        int64_t wgs = 0;
        for (int i = 0; i < count; ++i) {
            b.first[i] = (int)wgs;
            wgs += (L[i].strips + 1) / 2;
        }
        const dim3 g2((unsigned)wgs);
        const size_t lds = (size_t)v2_lds(M, (int)kt, W, MR, asym, 2).total;
        switch (G) {
        case 32: return asym ? launch_v2_ns2<32, true>(MR, (int)T, g2, block, lds, s, b)
                             : launch_v2_ns2<32, false>(MR, (int)T, g2, block, lds, s, b);
        case 64: return asym ? launch_v2_ns2<64, true>(MR, (int)T, g2, block, lds, s, b)
                             : launch_v2_ns2<64, false>(MR, (int)T, g2, block, lds, s, b);
        default: return asym ? launch_v2_ns2<128, true>(MR, (int)T, g2, block, lds, s, b)
                             : launch_v2_ns2<128, false>(MR, (int)T, g2, block, lds, s, b);
        }
    }
    if (T <= 8) {
        const V2Lds lay = v2_lds(M, (int)kt, W, MR, asym);
        if (lay.total <= kV2MaxLds) {
            b.ct = 0;
            const size_t lds = (size_t)lay.total;
            const dim3 g2 = count <= 4 ? grid_flat : grid;
            switch (G) {
            case 32: return asym ? launch_v2<32, true>(MR, (int)T, g2, block, lds, s, b)
                                 : launch_v2<32, false>(MR, (int)T, g2, block, lds, s, b);
            case 64: return asym ? launch_v2<64, true>(MR, (int)T, g2, block, lds, s, b)
                                 : launch_v2<64, false>(MR, (int)T, g2, block, lds, s, b);
            default: return asym ? launch_v2<128, true>(MR, (int)T, g2, block, lds, s, b)
                                 : launch_v2<128, false>(MR, (int)T, g2, block, lds, s, b);
            }
        }
    }

    // M >= 3 when the whole activation block does not fit: per-wave activation
    // rings (up to 8 rows with 8 tiles per wave, 16 rows with 4)
    if (T <= 8 && MR >= 2) {
        const int XI = xr_rows(M) / 4;
        const int64_t lds = xr_lds(M, W, MR);
        if (lds <= kXrMaxLds) {
            b.ct = 0;
            switch (G) {
            case 32: return asym ? launch_xr<32, true>((int)T, XI, grid, block, (size_t)lds, s, b)
                                 : launch_xr<32, false>((int)T, XI, grid, block, (size_t)lds, s, b);
            case 64: return asym ? launch_xr<64, true>((int)T, XI, grid, block, (size_t)lds, s, b)
                                 : launch_xr<64, false>((int)T, XI, grid, block, (size_t)lds, s, b);
            default: return asym ? launch_xr<128, true>((int)T, XI, grid, block, (size_t)lds, s, b)
                                 : launch_xr<128, false>((int)T, XI, grid, block, (size_t)lds, s, b);
            }
        }
    }

    // round-based kernel: activations staged in chunks of K tiles
    const int P = T <= 4 ? 4 : 8;
    // activation chunk: every K tile of a round when it fits the LDS budget
    const int64_t round_tiles = (int64_t)W * P;
    int64_t ct = kt < round_tiles ? kt : round_tiles;
    while (ct > 1 && gemv_lds_bytes(M, (int)ct, W, MR) > (int64_t)kMaxLds) ct = (ct + 1) / 2;
    if (ct < 1) ct = 1;
    b.ct = (int)ct;
    const size_t lds = (size_t)gemv_lds_bytes(M, (int)ct, W, MR);
    switch (G) {
    case 32: return asym ? launch_gm<32, true>(MR, P, grid, block, lds, s, b) : launch_gm<32, false>(MR, P, grid, block, lds, s, b);
    case 64: return asym ? launch_gm<64, true>(MR, P, grid, block, lds, s, b) : launch_gm<64, false>(MR, P, grid, block, lds, s, b);
    default: return asym ? launch_gm<128, true>(MR, P, grid, block, lds, s, b) : launch_gm<128, false>(MR, P, grid, block, lds, s, b);
    }
}

hipError_t launch_gemv_w4(const W4Layout &L, int M, const uint8_t *packed, const _Float16 *x,
                          _Float16 *y, void *, size_t, hipStream_t s)
{
    return launch_gemv_w4_batch(&L, 1, M, &packed, &x, &y, s);
}

}  // namespace lowbit
