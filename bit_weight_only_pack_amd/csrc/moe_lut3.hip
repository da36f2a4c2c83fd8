// moe_lut3.hip -- 3-bit LUT-codebook MoE: weight re-pack, routing alignment
// and the grouped expert GEMM with MXFP8 activations.
//
// Format ("vLLM PR #62759 analysis", section "Format"): every weight is a
// 3-bit index into an 8-entry E4M3 codebook; a codebook and one UE8M0
// exponent are shared by a tile of 8 output channels x 64 K.  Activations are
// MXFP8: E4M3 values with one UE8M0 scale per 32 K.  Rows reach the experts
// through sorted slot ids (section "A gather": a slot is valid when its id is
// below the number of routed slots); experts that are not local produce zero
// rows (section "Expert parallelism").
//
// MI355X design (the page's tensor-core LUT decode does not exist on CDNA4):
//   * Load-time re-pack into 16-column x 128-K units in the lane order of
//     v_mfma_scale_f32_16x16x128_f8f6f4, measured on gfx950: lane l holds
//     column (row) l % 16; with g = l / 16 its bytes 0..15 are K 16g..16g+15
//     and bytes 16..31 are K 64+16g..64+16g+15; the block scale of 32-K block
//     b of row/column r is taken from lane r + 16b.  A lane's 32 indices take
//     12 bytes arranged so
//     that each run of four indices becomes byte selectors with one to four
//     bit operations; one v_perm_b32 per four weights then turns selectors into
//     E4M3 bytes from the codebook held in two registers.  The 3-bit format is
//     kept: 768 index bytes + 32 codebook bytes + 4 exponent bytes per 2048
//     weights = 3.140625 bits per weight.
//   * The block-scaled fp8 MFMA applies the activation UE8M0 scale per 32 K
//     (scale A) and the tile exponent (scale B, the same exponent for both
//     32-K halves of a 64-K tile), accumulating in fp32.
//   * One workgroup per (expert, 128-column tile) loops over all 16-row
//     blocks of its expert, so each expert's weights stream from HBM once.
//   * The gate/up GEMM of the layer can leave as SiLU(gate) * up in MXFP8
//     (FUSE): a tile pairs gate columns with the matching up columns, and the
//     epilogue encodes them with the stand-alone kernels' definitions.
#include "lowbit_internal.hpp"
#include "moe_align.hpp"
#include "mxfp8.hpp"

#include <algorithm>

namespace lowbit {

namespace {

constexpr int kThreads = 256;
inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

// Bit position of index j (0..31) of a lane inside its 3 packed dwords.
// Indices 0..23 sit in bits 0-2 / 3-5 of the bytes of dwords 0..2; indices
// 24..31 use bits 6-7 of dwords 0/1 for their low two bits and bit 6/7 of
// dword 2 for the high bit.
__host__ __device__ inline void lut_put(uint32_t w[3], int j, uint32_t v)
{
    if (j < 24) {
        const int d = j / 8, half = (j / 4) & 1, b = j & 3;
        w[d] |= (v & 7u) << (8 * b + 3 * half);
    } else {
        const int hi = j >= 28, b = j & 3;
        w[hi] |= (v & 3u) << (8 * b + 6);
        w[2] |= ((v >> 2) & 1u) << (8 * b + 6 + hi);
    }
}

__host__ __device__ inline uint32_t lut_get(const uint32_t w[3], int j)
{
    if (j < 24) {
        const int d = j / 8, half = (j / 4) & 1, b = j & 3;
        return (w[d] >> (8 * b + 3 * half)) & 7u;
    }
    const int hi = j >= 28, b = j & 3;
    return ((w[hi] >> (8 * b + 6)) & 3u) | (((w[2] >> (8 * b + 6 + hi)) & 1u) << 2);
}

// ---------------------------------------------------------------- re-pack
// K offset (within a 128-K step) of byte j of lane group lg
__host__ __device__ inline int lane_k(int lg, int j) { return 64 * (j >> 4) + 16 * lg + (j & 15); }

__global__ void lut3_pack_idx(const uint8_t *__restrict__ idx, uint32_t *__restrict__ out, int64_t N, int64_t K,
                              int64_t strips, int64_t ksteps, int64_t total_lanes)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // one thread per lane-slot
    if (g >= total_lanes) return;
    const int lane = (int)(g & 63);
    const int64_t unit = g >> 6;                                       // (e, s, t)
    const int64_t t = unit % ksteps, s = (unit / ksteps) % strips, e = unit / (ksteps * strips);
    const int64_t n = s * 16 + (lane & 15);
    uint32_t w[3] = {0u, 0u, 0u};
    if (n < N)
        for (int j = 0; j < 32; ++j) {
            const int64_t k = t * 128 + lane_k(lane >> 4, j);
            if (k < K) lut_put(w, j, idx[(e * N + n) * K + k]);
        }
    out[g * 3 + 0] = w[0];
    out[g * 3 + 1] = w[1];
    out[g * 3 + 2] = w[2];
}

__global__ void lut3_unpack_idx(const uint32_t *__restrict__ in, uint8_t *__restrict__ idx, int64_t N, int64_t K,
                                int64_t strips, int64_t ksteps, int64_t total_lanes)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= total_lanes) return;
    const int lane = (int)(g & 63);
    const int64_t unit = g >> 6;
    const int64_t t = unit % ksteps, s = (unit / ksteps) % strips, e = unit / (ksteps * strips);
    const int64_t n = s * 16 + (lane & 15);
    if (n >= N) return;
    const uint32_t w[3] = {in[g * 3 + 0], in[g * 3 + 1], in[g * 3 + 2]};
    for (int j = 0; j < 32; ++j) {
        const int64_t k = t * 128 + lane_k(lane >> 4, j);
        if (k < K) idx[(e * N + n) * K + k] = (uint8_t)lut_get(w, j);
    }
}

// unit c = (column half h, K half kh) -> codebook / exponent of tile (n/8, k/64)
__global__ void lut3_pack_meta(const uint8_t *__restrict__ cb, const uint8_t *__restrict__ ex,
                               uint8_t *__restrict__ cb_out, uint8_t *__restrict__ ex_out, int64_t N, int64_t K,
                               int64_t strips, int64_t ksteps, int64_t total)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // one thread per (unit, c)
    if (g >= total) return;
    const int c = (int)(g & 3);
    const int64_t unit = g >> 2;
    const int64_t t = unit % ksteps, s = (unit / ksteps) % strips, e = unit / (ksteps * strips);
    const int64_t nt = s * 2 + (c >> 1), kt = t * 2 + (c & 1);       // tile indices (8 cols x 64 K)
    const int64_t ntiles = N / 8, ktiles = K / 64;
    const bool ok = nt < ntiles && kt < ktiles;
    const int64_t src = (e * ntiles + nt) * ktiles + kt;
    for (int i = 0; i < 8; ++i) cb_out[g * 8 + i] = ok ? cb[src * 8 + i] : (uint8_t)0;
    ex_out[g] = ok ? ex[src] : (uint8_t)127;
}

__global__ void lut3_unpack_meta(const uint8_t *__restrict__ cb_in, const uint8_t *__restrict__ ex_in,
                                 uint8_t *__restrict__ cb, uint8_t *__restrict__ ex, int64_t N, int64_t K,
                                 int64_t strips, int64_t ksteps, int64_t total)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= total) return;
    const int c = (int)(g & 3);
    const int64_t unit = g >> 2;
    const int64_t t = unit % ksteps, s = (unit / ksteps) % strips, e = unit / (ksteps * strips);
    const int64_t nt = s * 2 + (c >> 1), kt = t * 2 + (c & 1);
    const int64_t ntiles = N / 8, ktiles = K / 64;
    if (nt >= ntiles || kt >= ktiles) return;
    const int64_t dst = (e * ntiles + nt) * ktiles + kt;
    for (int i = 0; i < 8; ++i) cb[dst * 8 + i] = cb_in[g * 8 + i];
    ex[dst] = ex_in[g];
}

// ---------------------------------------------------------------- align
__global__ __launch_bounds__(kAlignThreads)
void moe_align_kernel(const int32_t *__restrict__ topk_ids, int num_valid, int E, int block_m,
                      const int32_t *__restrict__ expert_map, int32_t *__restrict__ sorted_ids,
                      int32_t *__restrict__ expert_offsets, int32_t *__restrict__ block_expert,
                      int32_t *__restrict__ num_post_padded, int capacity)
{
    moe_align_block(topk_ids, num_valid, E, block_m, expert_map, sorted_ids, expert_offsets, block_expert,
                    num_post_padded, capacity);
}

// ---------------------------------------------------------------- grouped GEMM
typedef int i8v __attribute__((ext_vector_type(8)));

constexpr int kMoeWaves = 4;          // 4 waves x 2 strips = 128 columns per workgroup
constexpr int kStripsPerWave = 2;
constexpr int kMaxMBlocks = 4;        // 16-row blocks held at once (64 rows); more rows -> more passes

struct MoeArgs {
    const uint8_t *idx, *cb, *ex;      // packed sections
    const uint8_t *aq, *as;            // activations [rows][K] E4M3, scales [rows][K/32] UE8M0
    const int32_t *sorted_ids, *expert_offsets, *block_expert;
    uint16_t *out;                     // bf16 [num_valid][N]
    uint8_t *fq, *fs;                  // fused gate/up: SiLU(gate) * up as MXFP8 [num_valid][N/2], [..][N/64]
    int E, N, K, strips, ksteps, a_row_div, num_valid, block_m, n_tiles, a_rows;
};

// 32 decoded E4M3 bytes of one lane from its 12 index bytes; bytes 0..15 use
// the codebook of the first 64-K half (c0 = lo dword, c1 = hi dword), bytes
// 16..31 that of the second half (c2, c3)
__device__ __forceinline__ i8v lut3_decode(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t c0, uint32_t c1,
                                           uint32_t c2, uint32_t c3)
{
    const uint32_t m7 = 0x07070707u;
    const uint32_t s0 = w0 & m7;
    const uint32_t s1 = (w0 >> 3) & m7;
    const uint32_t s2 = w1 & m7;
    const uint32_t s3 = (w1 >> 3) & m7;
    const uint32_t s4 = w2 & m7;
    const uint32_t s5 = (w2 >> 3) & m7;
    const uint32_t s6 = ((w0 >> 6) & 0x03030303u) | ((w2 >> 4) & 0x04040404u);
    const uint32_t s7 = ((w1 >> 6) & 0x03030303u) | ((w2 >> 5) & 0x04040404u);
    // selector byte v in 0..3 picks byte v of the lo dword, 4..7 byte v-4 of the hi dword
    i8v r;
    r[0] = (int)__builtin_amdgcn_perm(c1, c0, s0);
    r[1] = (int)__builtin_amdgcn_perm(c1, c0, s1);
    r[2] = (int)__builtin_amdgcn_perm(c1, c0, s2);
    r[3] = (int)__builtin_amdgcn_perm(c1, c0, s3);
    r[4] = (int)__builtin_amdgcn_perm(c3, c2, s4);
    r[5] = (int)__builtin_amdgcn_perm(c3, c2, s5);
    r[6] = (int)__builtin_amdgcn_perm(c3, c2, s6);
    r[7] = (int)__builtin_amdgcn_perm(c3, c2, s7);
    return r;
}

__global__ __launch_bounds__(kMoeWaves * 64)
void moe_lut3_gemm_kernel(MoeArgs p)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int e = blockIdx.x / p.n_tiles;                      // global expert
    const int nt = blockIdx.x % p.n_tiles;
    const int row0 = p.expert_offsets[e], row1 = p.expert_offsets[e + 1];
    if (row0 >= row1) return;                                  // no slot routed here
    const int local = p.block_expert[row0 / p.block_m];
    const int strip_base = nt * (kMoeWaves * kStripsPerWave) + wave * kStripsPerWave;

    if (local < 0) {
        // expert not on this device: its routed slots get zero rows
        for (int rr = row0 + (threadIdx.x >> 4); rr < row1; rr += kMoeWaves * 4) {
            const int sid = p.sorted_ids[rr];
            if (sid >= p.num_valid) continue;
            for (int c = (threadIdx.x & 15); c < kMoeWaves * kStripsPerWave * 16; c += 16) {
                const int n = nt * kMoeWaves * kStripsPerWave * 16 + c;
                if (n < p.N) p.out[(int64_t)sid * p.N + n] = 0;
            }
        }
        return;
    }

    const int64_t units_per_strip = p.ksteps;
    const int64_t expert_units = (int64_t)p.strips * p.ksteps;
    const auto irs = buffer_rsrc(p.idx, (uint32_t)((int64_t)(p.E) * expert_units * 768));
    const auto crs = buffer_rsrc(p.cb, (uint32_t)((int64_t)(p.E) * expert_units * 32));
    const auto ers = buffer_rsrc(p.ex, (uint32_t)((int64_t)(p.E) * expert_units * 4));
    const auto ars = buffer_rsrc(p.aq, (uint32_t)((int64_t)p.a_rows * p.K));
    const auto srs = buffer_rsrc(p.as, (uint32_t)((int64_t)p.a_rows * (p.K / 32)));
    const int colhalf = r16 >> 3;                              // which 8-column tile of the strip
    const int exsel = (colhalf << 1) | (kg >> 1);              // exponent of this lane's 32-K block
    const int k_chunks = p.K / 32;

    for (int pass = row0; pass < row1; pass += kMaxMBlocks * 16) {
        const int nmb = min(kMaxMBlocks, (row1 - pass) / 16);
        // slot ids and activation rows of this lane's A row in each block
        int arow[kMaxMBlocks];
        bool aok[kMaxMBlocks];
#pragma unroll
        for (int mb = 0; mb < kMaxMBlocks; ++mb) {
            const int sid = mb < nmb ? p.sorted_ids[pass + mb * 16 + r16] : p.num_valid;
            aok[mb] = sid < p.num_valid;
            arow[mb] = aok[mb] ? sid / p.a_row_div : 0;
        }
        f4 acc[kMaxMBlocks][kStripsPerWave];
#pragma unroll
        for (int mb = 0; mb < kMaxMBlocks; ++mb)
#pragma unroll
            for (int j = 0; j < kStripsPerWave; ++j) acc[mb][j] = f4{0.f, 0.f, 0.f, 0.f};

        for (int t = 0; t < p.ksteps; ++t) {
            // weights of this wave's strips for K step t
            uint32_t w[kStripsPerWave][3];
            u4 cbk[kStripsPerWave];
            int bscale[kStripsPerWave];
#pragma unroll
            for (int j = 0; j < kStripsPerWave; ++j) {
                const int s = strip_base + j;
                const bool ok = s < p.strips;
                const int64_t unit = ((int64_t)local * p.strips + s) * units_per_strip + t;
                const auto iv = __builtin_amdgcn_raw_buffer_load_b96(irs, ok ? (uint32_t)(unit * 768 + lane * 12) : kBufferOob, 0, 0);
                w[j][0] = iv[0];
                w[j][1] = iv[1];
                w[j][2] = iv[2];
                // both K halves' codebooks of this lane's 8-column tile (16 bytes)
                cbk[j] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (uint32_t)(unit * 32 + colhalf * 16) : kBufferOob, 0, 0);
                bscale[j] = ok ? (int)__builtin_amdgcn_raw_buffer_load_b8(ers, (uint32_t)(unit * 4 + exsel), 0, 0) : 127;
            }
            // activations of the lane's row: K 16kg..+16 and 64+16kg..+16 of this
            // step; the scale of 32-K block kg (this lane provides block kg's scale)
            i8v a[kMaxMBlocks];
            int ascale[kMaxMBlocks];
            const int kc = t * 4 + kg;                                 // 32-K block of the scale
            const int k_lo = t * 128 + 16 * kg, k_hi = k_lo + 64;
#pragma unroll
            for (int mb = 0; mb < kMaxMBlocks; ++mb) {
                const bool ok = mb < nmb && aok[mb];
                const uint32_t row = (uint32_t)arow[mb] * (uint32_t)p.K;
                const u4 lo = __builtin_amdgcn_raw_buffer_load_b128(ars, ok && k_lo < p.K ? row + k_lo : kBufferOob, 0, 0);
                const u4 hi = __builtin_amdgcn_raw_buffer_load_b128(ars, ok && k_hi < p.K ? row + k_hi : kBufferOob, 0, 0);
                a[mb] = i8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                ascale[mb] = ok && kc < k_chunks
                                 ? (int)__builtin_amdgcn_raw_buffer_load_b8(srs, (uint32_t)arow[mb] * (uint32_t)k_chunks + kc, 0, 0)
                                 : 127;
            }
#pragma unroll
            for (int j = 0; j < kStripsPerWave; ++j) {
                const i8v b = lut3_decode(w[j][0], w[j][1], w[j][2], cbk[j].x, cbk[j].y, cbk[j].z, cbk[j].w);
#pragma unroll
                for (int mb = 0; mb < kMaxMBlocks; ++mb)
                    if (mb < nmb)
                        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a[mb], b, acc[mb][j], 0, 0, 0, ascale[mb], 0, bscale[j]);
            }
        }
        // store: lane holds column (lane % 16), rows 4*(lane/16) + i of each block
#pragma unroll
        for (int mb = 0; mb < kMaxMBlocks; ++mb) {
            if (mb >= nmb) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sid = p.sorted_ids[pass + mb * 16 + kg * 4 + i];
                if (sid >= p.num_valid) continue;
#pragma unroll
                for (int j = 0; j < kStripsPerWave; ++j) {
                    const int n = (strip_base + j) * 16 + r16;
                    if (n < p.N) {
                        const __bf16 v = (__bf16)acc[mb][j][i];
                        p.out[(int64_t)sid * p.N + n] = __builtin_bit_cast(uint16_t, v);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- grouped GEMM, activations in LDS
// The same product as moe_lut3_gemm_kernel for passes whose activation rows
// fit in LDS.  One workgroup of 8 waves per (expert, group of column tiles):
// each pass stages its activation rows and block scales in LDS once, then
// every wave walks its strip of each tile of the group along K; the weight
// stream runs D - 1 K steps ahead of the MFMAs in a ring of register slots
// that continues from one tile into the next (unrolled so that no slot is
// copied while its loads are in flight), and it is the only vector-memory
// traffic of the loop: finished tiles go to an LDS output block, which is
// written out once per pass.  (A store inside the loop would be the last
// vector-memory operation before the next loads; reusing its registers
// would make the compiler wait for it, and so for every load in flight.)
constexpr int kGWaves = 16;                         // waves per workgroup
constexpr int kGSPW = 1;                            // strips per wave
constexpr int kGTileStrips = kGWaves * kGSPW;       // 16 strips = 256 columns per tile
constexpr int kLdsRowPad = 16;                      // bytes added to each staged row (rows fall in different banks)
constexpr int kMoeScaleBytesMax = 4 * kGWaves * 64; // block-scale bytes of one pass: four per thread

// LDS-direct load: lane i's 16 bytes land at lds + 16 i (no registers involved)
template <int BYTES>
__device__ __forceinline__ void lds_load(__amdgpu_buffer_rsrc_t rs, uint8_t *lds, uint32_t off)
{
    static_assert(BYTES == 16, "LDS-direct load size");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

struct WSlot {
    uint32_t w[kGSPW][3];
    u4 cbk[kGSPW];
    uint32_t bscale[kGSPW];
};

// K rounded up to whole 128-K steps: a staged row holds the zero-filled tail
// of its last step, which the MFMAs of that step read (times zero weights;
// bytes left unwritten could hold E4M3 NaN patterns)
__host__ __device__ constexpr int moe_kpad(int K) { return (K + 127) / 128 * 128; }

// LDS of one workgroup: activation rows, their block scales, slot ids, then
// the bf16 output block of the group's tiles
struct MoeLds {
    int s_off, sid_off, out_off, bytes;
};
__host__ __device__ inline MoeLds moe_lds_layout(int MB, int K, int tiles)
{
    MoeLds l;
    // the rows are filled by LDS-direct loads of 1 KiB per instruction, which
    // write whole chunks: the region is rounded up to the chunk size
    l.s_off = (MB * 16 * (moe_kpad(K) + kLdsRowPad) + 1023) & ~1023;
    l.sid_off = l.s_off + MB * 16 * (K / 32);
    l.out_off = (l.sid_off + MB * 16 * 4 + 15) & ~15;
    l.bytes = l.out_off + tiles * MB * 16 * kGTileStrips * 16 * 2;
    return l;
}
// the staging part alone (rows, scales, slot ids): what decides the pass size
__host__ __device__ inline int moe_lds_bytes(int MB, int K) { return moe_lds_layout(MB, K, 0).bytes; }

struct MoeGroupArgs {
    MoeArgs m;
    int gtiles, tiles_per_group, n_groups;         // tiles of 256 columns; tiles per workgroup
};

// FUSE (the gate/up GEMM of the layer, N = 2I, I % 128 == 0): a tile is 128
// gate columns (waves 0-7) and the matching 128 up columns (waves 8-15), and
// the pass's output leaves as SiLU(gate) * up in MXFP8 (mxfp8.hpp) instead of
// bf16 gate/up rows; gate and up are rounded to bf16 first, as the layer's
// stand-alone kernels see them.
// The fields the prologue's dependent reads need come first as scalar kernel
// arguments (13 dwords), which the hardware preloads into scalar registers:
// the first routing read goes out without a kernel-argument round trip.  The
// rest arrive with the argument block, read in parallel.
template <int MB, int D, bool FUSE>
__global__ __launch_bounds__(kGWaves * 64)
void moe_lut3_gemm_lds_kernel(const int32_t *expert_offsets, const int32_t *block_expert, const int32_t *sorted_ids,
                              int n_groups_a, int tiles_per_group_a, int gtiles_a, int block_m_a, int num_valid_a,
                              int strips_a, int ksteps_a, MoeGroupArgs ga)
{
    MoeArgs p = ga.m;
    p.expert_offsets = expert_offsets;
    p.block_expert = block_expert;
    p.sorted_ids = sorted_ids;
    p.block_m = block_m_a;
    p.num_valid = num_valid_a;
    p.strips = strips_a;
    p.ksteps = ksteps_a;
    ga.n_groups = n_groups_a;
    ga.tiles_per_group = tiles_per_group_a;
    ga.gtiles = gtiles_a;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int e = blockIdx.x / ga.n_groups;                   // global expert
    const int grp = blockIdx.x % ga.n_groups;
    const int tile0 = grp * ga.tiles_per_group;
    const int ntl = min(ga.tiles_per_group, ga.gtiles - tile0);
    if (ntl <= 0) return;
    const int row0 = p.expert_offsets[e], row1 = p.expert_offsets[e + 1];
    if (row0 >= row1) return;                                  // no slot routed here
    // the first pass's slot ids (lane i: row i of the pass, in every wave) go
    // out together with the local-expert read: both need only row0
    static_assert(MB * 16 <= 64, "one pass row per lane");
    int sidv = lane < min(MB * 16, row1 - row0) ? p.sorted_ids[row0 + lane] : p.num_valid;
    const int local = p.block_expert[row0 / p.block_m];
    const int col0 = tile0 * kGTileStrips * 16, col1 = min(p.N, (tile0 + ntl) * kGTileStrips * 16);
    constexpr int kHalf = kGTileStrips / 2;                    // FUSE: gate (and up) strips per tile
    const int half_strips = p.strips / 2;

    if (local < 0) {
        // expert not on this device: its routed slots get zero rows (FUSE: the
        // zero activation, codes 0 and scale byte 127, as MXFP8 gives for zeros)
        if constexpr (FUSE) {
            const int I = p.N / 2;
            const int a0 = tile0 * kHalf * 16, a1 = min(I, (tile0 + ntl) * kHalf * 16);
            for (int rr = row0 + (threadIdx.x >> 4); rr < row1; rr += kGWaves * 4) {
                const int sid = p.sorted_ids[rr];
                if (sid >= p.num_valid) continue;
                for (int a = a0 + (threadIdx.x & 15); a < a1; a += 16) {
                    p.fq[(int64_t)sid * I + a] = 0;
                    if ((a & 31) == 0) p.fs[(int64_t)sid * (I / 32) + a / 32] = 127;
                }
            }
        } else {
            for (int rr = row0 + (threadIdx.x >> 4); rr < row1; rr += kGWaves * 4) {
                const int sid = p.sorted_ids[rr];
                if (sid >= p.num_valid) continue;
                for (int n = col0 + (threadIdx.x & 15); n < col1; n += 16) p.out[(int64_t)sid * p.N + n] = 0;
            }
        }
        return;
    }

    const int K = p.K, ksteps = p.ksteps, k_chunks = K / 32;
    const int astride = moe_kpad(K) + kLdsRowPad;
    const MoeLds lay = moe_lds_layout(MB, K, ga.tiles_per_group);
    uint8_t *a_lds = smem;                                     // [MB*16][astride]
    uint8_t *s_lds = smem + lay.s_off;                         // [MB*16][k_chunks]
    int *sid_lds = reinterpret_cast<int *>(smem + lay.sid_off);   // [MB*16]
    uint16_t *o_lds = reinterpret_cast<uint16_t *>(smem + lay.out_off);   // [tile][MB*16][256] bf16
    constexpr int kTileCols = kGTileStrips * 16;

    // weight descriptors over the local expert's units (strips past N read zeros)
    const int64_t eunit0 = (int64_t)local * p.strips * ksteps;
    const uint32_t eunits = (uint32_t)(p.strips * ksteps);
    const auto irs = buffer_rsrc(p.idx + eunit0 * 768, eunits * 768);
    const auto crs = buffer_rsrc(p.cb + eunit0 * 32, eunits * 32);
    const auto ers = buffer_rsrc(p.ex + eunit0 * 4, eunits * 4);
    const auto ars = buffer_rsrc(p.aq, (uint32_t)((int64_t)p.a_rows * K));
    const auto srs = buffer_rsrc(p.as, (uint32_t)((int64_t)p.a_rows * k_chunks));
    const int colhalf = r16 >> 3;                              // which 8-column tile of the strip
    const int exsel = (colhalf << 1) | (kg >> 1);              // exponent of this lane's 32-K block
    const int total = ntl * ksteps;                            // (tile, K step) pairs of this wave

    // weights of pair g = ti * ksteps + t for this wave's two strips of tile ti
    auto load_w = [&](WSlot &ws, int g) __attribute__((always_inline)) {
        const int ti = g / ksteps, t = g - ti * ksteps;
        const bool live = g < total;
#pragma unroll
        for (int j = 0; j < kGSPW; ++j) {
            const int s = FUSE ? (wave / kHalf) * half_strips + (tile0 + ti) * kHalf + wave % kHalf
                               : (tile0 + ti) * kGTileStrips + wave * kGSPW + j;
            const bool ok = live && s < p.strips;
            const uint32_t unit = (uint32_t)(s * ksteps + t);
            const auto iv = __builtin_amdgcn_raw_buffer_load_b96(irs, ok ? unit * 768 + lane * 12 : kBufferOob, 0, 0);
            ws.w[j][0] = iv[0];
            ws.w[j][1] = iv[1];
            ws.w[j][2] = iv[2];
            // both K halves' codebooks of this lane's 8-column tile (16 bytes)
            ws.cbk[j] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? unit * 32 + colhalf * 16 : kBufferOob, 0, 0);
            // the unit's four tile exponents; the lane's own byte is picked at use
            ws.bscale[j] = __builtin_amdgcn_raw_buffer_load_b32(ers, ok ? unit * 4 : kBufferOob, 0, 0);
        }
    };

    for (int pass = row0; pass < row1; pass += MB * 16) {
        const int nmb = min(MB, (row1 - pass) / 16);
        const int prow = nmb * 16;
        if (pass != row0) {
            __syncthreads();                                   // previous pass done with the LDS blocks
            sidv = lane < prow ? p.sorted_ids[pass + lane] : p.num_valid;
        }
        // activation row of each pass row (lane i: row i), -1 for padding slots
        const int arowv = sidv < p.num_valid ? sidv / p.a_row_div : -1;
        if (wave == 0 && lane < MB * 16) sid_lds[lane] = lane < prow ? sidv : p.num_valid;
        // 1. stage the pass's activation rows and block scales.  The rows (each
        //    with its zero tail to whole 128-K steps and its padding) go
        //    straight into LDS by LDS-direct loads that cover the region byte
        //    for byte (bytes past K or past the pass's rows read zeros); the
        //    scales go to registers.  Both are issued before the pass's first
        //    weight loads: loads of a wave complete in issue order, so they
        //    land ahead of the weight ring.
        {
            const int abytes = prow * astride;
            for (int ci = wave; ci * 1024 < abytes; ci += kGWaves) {
                const int d = ci * 1024 + lane * 16;
                const int row = d / astride, k = d - row * astride;
                const int ar = __shfl(arowv, row < 64 ? row : 0);
                const bool ok = row < prow && ar >= 0 && k < K;
                lds_load<16>(ars, a_lds + ci * 1024, ok ? (uint32_t)ar * (uint32_t)K + (uint32_t)k : kBufferOob);
            }
        }
        // the block scales (one byte per row and 32-K block) into registers,
        // issued before the ring as well, written to LDS once they land
        constexpr int kScalePerThread = kMoeScaleBytesMax / (kGWaves * 64);
        const int sbytes = prow * k_chunks;
        uint32_t sv[kScalePerThread];
        int sidx[kScalePerThread];
#pragma unroll
        for (int u = 0; u < kScalePerThread; ++u) {
            const int b = (int)threadIdx.x + u * kGWaves * 64;
            const int row = b / k_chunks, c = b - row * k_chunks;
            const int ar = __shfl(arowv, row < 64 ? row : 0);
            const bool ok = b < sbytes && ar >= 0;
            sidx[u] = b;
            sv[u] = __builtin_amdgcn_raw_buffer_load_b8(srs, ok ? (uint32_t)ar * (uint32_t)k_chunks + (uint32_t)c
                                                            : kBufferOob, 0, 0);
        }
        //    Then the pass's first D - 1 weight steps (kept after the staging
        //    loads: the wait below counts on that order).
        __builtin_amdgcn_sched_barrier(0);
        WSlot wsl[D];
#pragma unroll
        for (int d = 0; d < D - 1; ++d) load_w(wsl[d], d);
        __builtin_amdgcn_sched_barrier(0);
        //    Every load issued before them has landed (the ring's may be in
        //    flight): scales to LDS, and publish rows, scales and slot ids.
        constexpr int kRing = (D - 1) * 3 * kGSPW;             // the ring's loads: D - 1 steps x (codes, codebooks, exponents)
        static_assert(kRing < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((kRing & 15) | ((kRing >> 4) << 14) | (7 << 4) | (15 << 8));   // vmcnt(kRing)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kScalePerThread; ++u)
            if (sidx[u] < sbytes) s_lds[sidx[u]] = (uint8_t)sv[u];
        __builtin_amdgcn_s_waitcnt((7 << 4) | 15 | (3 << 14));  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);

        f4 acc[MB][kGSPW];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < kGSPW; ++j) acc[mb][j] = f4{0.f, 0.f, 0.f, 0.f};

        // 2. stream the weights D - 1 pairs ahead (the first D - 1 are in flight)
        int ti = 0, t = 0;                                     // the pair being computed
        auto step = [&](int g, WSlot &wcur, WSlot &wpf) __attribute__((always_inline)) {
            load_w(wpf, g + D - 1);
            if (g < total) {
                const int k_lo = t * 128 + 16 * kg;
                const int kc = t * 4 + kg;                     // this lane supplies block kc's scale
#pragma unroll
                for (int j = 0; j < kGSPW; ++j) {
                    const i8v b = lut3_decode(wcur.w[j][0], wcur.w[j][1], wcur.w[j][2], wcur.cbk[j].x,
                                              wcur.cbk[j].y, wcur.cbk[j].z, wcur.cbk[j].w);
                    const int bs = (int)((wcur.bscale[j] >> (8 * exsel)) & 0xffu);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if (mb < nmb) {
                            const uint8_t *ar = a_lds + (mb * 16 + r16) * astride;
                            const u4 lo = *reinterpret_cast<const u4 *>(ar + k_lo);
                            const u4 hi = *reinterpret_cast<const u4 *>(ar + k_lo + 64);
                            const i8v a = i8v{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                              (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                            const int as = kc < k_chunks ? (int)s_lds[(mb * 16 + r16) * k_chunks + kc] : 127;
                            acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[mb][j], 0, 0,
                                                                                          0, as, 0, bs);
                        }
                    }
                }
                if (t == ksteps - 1) {
                    // 3. tile done: lane holds column (lane % 16), rows 4*(lane/16) + i
                    //    of each block; rounded to bf16 into the LDS output block
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if (mb >= nmb) continue;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
#pragma unroll
                            for (int j = 0; j < kGSPW; ++j) {
                                const int c = (wave * kGSPW + j) * 16 + r16;
                                const __bf16 v = (__bf16)acc[mb][j][i];
                                o_lds[(ti * MB * 16 + mb * 16 + kg * 4 + i) * kTileCols + c] =
                                    __builtin_bit_cast(uint16_t, v);
                            }
                        }
#pragma unroll
                        for (int j = 0; j < kGSPW; ++j) acc[mb][j] = f4{0.f, 0.f, 0.f, 0.f};
                    }
                }
                // advance (arithmetic, not a branch: keeps both counters in registers)
                const int last = t == ksteps - 1 ? 1 : 0;
                ti += last;
                t = last ? 0 : t + 1;
            }
        };
        // unrolled by D so every slot index is a constant; the tail repeats the order
        int g = 0;
        for (; g + D <= total; g += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) step(g + d, wsl[d], wsl[(d + D - 1) % D]);
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d) step(g + d, wsl[d], wsl[(d + D - 1) % D]);

        // 4. the pass's output rows, 16 bytes per thread and step
        __syncthreads();
        if constexpr (FUSE) {
            // SiLU(gate) * up of 8 activation columns per thread; the four
            // threads of a 32-block are one lane quad (rows change every 16
            // threads), as mx_block_put needs
            const int I = p.N / 2;
            constexpr int kActChunks = kTileCols / 2 / 8;      // 16 per row
            for (int idx = threadIdx.x; idx < ntl * nmb * 16 * kActChunks; idx += kGWaves * 64) {
                const int cc = idx % kActChunks;
                const int rr = idx / kActChunks;
                const int tl = rr / (nmb * 16), row = rr - tl * nmb * 16;
                const int sid = sid_lds[row];
                const int a = (tile0 + tl) * (kTileCols / 2) + cc * 8;
                if (sid >= p.num_valid || a >= I) continue;
                const uint16_t *src = o_lds + (tl * MB * 16 + row) * kTileCols + cc * 8;
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float act = mx::silu_f32(mx::bf16_to_f32(src[i])) * mx::bf16_to_f32(src[kTileCols / 2 + i]);
                    v[i] = mx::bf16_to_f32(mx::f32_to_bf16(act));
                }
                mx::mx_block_put(v, p.fq + (int64_t)sid * I + a, p.fs + (int64_t)sid * (I / 32) + a / 32,
                                 (cc & 3) == 0);
            }
            continue;
        }
        constexpr int kChunksPerRow = kTileCols / 8;
        for (int idx = threadIdx.x; idx < ntl * nmb * 16 * kChunksPerRow; idx += kGWaves * 64) {
            const int cc = idx % kChunksPerRow;
            const int rr = idx / kChunksPerRow;                // tile * nmb * 16 + row
            const int tl = rr / (nmb * 16), row = rr - tl * nmb * 16;
            const int sid = sid_lds[row];
            const int n = (tile0 + tl) * kTileCols + cc * 8;
            if (sid >= p.num_valid || n >= p.N) continue;
            const uint16_t *src = o_lds + (tl * MB * 16 + row) * kTileCols + cc * 8;
            uint16_t *dst = p.out + (int64_t)sid * p.N + n;
            if (n + 8 <= p.N && (p.N & 7) == 0) {
                *reinterpret_cast<u4 *>(dst) = *reinterpret_cast<const u4 *>(src);
            } else {
                for (int q = 0; q < 8 && n + q < p.N; ++q) dst[q] = src[q];
            }
        }
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers
Lut3Layout lut3_layout(int64_t E, int64_t N, int64_t K)
{
    Lut3Layout L;
    L.E = E; L.N = N; L.K = K;
    L.strips = (N + 15) / 16;
    L.ksteps = (K + 127) / 128;
    const int64_t units = E * L.strips * L.ksteps;
    L.idx_off = 0;
    L.cb_off = align256(units * 768);
    L.ex_off = align256(L.cb_off + units * 32);
    L.bytes = align256(L.ex_off + units * 4);
    return L;
}

hipError_t launch_lut3_pack(const Lut3Layout &L, const uint8_t *idx, const uint8_t *cb, const uint8_t *ex,
                            uint8_t *packed, hipStream_t s)
{
    const int64_t units = L.E * L.strips * L.ksteps;
    if (units == 0) return hipSuccess;
    const int64_t lanes = units * 64;
    lut3_pack_idx<<<blocks_for(lanes), kThreads, 0, s>>>(idx, reinterpret_cast<uint32_t *>(packed + L.idx_off), L.N,
                                                          L.K, L.strips, L.ksteps, lanes);
    lut3_pack_meta<<<blocks_for(units * 4), kThreads, 0, s>>>(cb, ex, packed + L.cb_off, packed + L.ex_off, L.N, L.K,
                                                              L.strips, L.ksteps, units * 4);
    return hipGetLastError();
}

hipError_t launch_lut3_unpack(const Lut3Layout &L, const uint8_t *packed, uint8_t *idx, uint8_t *cb, uint8_t *ex,
                              hipStream_t s)
{
    const int64_t units = L.E * L.strips * L.ksteps;
    if (units == 0) return hipSuccess;
    const int64_t lanes = units * 64;
    lut3_unpack_idx<<<blocks_for(lanes), kThreads, 0, s>>>(reinterpret_cast<const uint32_t *>(packed + L.idx_off), idx,
                                                            L.N, L.K, L.strips, L.ksteps, lanes);
    lut3_unpack_meta<<<blocks_for(units * 4), kThreads, 0, s>>>(packed + L.cb_off, packed + L.ex_off, cb, ex, L.N,
                                                                L.K, L.strips, L.ksteps, units * 4);
    return hipGetLastError();
}

hipError_t launch_moe_align(const int32_t *topk_ids, int num_valid, int E, int block_m, const int32_t *expert_map,
                            int32_t *sorted_ids, int32_t *expert_offsets, int32_t *block_expert,
                            int32_t *num_post_padded, int capacity, hipStream_t s)
{
    moe_align_kernel<<<1, kAlignThreads, 0, s>>>(topk_ids, num_valid, E, block_m, expert_map, sorted_ids,
                                                  expert_offsets, block_expert, num_post_padded, capacity);
    return hipGetLastError();
}

namespace {
// fq / fs non-null: the fused gate/up form (FUSE); returns hipErrorNotSupported
// when the shape does not allow it, before launching anything
hipError_t moe_gemm_common(const Lut3Layout &L, const uint8_t *packed, int E_global, const uint8_t *aq,
                           const uint8_t *as, int a_rows, int a_row_div, const int32_t *sorted_ids,
                           const int32_t *expert_offsets, const int32_t *block_expert, int num_valid, int block_m,
                           uint16_t *out, uint8_t *fq, uint8_t *fs, hipStream_t s)
{
    const bool fuse = fq != nullptr;
    MoeArgs p;
    p.idx = packed + L.idx_off;
    p.cb = packed + L.cb_off;
    p.ex = packed + L.ex_off;
    p.aq = aq;
    p.as = as;
    p.sorted_ids = sorted_ids;
    p.expert_offsets = expert_offsets;
    p.block_expert = block_expert;
    p.out = out;
    p.fq = fq;
    p.fs = fs;
    p.E = (int)L.E;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.strips = (int)L.strips;
    p.ksteps = (int)L.ksteps;
    p.a_row_div = a_row_div;
    p.num_valid = num_valid;
    p.block_m = block_m;
    p.n_tiles = (int)((L.strips + kMoeWaves * kStripsPerWave - 1) / (kMoeWaves * kStripsPerWave));
    p.a_rows = a_rows;
    const unsigned blocks = (unsigned)((int64_t)E_global * p.n_tiles);
    if (blocks == 0) return hipSuccess;
    // Activation rows in LDS when a pass of 32 rows (or 16) fits in 80 KB;
    // otherwise the kernel that reads activations straight from memory.
    constexpr int kMaxLds = 80 * 1024;
    constexpr int kMaxGroupLds = 150 * 1024;
    auto fits = [&](int m) { return moe_lds_bytes(m, p.K) <= kMaxLds && m * 16 * (p.K / 32) <= kMoeScaleBytesMax; };
    const int mb = fits(2) ? 2 : (fits(1) ? 1 : 0);
    if (fuse && (mb == 0 || L.N % 256 != 0)) return hipErrorNotSupported;
    if (mb > 0) {
        // workgroups of 8 waves over groups of 256-column tiles: about 256
        // workgroups in all, so each expert's activations are staged once per
        // group instead of once per tile
        MoeGroupArgs ga;
        ga.m = p;
        ga.gtiles = (int)((L.strips + kGTileStrips - 1) / kGTileStrips);   // FUSE: 128 activation columns each
        const int64_t want = (E_global * (int64_t)ga.gtiles + 255) / 256;     // tiles per workgroup for ~256
        ga.tiles_per_group = (int)std::max<int64_t>(1, std::min<int64_t>(want, ga.gtiles));
        // the group's output block has to fit the LDS as well
        while (ga.tiles_per_group > 1 && moe_lds_layout(mb, p.K, ga.tiles_per_group).bytes > kMaxGroupLds)
            --ga.tiles_per_group;
        ga.n_groups = (ga.gtiles + ga.tiles_per_group - 1) / ga.tiles_per_group;
        const unsigned gblocks = (unsigned)((int64_t)E_global * ga.n_groups);
        const int lds = moe_lds_layout(mb, p.K, ga.tiles_per_group).bytes;
        auto k = fuse ? (mb == 2 ? moe_lut3_gemm_lds_kernel<2, 5, true> : moe_lut3_gemm_lds_kernel<1, 5, true>)
                      : (mb == 2 ? moe_lut3_gemm_lds_kernel<2, 5, false> : moe_lut3_gemm_lds_kernel<1, 5, false>);
        hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        k<<<gblocks, kGWaves * 64, lds, s>>>(p.expert_offsets, p.block_expert, p.sorted_ids, ga.n_groups,
                                             ga.tiles_per_group, ga.gtiles, p.block_m, p.num_valid, p.strips,
                                             p.ksteps, ga);
    } else {
        moe_lut3_gemm_kernel<<<blocks, kMoeWaves * 64, 0, s>>>(p);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_moe_gemm(const Lut3Layout &L, const uint8_t *packed, int E_global, const uint8_t *aq,
                           const uint8_t *as, int a_rows, int a_row_div, const int32_t *sorted_ids,
                           const int32_t *expert_offsets, const int32_t *block_expert, int num_valid, int block_m,
                           uint16_t *out, hipStream_t s)
{
    return moe_gemm_common(L, packed, E_global, aq, as, a_rows, a_row_div, sorted_ids, expert_offsets, block_expert,
                           num_valid, block_m, out, nullptr, nullptr, s);
}

hipError_t launch_moe_gemm_silu(const Lut3Layout &L, const uint8_t *packed, int E_global, const uint8_t *aq,
                                const uint8_t *as, int a_rows, int a_row_div, const int32_t *sorted_ids,
                                const int32_t *expert_offsets, const int32_t *block_expert, int num_valid,
                                int block_m, uint8_t *act_q, uint8_t *act_s, hipStream_t s)
{
    return moe_gemm_common(L, packed, E_global, aq, as, a_rows, a_row_div, sorted_ids, expert_offsets, block_expert,
                           num_valid, block_m, nullptr, act_q, act_s, s);
}


}  // namespace lowbit
