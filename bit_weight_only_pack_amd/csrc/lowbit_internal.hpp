// lowbit_internal.hpp -- types, packed layouts and launcher declarations
// shared by the HIP sources of liblowbit.so (never by the CPU oracle).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lowbit.h"

namespace lowbit {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Raw buffer access: an SGPR descriptor plus a 32-bit byte offset per lane.
// Reads at an offset past `bytes` return zeros without touching memory,
// which lets kernels issue loads unconditionally.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kBufferOob = 0x80000000u;   // an offset past any descriptor used here
// Cache policy of loads that stream data read once (packed weights): the
// non-temporal hint, so streaming lines do not displace reused ones.
constexpr int kStreamLoad = 2;

constexpr int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
constexpr int64_t align256(int64_t v) { return round_up(v, 256); }

// ---------------------------------------------------------------------------
// Packed INT4 layout (one matrix of N outputs x K inputs).
//
// The weight is cut into tiles of 16 output rows x 128 K (1 KiB of codes).
// Tile (s, t) covers rows 16s..16s+15 and K 128t..128t+127; tiles are stored
// strip-major (all K tiles of strip s, then strip s+1) so that a wavefront
// walking one strip along K reads contiguous memory.  Inside a tile the
// 64 lanes of a wavefront each own 16 bytes, in the operand order of
// v_mfma_f32_16x16x32_f16 with the weight as the B matrix:
//   lane l, dword i (i = 0..3)  <->  row 16s + (l % 16),
//                                     K = 128t + 32i + 8(l / 16) + j, j = 0..7
// so one coalesced 16-byte load per lane feeds four MFMAs.  Inside a dword the
// eight 4-bit codes sit in nibble slots ordered k+0, k+2, k+4, k+6, k+1, k+3,
// k+5, k+7: masking with 0x000F000F (or 0x00F000F0, and the same after a
// shift by 8) puts the codes of k+2p and k+2p+1 into the two fp16 halves of a
// register, which is the unpack the kernels use.
//
// Scales follow in tile order: for tile (s, t), 16 rows x (128/G) fp16, row
// major, so a lane reads its row's (128/G) scales in one load.  Zero points
// (asymmetric only) use the same order as int8.  Rows past N and K past the
// end are padding: codes 0, scales 0, zeros 0.  Every section starts at a
// 256-byte boundary.
// ---------------------------------------------------------------------------
//
// Uniform b-bit codes (b = 1..8, formats LOWBIT_UINT) use the same tiles,
// with 256 * b bytes per tile.  A lane's 32 codes (MFMA block i = 0..3, K
// offset j = 0..7) are split into bit planes, b = 4 n4 + 2 n2 + n1 (n4 <= 2,
// n2, n1 <= 1), and each plane is its own region of the tile, lane-major, so
// every load of a wave is one dense span:
//   4-bit plane p (code bits 4p..4p+3), 1 KiB at 1024 p: 4 dwords per lane,
//     dword i in the INT4 nibble slots above, so (w >> 4q) & 0x000F000F holds
//     K offsets 2q, 2q+1;
//   2-bit plane (code bits 4 n4, +1), 512 B after the 4-bit planes: 2 dwords
//     per lane, dword i / 2 holds the pair q of block i at bits
//     2 (4 (i & 1) + q) and 16 + 2 (4 (i & 1) + q);
//   1-bit plane (code bit 4 n4 + 2 n2), 256 B last: 1 dword per lane, the
//     pair q of block i at bits 4 i + q and 16 + 4 i + q.
// A shift and a mask therefore give two codes in the two 16-bit halves, ready
// to be or-ed into fp16 1024.0.  At b = 4 the layout is the INT4 one.
//
// b = 3 instead keeps a lane's three dwords together (12 bytes, one load)
// and nibble-aligns them: dword d (0..2) holds the codes of MFMA block d in
// bits 0..2 of the INT4 nibble slots, so they unpack exactly as INT4 codes
// with a 3-bit mask; block 3's codes sit in the spare bit 3 of every nibble,
// code bit c in dword c, and three shift-and-merge steps gather them into a
// fourth dword of the same form.
//
// b = 8 keeps the two 1 KiB regions of the 4-bit planes (so each load of a
// wave is one dense KiB) but stores a code per byte: the lane's dword 2i + h
// (region (2i + h) / 4) holds block i's K offsets 4h, 4h + 2, 4h + 1, 4h + 3
// in bytes 0..3, so masking it (and its 8-bit shift) with 0x00FF00FF gives two
// codes in the two 16-bit halves, ready for fp16 1024.0.
// dword index inside a tile of plane dword k (0..b-1) of lane l
__host__ __device__ inline int wb_word(int bits, int lane, int k)
{
    if (bits == 3) return lane * 3 + k;
    const int n4 = bits / 4, n2 = (bits % 4) >= 2 ? 1 : 0;
    if (k < 4 * n4) return (k / 4) * 256 + lane * 4 + (k % 4);
    k -= 4 * n4;
    if (k < 2 * n2) return n4 * 256 + lane * 2 + k;
    return n4 * 256 + n2 * 128 + lane;
}
// ---------------------------------------------------------------------------
struct W4Layout {
    int64_t N, K;
    int G;
    bool asym;
    int bits;            // code width: 4 for the INT4 formats, 1..8 for LOWBIT_UINT
    int64_t strips;      // ceil(N / 16)
    int64_t ktiles;      // ceil(K / 128)
    int64_t codes_off, scales_off, zeros_off, bytes;
};

inline W4Layout wb_layout(int64_t N, int64_t K, int G, int bits, bool asym)
{
    W4Layout L;
    L.N = N; L.K = K; L.G = G; L.asym = asym; L.bits = bits;
    L.strips = (N + 15) / 16;
    L.ktiles = (K + 127) / 128;
    const int64_t tiles = L.strips * L.ktiles;
    const int64_t gpt = 128 / G;
    L.codes_off = 0;
    L.scales_off = align256(tiles * 256 * bits);
    L.zeros_off = align256(L.scales_off + tiles * 16 * gpt * 2);
    L.bytes = align256(L.zeros_off + (asym ? tiles * 16 * gpt : 0));
    return L;
}
inline W4Layout w4_layout(int64_t N, int64_t K, int G, bool asym) { return wb_layout(N, K, G, 4, asym); }

// slot of the code of K offset j (0..7) inside a packed dword
__host__ __device__ constexpr int w4_slot(int j) { return (j & 1) * 4 + (j >> 1); }

// LOWBIT_UINT(bits, asym) = 16 + 2 * bits + asym
constexpr int kUintBase = 16;
inline bool is_uint_fmt(int fmt) { return fmt >= kUintBase + 2 && fmt <= kUintBase + 17; }
inline int uint_bits(int fmt) { return (fmt - kUintBase) / 2; }
inline bool uint_asym(int fmt) { return ((fmt - kUintBase) & 1) != 0; }

// ---------------------------------------------------------------------------
// Launchers (enqueue only; argument validation happens in api.hip).
// ---------------------------------------------------------------------------
hipError_t launch_w4_pack(const W4Layout &L, const uint8_t *codes, const uint16_t *scales,
                          const int8_t *zeros, uint8_t *packed, hipStream_t s);
hipError_t launch_w4_unpack(const W4Layout &L, const uint8_t *packed, uint8_t *codes,
                            uint16_t *scales, int8_t *zeros, hipStream_t s);
hipError_t launch_w4_dequant(const W4Layout &L, const uint8_t *packed, float *w, hipStream_t s);
// b-bit codes (canonical: one code per byte, [N][K])
hipError_t launch_wb_pack(const W4Layout &L, const uint8_t *codes, const uint16_t *scales, const int8_t *zeros,
                          uint8_t *packed, hipStream_t s);
hipError_t launch_wb_unpack(const W4Layout &L, const uint8_t *packed, uint8_t *codes, uint16_t *scales,
                            int8_t *zeros, hipStream_t s);
hipError_t launch_wb_dequant(const W4Layout &L, const uint8_t *packed, float *w, hipStream_t s);
hipError_t launch_gemv_wb_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                const _Float16 *const *x, _Float16 *const *y, hipStream_t s);
size_t gemv_wb_lds(int M, int64_t kt_max, bool asym);    // 0: no kernel for this M and K

// A batch of independent GEMVs with the same format, M and group size, run by
// one launch (one workgroup per 16-row strip; blockIdx.y picks the problem).
constexpr int kMaxGemvBatch = 8;
struct GemvProblem {
    const uint8_t *codes, *scales, *zeros;
    const _Float16 *x;
    _Float16 *y;
    int N, K, ktiles, strips;
    int tw;                              // K tiles per wave of the streaming kernel
    int pad;
};
struct GemvBatch {
    GemvProblem p[kMaxGemvBatch];
    int first[kMaxGemvBatch];            // first workgroup of each problem when laid end to end
    int count, M, ct;
    int W;                               // waves per workgroup
};
hipError_t launch_gemv_w4_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                const _Float16 *const *x, _Float16 *const *y, hipStream_t s);

// W4A8 GEMV (gemv_w4a8.hip): dynamic per-token INT8 activations.
// gemv_w4a8_plan: 0 = the launch quantizes activations itself, 1 = needs a
// workspace of *ws_bytes for the prepared activation blocks, -1 = no kernel
// for this batch.
int gemv_w4a8_plan(const W4Layout *L, int count, int M, size_t *ws_bytes);
hipError_t launch_gemv_w4a8_batch(const W4Layout *L, int count, int M, const uint8_t *const *packed,
                                  const _Float16 *const *x, _Float16 *const *y, void *ws, hipStream_t s);
hipError_t launch_quant_act_i8(int M, int K, const _Float16 *x, int8_t *xq, float *sx, hipStream_t s);
// The W4A8 GEMV's static scratch (gemv_w4a8.hip): its size, and its device
// address on the current device (looked up once per device)
constexpr size_t kW4a8ScratchBytes = (size_t)512 << 10;
hipError_t w4a8_scratch(void **ptr);

// A chain of dependent GEMV stages run by one persistent launch
// (gemv_chain.hip).  Device buffer: counters, then the ChainProb table, then
// the per-stage arrival counts.
constexpr int kChainSlots = 32;          // completion counters per stage
constexpr int kChainSlotStride = 32;     // words between them (one per 128-byte line)
constexpr int kChainCtrHeader = 64;      // words before the first stage's counters
struct ChainProb {
    const uint8_t *codes, *scales, *zeros;
    const _Float16 *x;
    _Float16 *y;
    int N, K, ktiles, rounds;            // rounds = ceil(ktiles / 32)
    int item_begin, item_end, stage, pad;
};
struct ChainArgs {
    const ChainProb *probs;
    const int *arrivals;                 // workgroups that signal each stage
    uint32_t *ctr;
    int nprob, M, xrow;                  // xrow: LDS row stride of x in halfs
    uint32_t spin_limit;
};
struct ChainLayout {
    int64_t ctr_words, probs_off, arrivals_off, bytes;
};
inline ChainLayout chain_layout(int count, int stages)
{
    ChainLayout L;
    L.ctr_words = kChainCtrHeader + (int64_t)stages * kChainSlots * kChainSlotStride;
    L.probs_off = align256(L.ctr_words * 4);
    L.arrivals_off = align256(L.probs_off + (int64_t)count * (int64_t)sizeof(ChainProb));
    L.bytes = align256(L.arrivals_off + (int64_t)stages * 4);
    return L;
}
constexpr int kChainRoundTiles = 32;
size_t gemv_chain_lds_bytes(int M, int xrow);
int gemv_chain_occupancy(int G, bool asym, int M, size_t lds);
hipError_t launch_gemv_chain(int G, bool asym, const ChainArgs &a, int grid, hipStream_t s);

size_t gemv_w4_workspace(int M, int64_t N, int64_t K, int G);
hipError_t launch_gemv_w4(const W4Layout &L, int M, const uint8_t *packed, const _Float16 *x,
                          _Float16 *y, void *ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------------------
// Packed 3-bit LUT-codebook layout (E experts of N outputs x K inputs).
//
// Units of 16 output columns x 128 K (2048 weights), ordered expert, strip,
// K step.  Three sections, each 256-byte aligned:
//   idx : 768 bytes per unit, 12 per lane in the operand order of
//         v_mfma_scale_f32_16x16x128_f8f6f4 (lane l: column l % 16, K chunk
//         32 * (l / 16) .. +32); bit layout in moe_lut3.hip (lut_put)
//   cb  : 32 bytes per unit, the four 8-entry E4M3 codebooks of the unit's
//         tiles, ordered (column half, K half)
//   ex  : 4 bytes per unit, the four UE8M0 tile exponents in the same order
// Padding columns / K: index 0, codebook zeros, exponent 127.
// ---------------------------------------------------------------------------
struct Lut3Layout {
    int64_t E, N, K;
    int64_t strips, ksteps;
    int64_t idx_off, cb_off, ex_off, bytes;
};
Lut3Layout lut3_layout(int64_t E, int64_t N, int64_t K);
hipError_t launch_lut3_pack(const Lut3Layout &L, const uint8_t *idx, const uint8_t *cb, const uint8_t *ex,
                            uint8_t *packed, hipStream_t s);
hipError_t launch_lut3_unpack(const Lut3Layout &L, const uint8_t *packed, uint8_t *idx, uint8_t *cb, uint8_t *ex,
                              hipStream_t s);
hipError_t launch_moe_align(const int32_t *topk_ids, int num_valid, int E, int block_m, const int32_t *expert_map,
                            int32_t *sorted_ids, int32_t *expert_offsets, int32_t *block_expert,
                            int32_t *num_post_padded, int capacity, hipStream_t s);
hipError_t launch_moe_gemm(const Lut3Layout &L, const uint8_t *packed, int E_global, const uint8_t *aq,
                           const uint8_t *as, int a_rows, int a_row_div, const int32_t *sorted_ids,
                           const int32_t *expert_offsets, const int32_t *block_expert, int num_valid, int block_m,
                           uint16_t *out, hipStream_t s);
// the gate/up GEMM (N = 2I) with SiLU(gate) * up as MXFP8 for its output
// (act_q [num_valid][I] E4M3, act_s [num_valid][I/32] UE8M0) instead of the bf16
// rows; hipErrorNotSupported (nothing launched) when the shape does not allow it
hipError_t launch_moe_gemm_silu(const Lut3Layout &L, const uint8_t *packed, int E_global, const uint8_t *aq,
                                const uint8_t *as, int a_rows, int a_row_div, const int32_t *sorted_ids,
                                const int32_t *expert_offsets, const int32_t *block_expert, int num_valid,
                                int block_m, uint8_t *act_q, uint8_t *act_s, hipStream_t s);

// The MoE layer around the grouped GEMMs (moe_layer.hip)
hipError_t launch_mxfp8_rows(const uint16_t *x, int64_t R, int K, bool silu, uint8_t *q, uint8_t *scale,
                             hipStream_t s);
// the MoE layer's front end in one launch: routing (as launch_moe_align) and
// the MXFP8 quantization of the hidden states (as launch_mxfp8_rows)
hipError_t launch_moe_prep(const uint16_t *x, int T, int H, uint8_t *xq, uint8_t *xs, const int32_t *topk_ids,
                           int num_valid, int E, int block_m, const int32_t *expert_map, int32_t *sorted_ids,
                           int32_t *expert_offsets, int32_t *block_expert, int32_t *num_post_padded, int capacity,
                           hipStream_t s);
hipError_t launch_moe_combine(const uint16_t *out, const float *w, int T, int top_k, int H, uint16_t *y,
                              hipStream_t s);
struct MoeLayerWs {
    int64_t xq, xs, sorted, offsets, blocks, npp, gate_up, aq, as, down, bytes, capacity;
};
inline MoeLayerWs moe_layer_ws(int T, int top_k, int E, int H, int I, int block_m)
{
    MoeLayerWs w;
    const int64_t slots = (int64_t)T * top_k;
    w.capacity = slots + (int64_t)E * (block_m - 1);
    w.xq = 0;
    w.xs = align256(w.xq + (int64_t)T * H);
    w.sorted = align256(w.xs + (int64_t)T * (H / 32));
    w.offsets = align256(w.sorted + w.capacity * 4);
    w.blocks = align256(w.offsets + (int64_t)(E + 1) * 4);
    w.npp = align256(w.blocks + (w.capacity / block_m + 1) * 4);
    w.gate_up = align256(w.npp + 4);
    w.aq = align256(w.gate_up + slots * 2 * I * 2);
    w.as = align256(w.aq + slots * I);
    w.down = align256(w.as + slots * (I / 32));
    w.bytes = align256(w.down + slots * H * 2);
    return w;
}

size_t gemm_w4_workspace(int M, int64_t N, int64_t K, int G);
hipError_t launch_gemm_w4(const W4Layout &L, int M, const uint8_t *packed, const void *a, int a_bf16, void *c,
                          int c_bf16, void *ws, size_t ws_bytes, hipStream_t s);

}  // namespace lowbit
