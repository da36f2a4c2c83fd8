// moe_layer.hip -- the MoE layer around the two LUT3 grouped GEMMs: MXFP8
// quantization of bf16 rows (the hidden states before the gate/up GEMM, and
// SiLU(gate) * up before the down GEMM) and the router-weighted combine of the
// routed experts' outputs ("vLLM PR #62759 analysis", section "Emulation path":
// activations are quantized to MXFP8 before each expert GEMM; OCP MX: one
// UE8M0 scale per 32 consecutive elements, elements in E4M3).
//
// Definitions (the page leaves these steps open; the same readings define the
// CPU reference):
//   * gate/up GEMM output row [2I]: columns 0..I-1 gate, I..2I-1 up; SiLU(gate)
//     * up and the MXFP8 encoding as defined in mxfp8.hpp.
//   * combine: y[t][h] = RNE_bf16( sum_j w[t][j] * out[t*top_k + j][h] ),
//     fp32, j ascending.
//
// MI355X design: both kernels are HBM-bound elementwise passes (bytes read
// once, written once, 16-byte accesses per lane).  A 32-block is held by the
// four lanes of a quad, so its maximum is two DPP steps; the E4M3 rounding is
// done in integer arithmetic on the binary32 bits, exactly as defined.
#include "lowbit_internal.hpp"
#include "moe_align.hpp"
#include "mxfp8.hpp"

namespace lowbit {

namespace {

using namespace mx;

// Lane t of R x (K / 8) quantizes outputs 8c .. 8c + 7 of row r.  SILU: the
// input row is [2K] (gate | up), the output row K = I.
template <bool SILU>
__device__ __forceinline__ void mxfp8_row_lane(const uint16_t *x, int64_t R, int K, uint8_t *q, uint8_t *scale,
                                               int64_t t)
{
    const int cpr = K / 8;                           // lanes per row (a multiple of 4: K % 32 == 0)
    if (t >= R * cpr) return;                        // whole quads (R * cpr is a multiple of 4)
    const int64_t r = t / cpr;
    const int c = (int)(t - r * cpr);
    float v[8];
    if constexpr (SILU) {
        const us8 g = *reinterpret_cast<const us8 *>(x + r * 2 * K + c * 8);
        const us8 u = *reinterpret_cast<const us8 *>(x + r * 2 * K + K + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = silu_f32(bf16_to_f32(g[i])) * bf16_to_f32(u[i]);
            v[i] = bf16_to_f32(f32_to_bf16(a));
        }
    } else {
        const us8 g = *reinterpret_cast<const us8 *>(x + r * K + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(g[i]);
    }
    mx_block_put(v, q + r * K + c * 8, scale + r * (K / 32) + c / 4, (c & 3) == 0);
}

template <bool SILU>
__global__ __launch_bounds__(256) void mxfp8_rows_kernel(const uint16_t *x, int64_t R, int K, uint8_t *q,
                                                         uint8_t *scale)
{
    mxfp8_row_lane<SILU>(x, R, K, q, scale, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// The layer's front end in one launch (the two jobs are independent): block 0
// buckets the routed slots by expert, blocks 1.. quantize the hidden states to
// MXFP8, 1024 lanes each.
__global__ __launch_bounds__(kAlignThreads)
void moe_prep_kernel(const uint16_t *x, int64_t T, int H, uint8_t *xq, uint8_t *xs, const int32_t *topk_ids,
                     int num_valid, int E, int block_m, const int32_t *expert_map, int32_t *sorted_ids,
                     int32_t *expert_offsets, int32_t *block_expert, int32_t *num_post_padded, int capacity)
{
    if (blockIdx.x == 0)
        moe_align_block(topk_ids, num_valid, E, block_m, expert_map, sorted_ids, expert_offsets, block_expert,
                        num_post_padded, capacity);
    else
        mxfp8_row_lane<false>(x, T, H, xq, xs, (int64_t)(blockIdx.x - 1) * kAlignThreads + threadIdx.x);
}

// y[t][h .. h+8) = RNE_bf16(sum_j w[t][j] * out[t*top_k + j][h .. h+8)), fp32,
// j ascending
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *out, const float *w, int T, int top_k,
                                                          int H, uint16_t *y)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int cpr = H / 8;
    if (i >= (int64_t)T * cpr) return;
    const int64_t t = i / cpr;
    const int c = (int)(i - t * cpr);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < top_k; ++j) {
        const float wj = w[t * top_k + j];
        const us8 o = *reinterpret_cast<const us8 *>(out + (t * top_k + j) * H + c * 8);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(wj, bf16_to_f32(o[k]), acc[k]);
    }
    us8 r;
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = f32_to_bf16(acc[k]);
    *reinterpret_cast<us8 *>(y + t * H + c * 8) = r;
}

}  // namespace

hipError_t launch_mxfp8_rows(const uint16_t *x, int64_t R, int K, bool silu, uint8_t *q, uint8_t *scale,
                             hipStream_t s)
{
    const int64_t lanes = R * (K / 8);
    if (lanes == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((lanes + 255) / 256);
    if (silu)
        mxfp8_rows_kernel<true><<<blocks, 256, 0, s>>>(x, R, K, q, scale);
    else
        mxfp8_rows_kernel<false><<<blocks, 256, 0, s>>>(x, R, K, q, scale);
    return hipGetLastError();
}

hipError_t launch_moe_prep(const uint16_t *x, int T, int H, uint8_t *xq, uint8_t *xs, const int32_t *topk_ids,
                           int num_valid, int E, int block_m, const int32_t *expert_map, int32_t *sorted_ids,
                           int32_t *expert_offsets, int32_t *block_expert, int32_t *num_post_padded, int capacity,
                           hipStream_t s)
{
    const int64_t lanes = (int64_t)T * (H / 8);
    const unsigned blocks = 1 + (unsigned)((lanes + kAlignThreads - 1) / kAlignThreads);
    moe_prep_kernel<<<blocks, kAlignThreads, 0, s>>>(x, T, H, xq, xs, topk_ids, num_valid, E, block_m, expert_map,
                                                      sorted_ids, expert_offsets, block_expert, num_post_padded,
                                                      capacity);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t *out, const float *w, int T, int top_k, int H, uint16_t *y,
                              hipStream_t s)
{
    const int64_t lanes = (int64_t)T * (H / 8);
    if (lanes == 0) return hipSuccess;
    moe_combine_kernel<<<(unsigned)((lanes + 255) / 256), 256, 0, s>>>(out, w, T, top_k, H, y);
    return hipGetLastError();
}

}  // namespace lowbit
