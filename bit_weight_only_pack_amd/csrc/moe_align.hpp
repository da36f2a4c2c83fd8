// moe_align.hpp -- routing of the MoE layer: bucket the routed slots by
// expert ("vLLM PR #62759 analysis", section "A gather": the expert GEMM
// reads the rows routed to its expert through a sorted id list), shared by
// the standalone align kernel and the layer's front-end kernel.
#pragma once
#include "lowbit_internal.hpp"

namespace lowbit {

// ---------------------------------------------------------------- align
// Bucket the routed slots by expert (ascending expert, ascending slot id),
// pad each expert to a multiple of block_m with the sentinel num_valid, and
// record the expert of every block.  One workgroup of 1024 threads:
//   1. per-expert counts (LDS histogram) and the exclusive scan of the padded
//      counts (wave prefix sums, then a prefix over the wave totals);
//   2. placement, a chunk of slots at a time: every slot sets its bit in its
//      expert's bitmask of the chunk; a slot's rank among its expert's slots
//      is the number of set bits below its own plus that expert's count from
//      earlier chunks -- a stable order with no sequential pass;
//   3. block_expert.
// Every output position is written exactly once (slot ids by the placement,
// the sentinel in each expert's padding and past the padded length, -1 for
// the blocks past it), so no store has to complete before another one.
constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;
constexpr int kAlignMaskWords = 8192;             // LDS words for the chunk bitmasks (32 KB)
constexpr int kAlignIdCache = 4096;               // slot ids kept in LDS (as int16) between the passes

// the body of the align kernel, run by one whole 1024-thread workgroup
__device__ __forceinline__ void moe_align_block(const int32_t *__restrict__ topk_ids, int num_valid, int E,
                                                int block_m, const int32_t *__restrict__ expert_map,
                                                int32_t *__restrict__ sorted_ids,
                                                int32_t *__restrict__ expert_offsets,
                                                int32_t *__restrict__ block_expert,
                                                int32_t *__restrict__ num_post_padded, int capacity)
{
    __shared__ int counts[kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int running[kMaxExperts];
    __shared__ __attribute__((aligned(16))) int wave_sum[kAlignWaves];
    __shared__ uint32_t mask[kAlignMaskWords];
    __shared__ int16_t ids[kAlignIdCache];           // slot -> expert (or -1) for the first slots
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // 1. counts and padded offsets (thread e owns expert e, E <= 1024)
    counts[tid] = 0;
    running[tid] = 0;
    __syncthreads();
    for (int i = tid; i < num_valid; i += kAlignThreads) {
        int e = topk_ids[i];
        if (e < 0 || e >= E) e = -1;
        if (i < kAlignIdCache) ids[i] = (int16_t)e;
        if (e >= 0) atomicAdd(&counts[e], 1);
    }
    __syncthreads();
    const int padded = tid < E ? (counts[tid] + block_m - 1) / block_m * block_m : 0;
    int incl = padded;                                // inclusive prefix inside the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0;                                   // totals of the earlier waves
#pragma unroll
    for (int q = 0; q < kAlignWaves / 4; ++q) {
        const int4 v = reinterpret_cast<const int4 *>(wave_sum)[q];
        before += (4 * q + 0 < wave ? v.x : 0) + (4 * q + 1 < wave ? v.y : 0) + (4 * q + 2 < wave ? v.z : 0) +
                  (4 * q + 3 < wave ? v.w : 0);
    }
    const int excl = before + incl - padded;
    if (tid < E) offs[tid] = excl;
    if (tid == E - 1) offs[E] = excl + padded;
    __syncthreads();
    const int total = offs[E];
    if (tid < E) expert_offsets[tid] = offs[tid];
    if (tid == 0) {
        expert_offsets[E] = total;                    // (E may equal the thread count)
        num_post_padded[0] = total;
    }
    // the sentinel in each expert's padding and past the padded length; -1
    // for the blocks past it
    if (tid < E)
        for (int i = offs[tid] + counts[tid]; i < offs[tid + 1]; ++i) sorted_ids[i] = num_valid;
    for (int i = total + tid; i < capacity; i += kAlignThreads) sorted_ids[i] = num_valid;
    for (int b = total / block_m + tid; b < capacity / block_m; b += kAlignThreads) block_expert[b] = -1;

    // 2. stable placement, chunk by chunk: a chunk's bitmask holds
    //    chunk / 32 words per expert, rows one word longer than that so the
    //    rows of different experts start in different LDS banks
    const int words = max(1, min(32, kAlignMaskWords / E - 1));   // words per expert per chunk
    const int stride = words + 1;
    const int chunk = words * 32;
    for (int base = 0; base < num_valid; base += chunk) {
        for (int i = tid; i < E * stride; i += kAlignThreads) mask[i] = 0;
        __syncthreads();
        int e = -1, local = 0;
        if (tid < chunk && base + tid < num_valid) {
            const int i = base + tid;
            e = i < kAlignIdCache ? (int)ids[i] : topk_ids[i];
            if (e >= 0 && e < E) {
                local = tid;
                atomicOr(&mask[e * stride + (local >> 5)], 1u << (local & 31));
            } else {
                e = -1;
            }
        }
        __syncthreads();
        if (e >= 0) {
            const uint32_t *m = mask + e * stride;
            int rank = __builtin_popcount(m[local >> 5] & ((1u << (local & 31)) - 1u));
            for (int w = 0; w < (local >> 5); ++w) rank += __builtin_popcount(m[w]);
            sorted_ids[offs[e] + running[e] + rank] = base + local;
        }
        __syncthreads();
        if (tid < E) {
            int c = 0;
            for (int w = 0; w < words; ++w) c += __builtin_popcount(mask[tid * stride + w]);
            running[tid] += c;
        }
        __syncthreads();
    }

    // 3. expert of every block below the padded length
    if (tid < E) {
        const int local = expert_map ? expert_map[tid] : tid;
        for (int b = offs[tid] / block_m; b < offs[tid + 1] / block_m; ++b) block_expert[b] = local;
    }
}

}  // namespace lowbit
