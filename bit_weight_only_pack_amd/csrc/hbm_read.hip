// hbm_read.hip -- a read-only streaming kernel: the practical ceiling of HBM
// reads on this chip, measured beside the kernels' rooflines ("Low Bit Metal
// Kernels", practice sequence: measure the memory-bandwidth utilisation of a
// bandwidth-bound kernel).
//
// 1024 workgroups of 4 waves; each wave reads one contiguous chunk of the
// buffer (its 4096th part, in whole KiB), 16 KiB at a time with 16-byte
// non-temporal loads (consecutive lanes, consecutive blocks), all 16 loads in
// flight before the first is used.  Each workgroup stores the XOR of the
// 32-bit words it read to its own sink word: no load is dead, the result can
// be checked, and no two workgroups touch one address.  (Measured on MI355X
// over 2 GiB: 6.9 TB/s; a grid-stride sweep of the same loads 5.9-6.1 TB/s.)
#include "lowbit_internal.hpp"

namespace lowbit {

namespace {

constexpr int kReadWaves = 4;
constexpr int kReadUnroll = 16;                   // KiB per wave in flight

__global__ __launch_bounds__(kReadWaves * 64) void hbm_read_kernel(const u4 *__restrict__ p, int64_t n16,
                                                                  int64_t per_wave, uint32_t *sink)
{
    __shared__ uint32_t part[kReadWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t b0 = ((int64_t)blockIdx.x * kReadWaves + wave) * per_wave;
    const int64_t b1 = b0 + per_wave < n16 ? b0 + per_wave : n16;
    uint32_t acc = 0u;
    for (int64_t b = b0; b < b1; b += kReadUnroll * 64) {
        u4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = b + u * 64 + lane;
            v[u] = i < b1 ? __builtin_nontemporal_load(p + i) : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    constexpr int64_t waves = (int64_t)LOWBIT_HBM_READ_SINK_WORDS * kReadWaves;
    const int64_t per_wave = ((n16 + waves - 1) / waves + 63) / 64 * 64;   // whole KiB per wave
    hbm_read_kernel<<<LOWBIT_HBM_READ_SINK_WORDS, kReadWaves * 64, 0, s>>>(static_cast<const u4 *>(buf), n16,
                                                                          per_wave, sink);
    return hipGetLastError();
}

}  // namespace lowbit
