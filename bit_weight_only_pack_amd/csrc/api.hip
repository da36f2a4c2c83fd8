// api.hip -- the C ABI of liblowbit.so: host-side argument validation and
// dispatch to the launchers.  Nothing here allocates device memory; every
// error is detected before the first enqueue.
#include "lowbit_internal.hpp"

#include <vector>

namespace lowbit {
// hbm_read.hip: read-only streaming of `bytes` (a multiple of 16), *sink ^= XOR of all 32-bit words
hipError_t launch_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s);
}  // namespace lowbit

using namespace lowbit;

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return LOWBIT_OK;
    g_last_hip_error = (int)e;
    return LOWBIT_E_HIP;
}

bool is_w4(int fmt) { return fmt == LOWBIT_W4_SYM || fmt == LOWBIT_W4_ASYM; }

bool w4_group_ok(int G) { return G == 32 || G == 64 || G == 128; }

// Shape rules shared by every W4 entry point.
int check_w4_shape(int fmt, int N, int K, int G)
{
    if (!is_w4(fmt)) return LOWBIT_E_UNSUPPORTED;
    if (N < 0 || K < 0) return LOWBIT_E_INVALID_ARG;
    if (G <= 0 || K % G != 0) return LOWBIT_E_INVALID_ARG;
    if (!w4_group_ok(G)) return LOWBIT_E_UNSUPPORTED;
    // indices inside the kernels are 32-bit for rows and K offsets
    if ((int64_t)N > (1 << 30) || (int64_t)K > (1 << 30)) return LOWBIT_E_UNSUPPORTED;
    return LOWBIT_OK;
}

// dense group-wise formats: INT4 (nibble-packed canonical codes) and uniform
// b-bit codes (one code per byte)
bool is_dense(int fmt) { return is_w4(fmt) || is_uint_fmt(fmt); }

int check_dense_shape(int fmt, int N, int K, int G)
{
    if (is_uint_fmt(fmt)) {
        const int bits = uint_bits(fmt);
        if (bits < 1 || bits > 8) return LOWBIT_E_UNSUPPORTED;
        return check_w4_shape(uint_asym(fmt) ? LOWBIT_W4_ASYM : LOWBIT_W4_SYM, N, K, G);
    }
    return check_w4_shape(fmt, N, K, G);
}

bool dense_asym(int fmt) { return is_uint_fmt(fmt) ? uint_asym(fmt) : fmt == LOWBIT_W4_ASYM; }

W4Layout dense_layout(int fmt, int64_t N, int64_t K, int G)
{
    return is_uint_fmt(fmt) ? wb_layout(N, K, G, uint_bits(fmt), uint_asym(fmt)) : w4_layout(N, K, G, fmt == LOWBIT_W4_ASYM);
}

// canonical code bytes of one matrix: two codes per byte for INT4, one otherwise
int64_t dense_code_bytes(int fmt, int64_t N, int64_t K) { return is_uint_fmt(fmt) ? N * K : N * (K / 2); }

// The GEMV and GEMM kernels address their operands through buffer
// descriptors with 32-bit byte offsets, and an offset of 2^31 stands for "past
// the end" (it reads zeros).  Every region one descriptor spans must therefore
// stay below 2^31 bytes: the activation rows, one 16-row strip of codes (the
// GEMV's descriptors are per strip), and for the GEMM the whole packed blob.
constexpr int64_t kOffsetLimit = (int64_t)1 << 31;
bool gemv_offsets_ok(int M, int64_t K) { return (int64_t)M * K * 2 < kOffsetLimit && K * 16 < kOffsetLimit; }

bool is_lut3(int fmt) { return fmt == LOWBIT_LUT3_E4M3; }

int check_lut3_shape(int E, int N, int K)
{
    if (E < 0 || N < 0 || K < 0) return LOWBIT_E_INVALID_ARG;
    if (N % 8 != 0 || K % 64 != 0) return LOWBIT_E_INVALID_ARG;
    // 32-bit byte offsets inside the kernels
    if (lut3_layout(E, N, K).bytes >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    return LOWBIT_OK;
}

}  // namespace

extern "C" {

const char *lowbit_strerror(int status)
{
    switch (status) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_E_INVALID_ARG: return "invalid argument";
    case LOWBIT_E_UNSUPPORTED: return "unsupported format, group size or shape";
    case LOWBIT_E_WORKSPACE: return "workspace or packed buffer too small";
    case LOWBIT_E_HIP: return "HIP runtime error (see lowbit_last_hip_error)";
    default: return "unknown status";
    }
}

int lowbit_last_hip_error(void) { return g_last_hip_error; }

int lowbit_version(void) { return 1; }

size_t lowbit_packed_bytes(int fmt, int E, int N, int K, int group_size)
{
    if (E < 0) return 0;
    if (is_dense(fmt)) {
        if (check_dense_shape(fmt, N, K, group_size) != LOWBIT_OK) return 0;
        return (size_t)E * (size_t)dense_layout(fmt, N, K, group_size).bytes;
    }
    if (is_lut3(fmt)) {
        if (check_lut3_shape(E, N, K) != LOWBIT_OK) return 0;
        return (size_t)lut3_layout(E, N, K).bytes;
    }
    return 0;
}

int lowbit_pack_weights(int fmt, int E, int N, int K, int group_size, const void *codes,
                        const void *scales, const void *zeros, void *packed, size_t packed_bytes,
                        void *stream)
{
    if (E < 0) return LOWBIT_E_INVALID_ARG;
    if (is_lut3(fmt)) {
        int st = check_lut3_shape(E, N, K);
        if (st != LOWBIT_OK) return st;
        const Lut3Layout L = lut3_layout(E, N, K);
        if (packed_bytes < (size_t)L.bytes) return LOWBIT_E_WORKSPACE;
        if ((int64_t)E * N * K == 0) return LOWBIT_OK;
        if (packed == nullptr || codes == nullptr || scales == nullptr || zeros == nullptr) return LOWBIT_E_INVALID_ARG;
        return hip_status(launch_lut3_pack(L, static_cast<const uint8_t *>(codes), static_cast<const uint8_t *>(scales),
                                           static_cast<const uint8_t *>(zeros), static_cast<uint8_t *>(packed),
                                           (hipStream_t)stream));
    }
    if (!is_dense(fmt)) return LOWBIT_E_UNSUPPORTED;
    int st = check_dense_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    const bool asym = dense_asym(fmt);
    if (asym != (zeros != nullptr)) return LOWBIT_E_INVALID_ARG;
    const W4Layout L = dense_layout(fmt, N, K, group_size);
    if (packed_bytes < (size_t)E * (size_t)L.bytes) return LOWBIT_E_WORKSPACE;
    if (E == 0) return LOWBIT_OK;
    if (packed == nullptr) return LOWBIT_E_INVALID_ARG;
    if ((int64_t)N * K > 0 && (codes == nullptr || scales == nullptr)) return LOWBIT_E_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const int64_t ncode = dense_code_bytes(fmt, N, K), nmeta = (int64_t)N * (K / group_size);
    for (int e = 0; e < E; ++e) {
        const uint8_t *c = static_cast<const uint8_t *>(codes) + e * ncode;
        const uint16_t *sc = static_cast<const uint16_t *>(scales) + e * nmeta;
        const int8_t *z = asym ? static_cast<const int8_t *>(zeros) + e * nmeta : nullptr;
        uint8_t *dst = static_cast<uint8_t *>(packed) + (int64_t)e * L.bytes;
        hipError_t err = is_w4(fmt) ? launch_w4_pack(L, c, sc, z, dst, s) : launch_wb_pack(L, c, sc, z, dst, s);
        if (err != hipSuccess) return hip_status(err);
    }
    return LOWBIT_OK;
}

int lowbit_unpack_weights(int fmt, int E, int N, int K, int group_size, const void *packed,
                          size_t packed_bytes, void *codes, void *scales, void *zeros, void *stream)
{
    if (E < 0) return LOWBIT_E_INVALID_ARG;
    if (is_lut3(fmt)) {
        int st = check_lut3_shape(E, N, K);
        if (st != LOWBIT_OK) return st;
        const Lut3Layout L = lut3_layout(E, N, K);
        if (packed_bytes < (size_t)L.bytes) return LOWBIT_E_WORKSPACE;
        if ((int64_t)E * N * K == 0) return LOWBIT_OK;
        if (packed == nullptr || codes == nullptr || scales == nullptr || zeros == nullptr) return LOWBIT_E_INVALID_ARG;
        return hip_status(launch_lut3_unpack(L, static_cast<const uint8_t *>(packed), static_cast<uint8_t *>(codes),
                                             static_cast<uint8_t *>(scales), static_cast<uint8_t *>(zeros),
                                             (hipStream_t)stream));
    }
    if (!is_dense(fmt)) return LOWBIT_E_UNSUPPORTED;
    int st = check_dense_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    const bool asym = dense_asym(fmt);
    if (asym != (zeros != nullptr)) return LOWBIT_E_INVALID_ARG;
    const W4Layout L = dense_layout(fmt, N, K, group_size);
    if (packed_bytes < (size_t)E * (size_t)L.bytes) return LOWBIT_E_WORKSPACE;
    if (E == 0 || (int64_t)N * K == 0) return LOWBIT_OK;
    if (packed == nullptr || codes == nullptr || scales == nullptr) return LOWBIT_E_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const int64_t ncode = dense_code_bytes(fmt, N, K), nmeta = (int64_t)N * (K / group_size);
    for (int e = 0; e < E; ++e) {
        const uint8_t *src = static_cast<const uint8_t *>(packed) + (int64_t)e * L.bytes;
        uint8_t *c = static_cast<uint8_t *>(codes) + e * ncode;
        uint16_t *sc = static_cast<uint16_t *>(scales) + e * nmeta;
        int8_t *z = asym ? static_cast<int8_t *>(zeros) + e * nmeta : nullptr;
        hipError_t err = is_w4(fmt) ? launch_w4_unpack(L, src, c, sc, z, s) : launch_wb_unpack(L, src, c, sc, z, s);
        if (err != hipSuccess) return hip_status(err);
    }
    return LOWBIT_OK;
}

int lowbit_dequant(int fmt, int N, int K, int group_size, const void *packed, size_t packed_bytes,
                   float *w_out, void *stream)
{
    int st = check_dense_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    const W4Layout L = dense_layout(fmt, N, K, group_size);
    if (packed_bytes < (size_t)L.bytes) return LOWBIT_E_WORKSPACE;
    if ((int64_t)N * K == 0) return LOWBIT_OK;
    if (packed == nullptr || w_out == nullptr) return LOWBIT_E_INVALID_ARG;
    const uint8_t *src = static_cast<const uint8_t *>(packed);
    return hip_status(is_w4(fmt) ? launch_w4_dequant(L, src, w_out, (hipStream_t)stream)
                                 : launch_wb_dequant(L, src, w_out, (hipStream_t)stream));
}

int lowbit_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0) return LOWBIT_E_INVALID_ARG;
    if (bytes == 0) return LOWBIT_OK;
    if (buf == nullptr || sink == nullptr || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return LOWBIT_E_INVALID_ARG;
    return hip_status(launch_hbm_read(buf, bytes, sink, (hipStream_t)stream));
}

size_t lowbit_workspace_bytes(int op, int fmt, int M, int N, int K, int group_size)
{
    if (!is_dense(fmt) || check_dense_shape(fmt, N, K, group_size) != LOWBIT_OK || M < 0) return 0;
    if (!is_w4(fmt)) return 0;                        // b-bit GEMV: no workspace
    if (op == LOWBIT_OP_GEMV) return gemv_w4_workspace(M, N, K, group_size);
    if (op == LOWBIT_OP_GEMM) return gemm_w4_workspace(M, N, K, group_size);
    if (op == LOWBIT_OP_GEMV_W4A8) {
        if (M == 0 || N == 0) return 0;
        const W4Layout L = w4_layout(N, K, group_size, fmt == LOWBIT_W4_ASYM);
        size_t ws = 0;
        gemv_w4a8_plan(&L, 1, M, &ws);
        return ws;
    }
    return 0;
}

int lowbit_gemv(int fmt, int M, int N, int K, int group_size, const void *packed, const void *x,
                void *y, void *workspace, size_t ws_bytes, void *stream)
{
    if (is_uint_fmt(fmt)) {
        lowbit_gemv_problem p = {packed, x, y, N, K};
        return lowbit_gemv_batched(fmt, M, group_size, 1, &p, stream);
    }
    int st = check_w4_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    if (M < 0) return LOWBIT_E_INVALID_ARG;
    if (M > 16) return LOWBIT_E_UNSUPPORTED;
    if (M == 0 || N == 0) return LOWBIT_OK;
    if (packed == nullptr || y == nullptr || (K > 0 && x == nullptr)) return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return LOWBIT_E_INVALID_ARG;
    if (!gemv_offsets_ok(M, K)) return LOWBIT_E_UNSUPPORTED;
    if (ws_bytes < gemv_w4_workspace(M, N, K, group_size)) return LOWBIT_E_WORKSPACE;
    const W4Layout L = w4_layout(N, K, group_size, fmt == LOWBIT_W4_ASYM);
    return hip_status(launch_gemv_w4(L, M, static_cast<const uint8_t *>(packed),
                                     static_cast<const _Float16 *>(x), static_cast<_Float16 *>(y), workspace,
                                     ws_bytes, (hipStream_t)stream));
}

int lowbit_gemv_batched(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems, void *stream)
{
    if (count < 0 || M < 0) return LOWBIT_E_INVALID_ARG;
    if (count > kMaxGemvBatch || M > 16) return LOWBIT_E_UNSUPPORTED;
    if (count == 0 || M == 0) return LOWBIT_OK;
    if (problems == nullptr) return LOWBIT_E_INVALID_ARG;
    W4Layout L[kMaxGemvBatch];
    const uint8_t *packed[kMaxGemvBatch];
    const _Float16 *x[kMaxGemvBatch];
    _Float16 *y[kMaxGemvBatch];
    int n = 0;
    int64_t kt_max = 0;
    for (int i = 0; i < count; ++i) {
        const lowbit_gemv_problem &p = problems[i];
        int st = check_dense_shape(fmt, p.N, p.K, group_size);
        if (st != LOWBIT_OK) return st;
        if (p.N == 0) continue;                        // nothing to compute for this one
        if (p.packed == nullptr || p.y == nullptr || (p.K > 0 && p.x == nullptr)) return LOWBIT_E_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(p.x) % 16 != 0) return LOWBIT_E_INVALID_ARG;
        if (!gemv_offsets_ok(M, p.K)) return LOWBIT_E_UNSUPPORTED;
        L[n] = dense_layout(fmt, p.N, p.K, group_size);
        kt_max = L[n].ktiles > kt_max ? L[n].ktiles : kt_max;
        packed[n] = static_cast<const uint8_t *>(p.packed);
        x[n] = static_cast<const _Float16 *>(p.x);
        y[n] = static_cast<_Float16 *>(p.y);
        ++n;
    }
    if (is_uint_fmt(fmt)) {
        if (n > 0 && gemv_wb_lds(M, kt_max, uint_asym(fmt)) == 0) return LOWBIT_E_UNSUPPORTED;
        return hip_status(launch_gemv_wb_batch(L, n, M, packed, x, y, (hipStream_t)stream));
    }
    return hip_status(launch_gemv_w4_batch(L, n, M, packed, x, y, (hipStream_t)stream));
}

int lowbit_quant_act_i8(int M, int K, const void *x, int8_t *xq, float *x_scale, void *stream)
{
    if (M < 0 || K < 0 || K % 8 != 0) return LOWBIT_E_INVALID_ARG;
    if (M == 0) return LOWBIT_OK;
    if (x_scale == nullptr || (K > 0 && (x == nullptr || xq == nullptr))) return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(xq) % 8 != 0)
        return LOWBIT_E_INVALID_ARG;
    if ((int64_t)M * K >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    return hip_status(launch_quant_act_i8(M, K, static_cast<const _Float16 *>(x), xq, x_scale, (hipStream_t)stream));
}

namespace {

// Shared by the single and batched W4A8 entry points: validates the
// problems, keeps the non-empty ones, checks the plan and the workspace.
int w4a8_prepare(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems, void *workspace,
                 size_t ws_bytes, W4Layout *L, const uint8_t **packed, const _Float16 **x, _Float16 **y, int *n_out,
                 size_t *need_out = nullptr)
{
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const lowbit_gemv_problem &p = problems[i];
        int st = check_w4_shape(fmt, p.N, p.K, group_size);
        if (st != LOWBIT_OK) return st;
        if (p.N == 0) continue;
        if (p.packed == nullptr || p.y == nullptr || (p.K > 0 && p.x == nullptr)) return LOWBIT_E_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(p.x) % 16 != 0) return LOWBIT_E_INVALID_ARG;
        if (!gemv_offsets_ok(M, p.K)) return LOWBIT_E_UNSUPPORTED;
        L[n] = w4_layout(p.N, p.K, group_size, fmt == LOWBIT_W4_ASYM);
        packed[n] = static_cast<const uint8_t *>(p.packed);
        x[n] = static_cast<const _Float16 *>(p.x);
        y[n] = static_cast<_Float16 *>(p.y);
        ++n;
    }
    *n_out = n;
    if (n == 0) return LOWBIT_OK;
    size_t need = 0;
    const int mode = gemv_w4a8_plan(L, n, M, &need);
    if (mode < 0) return LOWBIT_E_UNSUPPORTED;
    if (need_out) *need_out = need;
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LOWBIT_E_WORKSPACE;
    if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return LOWBIT_E_INVALID_ARG;
    return LOWBIT_OK;
}

}  // namespace

int lowbit_gemv_w4a8(int fmt, int M, int N, int K, int group_size, const void *packed, const void *x, void *y,
                     void *workspace, size_t ws_bytes, void *stream)
{
    int st = check_w4_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    if (M < 0) return LOWBIT_E_INVALID_ARG;
    if (M > 16) return LOWBIT_E_UNSUPPORTED;
    if (M == 0 || N == 0) return LOWBIT_OK;
    lowbit_gemv_problem p = {packed, x, y, N, K};
    return lowbit_gemv_w4a8_batched(fmt, M, group_size, 1, &p, workspace, ws_bytes, stream);
}

size_t lowbit_gemv_w4a8_batched_workspace_bytes(int fmt, int M, int group_size, int count,
                                                const lowbit_gemv_problem *problems)
{
    if (count <= 0 || count > kMaxGemvBatch || M <= 0 || M > 16 || problems == nullptr) return 0;
    W4Layout L[kMaxGemvBatch];
    int n = 0;
    for (int i = 0; i < count; ++i) {
        if (check_w4_shape(fmt, problems[i].N, problems[i].K, group_size) != LOWBIT_OK) return 0;
        if (problems[i].N == 0) continue;
        L[n++] = w4_layout(problems[i].N, problems[i].K, group_size, fmt == LOWBIT_W4_ASYM);
    }
    if (n == 0) return 0;
    size_t ws = 0;
    gemv_w4a8_plan(L, n, M, &ws);
    return ws;
}

int lowbit_gemv_w4a8_batched(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems,
                             void *workspace, size_t ws_bytes, void *stream)
{
    if (count < 0 || M < 0) return LOWBIT_E_INVALID_ARG;
    if (count > kMaxGemvBatch || M > 16) return LOWBIT_E_UNSUPPORTED;
    if (count == 0 || M == 0) return LOWBIT_OK;
    if (problems == nullptr) return LOWBIT_E_INVALID_ARG;
    W4Layout L[kMaxGemvBatch];
    const uint8_t *packed[kMaxGemvBatch];
    const _Float16 *x[kMaxGemvBatch];
    _Float16 *y[kMaxGemvBatch];
    int n = 0;
    int st = w4a8_prepare(fmt, M, group_size, count, problems, workspace, ws_bytes, L, packed, x, y, &n);
    if (st != LOWBIT_OK || n == 0) return st;
    return hip_status(launch_gemv_w4a8_batch(L, n, M, packed, x, y, workspace, (hipStream_t)stream));
}

int lowbit_gemv_w4a8_batched_noalloc(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems,
                                     void *stream)
{
    if (count < 0 || M < 0) return LOWBIT_E_INVALID_ARG;
    if (count > kMaxGemvBatch || M > 16) return LOWBIT_E_UNSUPPORTED;
    if (count == 0 || M == 0) return LOWBIT_OK;
    if (problems == nullptr) return LOWBIT_E_INVALID_ARG;
    W4Layout L[kMaxGemvBatch];
    const uint8_t *packed[kMaxGemvBatch];
    const _Float16 *x[kMaxGemvBatch];
    _Float16 *y[kMaxGemvBatch];
    int n = 0;
    size_t need = 0;
    // validated against the scratch size before any HIP call; the address is a
    // placeholder here (never dereferenced: only its alignment is checked)
    int st = w4a8_prepare(fmt, M, group_size, count, problems, reinterpret_cast<void *>(256), kW4a8ScratchBytes, L,
                          packed, x, y, &n, &need);
    if (st != LOWBIT_OK || n == 0) return st;
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = w4a8_scratch(&ws);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(launch_gemv_w4a8_batch(L, n, M, packed, x, y, ws, (hipStream_t)stream));
}

size_t lowbit_gemv_chain_bytes(int count, int stages)
{
    if (count <= 0 || stages <= 0 || stages > count) return 0;
    return (size_t)chain_layout(count, stages).bytes;
}

int lowbit_gemv_chain_init(lowbit_gemv_chain *chain, int fmt, int M, int group_size, int count,
                           const lowbit_gemv_problem *problems, const int *stage_of, unsigned spin_limit,
                           void *buf, size_t buf_bytes, void *stream)
{
    if (chain == nullptr || problems == nullptr || stage_of == nullptr || buf == nullptr) return LOWBIT_E_INVALID_ARG;
    if (count <= 0 || M <= 0) return LOWBIT_E_INVALID_ARG;
    if (!is_w4(fmt) || !w4_group_ok(group_size) || M > 4) return LOWBIT_E_UNSUPPORTED;
    if (stage_of[0] != 0) return LOWBIT_E_INVALID_ARG;
    for (int i = 1; i < count; ++i) {
        const int d = stage_of[i] - stage_of[i - 1];
        if (d != 0 && d != 1) return LOWBIT_E_INVALID_ARG;
    }
    const int stages = stage_of[count - 1] + 1;
    const ChainLayout CL = chain_layout(count, stages);
    if (buf_bytes < (size_t)CL.bytes) return LOWBIT_E_WORKSPACE;

    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e);
    const int grid = cus;

    const bool asym = fmt == LOWBIT_W4_ASYM;
    std::vector<uint8_t> img((size_t)CL.bytes, 0);
    ChainProb *P = reinterpret_cast<ChainProb *>(img.data() + CL.probs_off);
    int *arrivals = reinterpret_cast<int *>(img.data() + CL.arrivals_off);
    std::vector<int64_t> stage_items(stages, 0);
    int64_t items = 0, max_ktiles = 0;
    for (int i = 0; i < count; ++i) {
        const lowbit_gemv_problem &q = problems[i];
        int st = check_w4_shape(fmt, q.N, q.K, group_size);
        if (st != LOWBIT_OK) return st;
        if (q.N == 0 || q.K == 0) return LOWBIT_E_UNSUPPORTED;
        if (q.packed == nullptr || q.x == nullptr || q.y == nullptr) return LOWBIT_E_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(q.x) % 16 != 0) return LOWBIT_E_INVALID_ARG;
        const W4Layout L = w4_layout(q.N, q.K, group_size, asym);
        if ((int64_t)M * q.K * 2 >= ((int64_t)1 << 31) || (int64_t)M * q.N * 2 >= ((int64_t)1 << 31))
            return LOWBIT_E_UNSUPPORTED;
        const uint8_t *pk = static_cast<const uint8_t *>(q.packed);
        ChainProb &c = P[i];
        c.codes = pk + L.codes_off;
        c.scales = pk + L.scales_off;
        c.zeros = asym ? pk + L.zeros_off : nullptr;
        c.x = static_cast<const _Float16 *>(q.x);
        c.y = static_cast<_Float16 *>(q.y);
        c.N = q.N;
        c.K = q.K;
        c.ktiles = (int)L.ktiles;
        c.rounds = (int)((L.ktiles + kChainRoundTiles - 1) / kChainRoundTiles);
        c.item_begin = (int)items;
        items += L.strips;
        if (items >= ((int64_t)1 << 30)) return LOWBIT_E_UNSUPPORTED;
        c.item_end = (int)items;
        c.stage = stage_of[i];
        c.pad = 0;
        stage_items[stage_of[i]] += L.strips;
        if (L.ktiles > max_ktiles) max_ktiles = L.ktiles;
    }
    for (int s = 0; s < stages; ++s)
        arrivals[s] = (int)(stage_items[s] < grid ? stage_items[s] : grid);
    // x window: whole rows of M x round_up(K, 512) halfs plus a 16-byte pad
    const int64_t xrow = round_up(max_ktiles * 128, 512) + 8;
    if ((int64_t)M * (xrow - 8) > 65536) return LOWBIT_E_UNSUPPORTED;
    const size_t lds = gemv_chain_lds_bytes(M, (int)xrow);
    if (gemv_chain_occupancy(group_size, asym, M, lds) < 1) return LOWBIT_E_UNSUPPORTED;

    e = hipMemcpyAsync(buf, img.data(), img.size(), hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);

    chain->fmt = fmt;
    chain->M = M;
    chain->group_size = group_size;
    chain->count = count;
    chain->stages = stages;
    chain->grid = grid;
    chain->xrow = (int)xrow;
    chain->spin_limit = spin_limit ? spin_limit : (1u << 20);
    chain->buf = buf;
    chain->buf_bytes = (size_t)CL.bytes;
    return LOWBIT_OK;
}

int lowbit_gemv_chain_run(const lowbit_gemv_chain *chain, void *stream)
{
    if (chain == nullptr || chain->buf == nullptr || chain->count <= 0 || chain->grid <= 0) return LOWBIT_E_INVALID_ARG;
    const ChainLayout CL = chain_layout(chain->count, chain->stages);
    uint8_t *b = static_cast<uint8_t *>(chain->buf);
    ChainArgs a;
    a.probs = reinterpret_cast<const ChainProb *>(b + CL.probs_off);
    a.arrivals = reinterpret_cast<const int *>(b + CL.arrivals_off);
    a.ctr = reinterpret_cast<uint32_t *>(b);
    a.nprob = chain->count;
    a.M = chain->M;
    a.xrow = chain->xrow;
    a.spin_limit = chain->spin_limit;
    return hip_status(launch_gemv_chain(chain->group_size, chain->fmt == LOWBIT_W4_ASYM, a, chain->grid,
                                        (hipStream_t)stream));
}

int lowbit_gemv_chain_error(const lowbit_gemv_chain *chain, unsigned *error, void *stream)
{
    if (chain == nullptr || chain->buf == nullptr || error == nullptr) return LOWBIT_E_INVALID_ARG;
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, chain->buf, 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    *error = v;
    return LOWBIT_OK;
}

int lowbit_gemm(int fmt, int M, int N, int K, int group_size, const void *packed, const void *a, int a_dtype,
                void *c, int c_dtype, void *workspace, size_t ws_bytes, void *stream)
{
    int st = check_w4_shape(fmt, N, K, group_size);
    if (st != LOWBIT_OK) return st;
    if (M < 0) return LOWBIT_E_INVALID_ARG;
    if ((a_dtype != LOWBIT_F16 && a_dtype != LOWBIT_BF16) || (c_dtype != LOWBIT_F16 && c_dtype != LOWBIT_BF16))
        return LOWBIT_E_UNSUPPORTED;
    if (M == 0 || N == 0) return LOWBIT_OK;
    if (packed == nullptr || c == nullptr || (K > 0 && a == nullptr)) return LOWBIT_E_INVALID_ARG;
    if ((int64_t)M * K > (int64_t)INT32_MAX || (int64_t)M * N > (int64_t)INT32_MAX) return LOWBIT_E_UNSUPPORTED;
    const W4Layout L = w4_layout(N, K, group_size, fmt == LOWBIT_W4_ASYM);
    // A and the packed blob are each one 32-bit-offset descriptor
    if ((int64_t)M * K * 2 >= kOffsetLimit || L.bytes >= kOffsetLimit) return LOWBIT_E_UNSUPPORTED;
    const size_t need = gemm_w4_workspace(M, N, K, group_size);
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LOWBIT_E_WORKSPACE;
    return hip_status(launch_gemm_w4(L, M, static_cast<const uint8_t *>(packed), a, a_dtype == LOWBIT_BF16, c,
                                     c_dtype == LOWBIT_BF16, workspace, ws_bytes, (hipStream_t)stream));
}

int lowbit_moe_align(const int32_t *topk_ids, int T, int top_k, int E, int block_m, const int32_t *expert_map,
                     int32_t *sorted_ids, int32_t *expert_offsets, int32_t *block_expert,
                     int32_t *num_post_padded, void *stream)
{
    if (T < 0 || top_k < 0 || E <= 0 || block_m <= 0) return LOWBIT_E_INVALID_ARG;
    if (E > 1024 || block_m > 4096) return LOWBIT_E_UNSUPPORTED;
    const int64_t num_valid = (int64_t)T * top_k;
    const int64_t capacity = num_valid + (int64_t)E * (block_m - 1);
    if (capacity >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    if (sorted_ids == nullptr || expert_offsets == nullptr || block_expert == nullptr || num_post_padded == nullptr)
        return LOWBIT_E_INVALID_ARG;
    if (num_valid > 0 && topk_ids == nullptr) return LOWBIT_E_INVALID_ARG;
    return hip_status(launch_moe_align(topk_ids, (int)num_valid, E, block_m, expert_map, sorted_ids, expert_offsets,
                                       block_expert, num_post_padded, (int)capacity, (hipStream_t)stream));
}

int lowbit_moe_gemm(int fmt, int E_local, int N, int K, const void *packed, int E, const uint8_t *a_e4m3,
                    const uint8_t *a_ue8m0, int a_rows, int a_row_div, const int32_t *sorted_ids,
                    const int32_t *expert_offsets, const int32_t *block_expert, int num_valid, int block_m,
                    void *out, void *stream)
{
    if (!is_lut3(fmt)) return LOWBIT_E_UNSUPPORTED;
    int st = check_lut3_shape(E_local, N, K);
    if (st != LOWBIT_OK) return st;
    if (E <= 0 || a_rows < 0 || a_row_div <= 0 || num_valid < 0 || block_m <= 0) return LOWBIT_E_INVALID_ARG;
    if (block_m % 16 != 0) return LOWBIT_E_UNSUPPORTED;
    if (num_valid > 0 && (int64_t)(num_valid - 1) / a_row_div >= a_rows) return LOWBIT_E_INVALID_ARG;
    if ((int64_t)a_rows * K >= ((int64_t)1 << 31) || (int64_t)num_valid * N >= ((int64_t)1 << 31))
        return LOWBIT_E_UNSUPPORTED;
    if (num_valid == 0 || N == 0) return LOWBIT_OK;
    if (packed == nullptr || out == nullptr || sorted_ids == nullptr || expert_offsets == nullptr ||
        block_expert == nullptr || (K > 0 && (a_e4m3 == nullptr || a_ue8m0 == nullptr)))
        return LOWBIT_E_INVALID_ARG;
    const Lut3Layout L = lut3_layout(E_local, N, K);
    return hip_status(launch_moe_gemm(L, static_cast<const uint8_t *>(packed), E, a_e4m3, a_ue8m0, a_rows,
                                      a_row_div, sorted_ids, expert_offsets, block_expert, num_valid, block_m,
                                      static_cast<uint16_t *>(out), (hipStream_t)stream));
}

int lowbit_moe_gemm_silu_quant(int fmt, int E_local, int I, int K, const void *packed, int E, const uint8_t *a_e4m3,
                               const uint8_t *a_ue8m0, int a_rows, int a_row_div, const int32_t *sorted_ids,
                               const int32_t *expert_offsets, const int32_t *block_expert, int num_valid,
                               int block_m, uint8_t *q, uint8_t *scale, void *stream)
{
    if (!is_lut3(fmt)) return LOWBIT_E_UNSUPPORTED;
    if (I < 0 || I > (1 << 29)) return LOWBIT_E_INVALID_ARG;
    int st = check_lut3_shape(E_local, 2 * I, K);
    if (st != LOWBIT_OK) return st;
    if (E <= 0 || a_rows < 0 || a_row_div <= 0 || num_valid < 0 || block_m <= 0) return LOWBIT_E_INVALID_ARG;
    if (block_m % 16 != 0 || I % 128 != 0 || K > 4864) return LOWBIT_E_UNSUPPORTED;
    if (num_valid > 0 && (int64_t)(num_valid - 1) / a_row_div >= a_rows) return LOWBIT_E_INVALID_ARG;
    if ((int64_t)a_rows * K >= ((int64_t)1 << 31) || (int64_t)num_valid * I >= ((int64_t)1 << 31))
        return LOWBIT_E_UNSUPPORTED;
    if (num_valid == 0 || I == 0) return LOWBIT_OK;
    if (packed == nullptr || q == nullptr || scale == nullptr || sorted_ids == nullptr ||
        expert_offsets == nullptr || block_expert == nullptr || (K > 0 && (a_e4m3 == nullptr || a_ue8m0 == nullptr)))
        return LOWBIT_E_INVALID_ARG;
    const hipError_t e = launch_moe_gemm_silu(lut3_layout(E_local, 2 * I, K), static_cast<const uint8_t *>(packed),
                                              E, a_e4m3, a_ue8m0, a_rows, a_row_div, sorted_ids, expert_offsets,
                                              block_expert, num_valid, block_m, q, scale, (hipStream_t)stream);
    return e == hipErrorNotSupported ? LOWBIT_E_UNSUPPORTED : hip_status(e);
}

int lowbit_mxfp8_quant(const void *x, int R, int K, uint8_t *q, uint8_t *scale, void *stream)
{
    if (R < 0 || K < 0 || K % 32 != 0) return LOWBIT_E_INVALID_ARG;
    if (R == 0 || K == 0) return LOWBIT_OK;
    if (x == nullptr || q == nullptr || scale == nullptr) return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 8 != 0)
        return LOWBIT_E_INVALID_ARG;
    if ((int64_t)R * K >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    return hip_status(launch_mxfp8_rows(static_cast<const uint16_t *>(x), R, K, false, q, scale, (hipStream_t)stream));
}

int lowbit_moe_silu_mul_quant(const void *gate_up, int R, int I, uint8_t *q, uint8_t *scale, void *stream)
{
    if (R < 0 || I < 0 || I % 32 != 0) return LOWBIT_E_INVALID_ARG;
    if (R == 0 || I == 0) return LOWBIT_OK;
    if (gate_up == nullptr || q == nullptr || scale == nullptr) return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(gate_up) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 8 != 0)
        return LOWBIT_E_INVALID_ARG;
    if ((int64_t)R * 2 * I >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    return hip_status(launch_mxfp8_rows(static_cast<const uint16_t *>(gate_up), R, I, true, q, scale,
                                        (hipStream_t)stream));
}

int lowbit_moe_combine(const void *expert_out, const float *topk_weights, int T, int top_k, int H, void *y,
                       void *stream)
{
    if (T < 0 || top_k < 0 || H < 0 || H % 8 != 0) return LOWBIT_E_INVALID_ARG;
    if (T == 0 || H == 0) return LOWBIT_OK;
    if (y == nullptr || (top_k > 0 && (expert_out == nullptr || topk_weights == nullptr)))
        return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(expert_out) % 16 != 0 || reinterpret_cast<uintptr_t>(y) % 16 != 0)
        return LOWBIT_E_INVALID_ARG;
    if ((int64_t)T * top_k * H >= ((int64_t)1 << 31)) return LOWBIT_E_UNSUPPORTED;
    return hip_status(launch_moe_combine(static_cast<const uint16_t *>(expert_out), topk_weights, T, top_k, H,
                                         static_cast<uint16_t *>(y), (hipStream_t)stream));
}

namespace {
int moe_layer_check(int E_local, int E, int H, int I, int T, int top_k, int block_m)
{
    if (E_local < 0 || E <= 0 || H <= 0 || I <= 0 || T < 0 || top_k <= 0 || block_m <= 0) return LOWBIT_E_INVALID_ARG;
    if (H % 64 != 0 || I % 64 != 0) return LOWBIT_E_INVALID_ARG;     // both GEMMs' K is a multiple of 64
    if (E > 1024 || block_m % 16 != 0 || block_m > 4096) return LOWBIT_E_UNSUPPORTED;
    const MoeLayerWs w = moe_layer_ws(T, top_k, E, H, I, block_m);
    if (w.capacity >= ((int64_t)1 << 31) || w.bytes >= ((int64_t)1 << 40) ||
        (int64_t)T * top_k * 2 * I >= ((int64_t)1 << 31) || (int64_t)T * top_k * H >= ((int64_t)1 << 31))
        return LOWBIT_E_UNSUPPORTED;
    if (check_lut3_shape(E_local, 2 * I, H) != LOWBIT_OK || check_lut3_shape(E_local, H, I) != LOWBIT_OK)
        return LOWBIT_E_UNSUPPORTED;
    return LOWBIT_OK;
}
}  // namespace

size_t lowbit_moe_layer_workspace_bytes(int T, int top_k, int E, int H, int I, int block_m)
{
    if (moe_layer_check(0, E, H, I, T, top_k, block_m) != LOWBIT_OK) return 0;
    return (size_t)moe_layer_ws(T, top_k, E, H, I, block_m).bytes;
}

int lowbit_moe_layer(const void *w13, const void *w2, int E_local, int E, int H, int I, const void *x,
                     const int32_t *topk_ids, const float *topk_weights, int T, int top_k, const int32_t *expert_map,
                     int block_m, void *y, void *workspace, size_t ws_bytes, void *stream)
{
    int st = moe_layer_check(E_local, E, H, I, T, top_k, block_m);
    if (st != LOWBIT_OK) return st;
    if (T == 0) return LOWBIT_OK;
    if (x == nullptr || topk_ids == nullptr || topk_weights == nullptr || y == nullptr || workspace == nullptr ||
        (E_local > 0 && (w13 == nullptr || w2 == nullptr)) || (expert_map == nullptr && E > E_local))
        return LOWBIT_E_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(y) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return LOWBIT_E_INVALID_ARG;
    const MoeLayerWs w = moe_layer_ws(T, top_k, E, H, I, block_m);
    if (ws_bytes < (size_t)w.bytes) return LOWBIT_E_WORKSPACE;
    const hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint8_t *xq = ws + w.xq, *xs = ws + w.xs, *aq = ws + w.aq, *as = ws + w.as;
    int32_t *sorted = reinterpret_cast<int32_t *>(ws + w.sorted), *offs = reinterpret_cast<int32_t *>(ws + w.offsets);
    int32_t *blk = reinterpret_cast<int32_t *>(ws + w.blocks), *npp = reinterpret_cast<int32_t *>(ws + w.npp);
    uint16_t *gu = reinterpret_cast<uint16_t *>(ws + w.gate_up), *down = reinterpret_cast<uint16_t *>(ws + w.down);
    const int slots = T * top_k;
    hipError_t e = launch_moe_prep(static_cast<const uint16_t *>(x), T, H, xq, xs, topk_ids, slots, E, block_m,
                                   expert_map, sorted, offs, blk, npp, (int)w.capacity, s);
    if (e == hipSuccess) {
        // gate/up with SiLU(gate) * up -> MXFP8 in its epilogue where the shape
        // allows it; otherwise bf16 gate/up rows and the stand-alone pass
        e = launch_moe_gemm_silu(lut3_layout(E_local, 2 * I, H), static_cast<const uint8_t *>(w13), E, xq, xs, T,
                                 top_k, sorted, offs, blk, slots, block_m, aq, as, s);
        if (e == hipErrorNotSupported) {
            e = launch_moe_gemm(lut3_layout(E_local, 2 * I, H), static_cast<const uint8_t *>(w13), E, xq, xs, T,
                                top_k, sorted, offs, blk, slots, block_m, gu, s);
            if (e == hipSuccess) e = launch_mxfp8_rows(gu, slots, I, true, aq, as, s);
        }
    }
    if (e == hipSuccess)
        e = launch_moe_gemm(lut3_layout(E_local, H, I), static_cast<const uint8_t *>(w2), E, aq, as, slots, 1, sorted,
                            offs, blk, slots, block_m, down, s);
    if (e == hipSuccess) e = launch_moe_combine(down, topk_weights, T, top_k, H, static_cast<uint16_t *>(y), s);
    return hip_status(e);
}

}  // extern "C"
