/*
 * lowbit.h -- C ABI of liblowbit.so: low-bit weight-only matmul with fused
 * group-wise dequantization on AMD Instinct MI355X (gfx950).
 *
 * What is computed (web pages cited by title and section):
 *   - "Low Bit Metal Kernels" (GPU MODE lecture 49 notes), MSL listing
 *     `int4_matmul`: weights are INT4 codes packed two per byte, the low
 *     nibble being the even K row and the high nibble the odd one; each is
 *     dequantized just before use as (code - zero) * scale[group] and
 *     multiplied with fp16 activations (buffer arguments W_packed, scales, X,
 *     Y, M, N, K).
 *   - "Low Bit ARM kernels" (GPU MODE lecture 38 notes): decode at batch 1 is
 *     a GEMV and dominates latency, prefill is a GEMM; quantization is
 *     group-wise along K with groups of 32, 64 or 128, symmetric (scale only)
 *     or asymmetric (fp16 scale plus int8 zero point per group); weights are
 *     re-packed offline into the kernel's layout; kernels are plain native
 *     functions.
 *   - "vLLM PR #62759 analysis" (LUT-B MoE with MXFP8 activations): 3-bit
 *     LUT-codebook expert weights, MXFP8 activations, grouped expert GEMM over
 *     rows bucketed per expert, zero rows for experts that are not local.
 *
 * Conventions, for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains device memory.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Arguments are validated on the host before anything is
 *     enqueued; a call that returns an error has enqueued nothing.  Faults in
 *     enqueued kernels surface at the caller's next synchronisation.
 *   - Matrices are row-major and densely packed unless stated otherwise.
 *   - Return value: LOWBIT_OK or one of the LOWBIT_E_* codes.  No call throws
 *     or aborts.  Calls are thread-safe; the library keeps no mutable global
 *     state besides the per-thread last HIP error.
 *   - Shapes: M, N, K >= 0.  M == 0 or N == 0 is a valid empty call that
 *     enqueues nothing.  K == 0 gives an all-zero output.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define LOWBIT_OK             0
#define LOWBIT_E_INVALID_ARG  1  /* null pointer, negative size, K % group_size != 0, ... */
#define LOWBIT_E_UNSUPPORTED  2  /* valid request this library has no kernel for */
#define LOWBIT_E_WORKSPACE    3  /* workspace or packed buffer smaller than required */
#define LOWBIT_E_HIP          4  /* a HIP call failed; see lowbit_last_hip_error() */

/* ---- weight formats ---------------------------------------------------- */
#define LOWBIT_W4_SYM     0  /* INT4 codes, fp16 scale per group, zero point 8   */
#define LOWBIT_W4_ASYM    1  /* INT4 codes, fp16 scale + int8 zero point / group */
#define LOWBIT_LUT3_E4M3  2  /* 3-bit index into an 8-entry E4M3 codebook per
                                8 outputs x 64 K tile, one UE8M0 exponent per tile */
/* Uniform b-bit codes, b = 1..8 ("Low Bit ARM kernels": one unpack routine per
 * bit width 1-8), fp16 scale per group, zero point 2^(b-1) (asym = 0) or an
 * int8 zero point per group (asym = 1):  w = (q - z) * s, 0 <= q < 2^b.
 * Canonical codes are one per byte (bits above b are ignored). */
#define LOWBIT_UINT(bits, asym) (16 + 2 * (bits) + ((asym) ? 1 : 0))

/* ---- activation / output element types --------------------------------- */
#define LOWBIT_F16   0
#define LOWBIT_BF16  1

/* ---- operations (for lowbit_workspace_bytes) ---------------------------- */
#define LOWBIT_OP_GEMV       0
#define LOWBIT_OP_GEMM       1
#define LOWBIT_OP_GEMV_W4A8  2

/* Human-readable text for a status code (static storage, never NULL). */
const char *lowbit_strerror(int status);

/* HIP error code (hipError_t value) of the last call on this thread that
 * returned LOWBIT_E_HIP; 0 if none. */
int lowbit_last_hip_error(void);

/* ABI version of this library (incremented on any incompatible change). */
int lowbit_version(void);

/*
 * Size in bytes of the packed weight blob for E matrices of N outputs x K
 * inputs.  For W4 formats the blob of matrix e starts at
 * e * lowbit_packed_bytes(fmt, 1, N, K, group_size).  Returns 0 for an
 * invalid combination (W4: group_size not in {32, 64, 128}, K % group_size,
 * negative sizes).  Pure host arithmetic; never touches the GPU.
 */
size_t lowbit_packed_bytes(int fmt, int E, int N, int K, int group_size);

/*
 * Offline re-pack of canonical quantized weights into the device layout the
 * kernels read ("Low Bit ARM kernels": weights are pre-packed once into a
 * cache-friendly layout; the vLLM PR #62759 analysis, "weights pre-arranged
 * at load time": the costly layout transform is a one-off at load).  The
 * packing is a lossless permutation: lowbit_unpack_weights returns the input
 * bytes exactly.
 *
 * W4 formats (group_size in {32, 64, 128}, K % group_size == 0):
 *   codes  : u8  [E][N][K/2]   byte j of row n holds k = 2j (low nibble) and
 *                               k = 2j+1 (high nibble); codes 0..15
 *   scales : f16 [E][N][K/group_size]
 *   zeros  : i8  [E][N][K/group_size] for LOWBIT_W4_ASYM; must be NULL for
 *            LOWBIT_W4_SYM (zero point 8)
 * LOWBIT_UINT(bits, asym) (same group sizes and shape rules as W4):
 *   codes  : u8  [E][N][K]    one code per weight, 0 <= q < 2^bits
 *   scales : f16 [E][N][K/group_size]
 *   zeros  : i8  [E][N][K/group_size] when asym, else NULL (zero point 2^(bits-1))
 * LOWBIT_LUT3_E4M3 (group_size ignored, N % 8 == 0, K % 64 == 0):
 *   codes  : u8  [E][N][K]           one index 0..7 per weight
 *   scales : u8  [E][N/8][K/64][8]   E4M3 codebook of each 8 x 64 tile
 *   zeros  : u8  [E][N/8][K/64]      UE8M0 exponent of each tile
 * packed : output, packed_bytes >= lowbit_packed_bytes(fmt, E, N, K, group_size)
 *          (else LOWBIT_E_WORKSPACE).  Padding inside the blob is written too,
 *          so the blob is fully defined.
 * Inputs must not overlap the output.
 */
int lowbit_pack_weights(int fmt, int E, int N, int K, int group_size,
                        const void *codes, const void *scales, const void *zeros,
                        void *packed, size_t packed_bytes, void *stream);

/*
 * Inverse of lowbit_pack_weights (test and export hook): writes the canonical
 * arrays described above.  zeros must be NULL for LOWBIT_W4_SYM.
 */
int lowbit_unpack_weights(int fmt, int E, int N, int K, int group_size,
                          const void *packed, size_t packed_bytes,
                          void *codes, void *scales, void *zeros, void *stream);

/*
 * Dequantize one packed W4 or LOWBIT_UINT matrix to fp32 (test hook):
 *   w[n][k] = (q[n][k] - z) * s[n][k / group_size],  w_out f32 [N][K].
 * The product is exact in fp32 (|q - z| <= 383 has 9 significant bits, an
 * fp16 scale 11), so the result is bit-identical to any exact evaluation.
 */
int lowbit_dequant(int fmt, int N, int K, int group_size,
                   const void *packed, size_t packed_bytes, float *w_out, void *stream);

/*
 * Read-only streaming of a device buffer: the practical ceiling of HBM reads,
 * measured beside the kernels' rooflines ("Low Bit Metal Kernels", practice
 * sequence: measure the memory-bandwidth utilisation of a bandwidth-bound
 * kernel).  Every 16-byte block is read once with non-temporal loads by
 * LOWBIT_HBM_READ_SINK_WORDS workgroups, each of which stores the XOR of the
 * 32-bit words it read to its own sink word, so that
 *   XOR of sink[0 .. LOWBIT_HBM_READ_SINK_WORDS)  ==  XOR of all 32-bit words of buf
 * (no load is dead and the result can be checked; with bytes > 0 every sink
 * word is written).
 *   buf   : device pointer, 16-byte aligned, `bytes` readable bytes
 *   bytes : a multiple of 16 (0: nothing is enqueued)
 *   sink  : device uint32 [LOWBIT_HBM_READ_SINK_WORDS] (output), 4-byte aligned
 * Errors: LOWBIT_E_INVALID_ARG for a negative or ragged size, a null or
 * misaligned pointer; nothing is enqueued then.
 */
#define LOWBIT_HBM_READ_SINK_WORDS 1024
int lowbit_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/*
 * Workspace bytes an operation needs for this shape (0 if none).  Pass a
 * workspace of at least this size to that operation.
 */
size_t lowbit_workspace_bytes(int op, int fmt, int M, int N, int K, int group_size);

/*
 * Decode GEMV / small-batch product with W4 weights ("Low Bit Metal
 * Kernels", int4_matmul; "Low Bit ARM kernels", decode = GEMV):
 *   y[m][n] = sum_k x[m][k] * (q[n][k] - z) * s[n][k / group_size]
 * accumulated in fp32, rounded to nearest even into fp16.
 *   fmt     : LOWBIT_W4_SYM, LOWBIT_W4_ASYM or LOWBIT_UINT(bits, asym)
 *             (b-bit codes: K <= 16384, and M * round_up(2K, 1024) bytes of x
 *             -- 2.5K per row for M = 1 symmetric -- plus 4, 8 or 16 KiB of
 *             partial sums for M = 1, <= 8, <= 16 must fit 160 KiB of LDS;
 *             else LOWBIT_E_UNSUPPORTED.  At K = 16384: M <= 4)
 *   M       : 0..16 rows (tokens); larger M -> LOWBIT_E_UNSUPPORTED (use lowbit_gemm)
 *   packed  : blob from lowbit_pack_weights(fmt, 1, N, K, group_size, ...)
 *   x       : f16 [M][K], 16-byte aligned
 *   y       : f16 [M][N] (output; must not overlap x or packed)
 *   workspace / ws_bytes : per lowbit_workspace_bytes(LOWBIT_OP_GEMV, ...)
 *            (may be NULL when that is 0)
 */
int lowbit_gemv(int fmt, int M, int N, int K, int group_size,
                const void *packed, const void *x, void *y,
                void *workspace, size_t ws_bytes, void *stream);

/* One GEMV of a batch: y = x @ W^T with W packed for (fmt, 1, N, K, group_size). */
typedef struct lowbit_gemv_problem {
    const void *packed;  /* device blob from lowbit_pack_weights               */
    const void *x;       /* device f16 [M][K], 16-byte aligned                 */
    void *y;             /* device f16 [M][N]; must not overlap any input      */
    int N, K;
} lowbit_gemv_problem;

/*
 * Up to 8 independent GEMVs (same fmt, M and group_size, any N and K) in one
 * launch, each with exactly the result of lowbit_gemv.  This is the fused
 * launch for projections that read the same layer input, e.g. q/k/v and
 * gate/up of a decoder layer ("BaseRT" wiki chapter, "BaseRT's approach":
 * interleaved QKV weights and fewer, batched submissions cut the per-kernel
 * overhead that dominates batch-1 decode).  `problems` is a HOST array of
 * `count` entries, read during the call.  count > 8 -> LOWBIT_E_UNSUPPORTED.
 * No workspace.
 */
int lowbit_gemv_batched(int fmt, int M, int group_size, int count,
                        const lowbit_gemv_problem *problems, void *stream);

/*
 * Dynamic per-token INT8 quantization of activations ("Low Bit ARM kernels",
 * measurements section: 4-bit weights run with dynamic INT8 activations; the
 * page names the scheme, the rounding below is this library's definition).
 * For each token row m, in binary32 with correctly rounded operations:
 *   amax = max_k |x[m][k]|,  inv = 127 / amax,  x_scale[m] = amax / 127,
 *   xq[m][k] = round-to-nearest-even(x[m][k] * inv)   (in [-127, 127])
 * A row of zeros gives x_scale 0 and codes 0.  x must be finite.
 *   x       : f16 [M][K], 16-byte aligned; K % 8 == 0
 *   xq      : i8  [M][K] (output), 8-byte aligned
 *   x_scale : f32 [M]    (output)
 * This is the quantization lowbit_gemv_w4a8 applies internally; it is
 * exported as a building block and test hook.
 */
int lowbit_quant_act_i8(int M, int K, const void *x, int8_t *xq, float *x_scale, void *stream);

/*
 * W4A8 decode GEMV / small-batch product: W4 weights against dynamically
 * quantized INT8 activations on the int8 matrix cores ("Low Bit ARM kernels":
 * 4-bit weights with dynamic INT8 activations, group size 32; unpacked weights
 * kept as int8 and fed to int8 matrix-multiply instructions with int32
 * accumulation):
 *   y[m][n] = x_scale[m] * sum_g s[n][g] * sum_{k in g} xq[m][k] * (q[n][k] - z)
 * with xq, x_scale as lowbit_quant_act_i8 defines them; the inner sums are
 * exact int32, the scales are applied in fp32, y is rounded to nearest even
 * into fp16.  Arguments as lowbit_gemv (same packed blob).
 *   M         : 0..16 rows; K <= 16384 (else LOWBIT_E_UNSUPPORTED)
 *   workspace : >= lowbit_workspace_bytes(LOWBIT_OP_GEMV_W4A8, ...) bytes,
 *               256-byte aligned; 0 (no workspace) at M = 1, where the
 *               launch quantizes the activations itself.  From M = 2 a first
 *               kernel quantizes them into the workspace (one pass instead of
 *               one per workgroup).
 */
int lowbit_gemv_w4a8(int fmt, int M, int N, int K, int group_size, const void *packed, const void *x, void *y,
                     void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of lowbit_gemv_w4a8_batched for these problems (HOST
 * array, read during the call); 0 when none is needed or the batch is invalid. */
size_t lowbit_gemv_w4a8_batched_workspace_bytes(int fmt, int M, int group_size, int count,
                                                const lowbit_gemv_problem *problems);

/*
 * Up to 8 independent W4A8 GEMVs in one launch (same fmt, M and group_size),
 * each with exactly the result of lowbit_gemv_w4a8: the batched form for
 * projections that share a layer input (q/k/v, gate/up), as
 * lowbit_gemv_batched.  workspace: >= lowbit_gemv_w4a8_batched_workspace_bytes
 * (may be NULL when that is 0).
 */
int lowbit_gemv_w4a8_batched(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * lowbit_gemv_w4a8_batched without a workspace argument, for callers that
 * cannot allocate device memory at all (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The activation blocks go
 * to a static 512 KiB device array inside the library instead of a caller
 * workspace; the call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine).  Results equal lowbit_gemv_w4a8_batched's bit
 * for bit (same kernels).
 *   Limit: the plan's workspace (lowbit_gemv_w4a8_batched_workspace_bytes for
 *   the same problems) must be <= 512 KiB, else LOWBIT_E_WORKSPACE before
 *   anything is enqueued; every 8B decode launch up to M = 8 fits (at most 130 KB; M = 1 needs
 *   none).  The scratch address of a device is looked up on the first call
 *   made with that device current (a failure returns LOWBIT_E_HIP).
 *   Calls that overlap on one GPU (different streams, or different host
 *   threads) share that GPU's array and race: serialize them.  Each call
 *   rewrites every scratch byte it later reads, so nothing needs clearing.
 */
int lowbit_gemv_w4a8_batched_noalloc(int fmt, int M, int group_size, int count, const lowbit_gemv_problem *problems,
                                     void *stream);

/*
 * A chain of dependent GEMV stages executed by ONE persistent launch: a whole
 * decode step (every projection of every layer) as a single submission
 * ("BaseRT" wiki chapter, limitations and approach: at batch 1 the per-command
 * submission overhead dominates, so the many small operations of a step are
 * encoded into one submission; "Low Bit ARM kernels": each projection is a
 * bandwidth-bound GEMV).
 *
 * Problem i (same fmt, M and group_size for all) belongs to stage stage_of[i];
 * stage_of[0] == 0 and stage_of[i] - stage_of[i-1] is 0 or 1.  Every problem
 * of stage s+1 reads its x only after every problem of stage s has written its
 * y, so the y of one stage may be the x of the next.  Within one stage no y
 * may overlap any input of that stage.  Each y is the product lowbit_gemv
 * defines (fp32 accumulation in a fixed order, fp16 RNE); the summation order
 * is fixed, so a run is bit-reproducible.
 *
 * Usage: lowbit_gemv_chain_bytes -> allocate a device buffer of that size ->
 * lowbit_gemv_chain_init (once; copies the plan into the buffer, host-
 * synchronous) -> lowbit_gemv_chain_run (each step; asynchronous, capturable
 * in a graph: the buffer needs no clearing between runs).  Runs of one chain
 * must not overlap in time (keep them on one stream).  The device buffer, the
 * weights and the x/y buffers named at init must stay valid while the chain is
 * used; x contents may change between runs.
 *
 * Limits: 1 <= M <= 4; every problem has N >= 1 and K >= 1 (else
 * LOWBIT_E_UNSUPPORTED), M * K * 2 bytes of x must fit the LDS window
 * (M * round_up(K, 512) <= 65536 halfs, else LOWBIT_E_UNSUPPORTED).
 */
typedef struct lowbit_gemv_chain {
    int fmt, M, group_size;
    int count;                 /* problems */
    int stages;
    int grid;                  /* persistent workgroups: one per compute unit */
    int xrow;                  /* internal: LDS row stride of x */
    unsigned spin_limit;       /* polls before a dependency wait gives up */
    void *buf;                 /* the device buffer passed to init */
    size_t buf_bytes;
} lowbit_gemv_chain;

/* Device bytes of the chain buffer for `count` problems in `stages` stages
 * (0 for invalid counts). */
size_t lowbit_gemv_chain_bytes(int count, int stages);

/*
 * Validate the problems (HOST arrays `problems` and `stage_of`, read during
 * the call), build the plan and copy it with zeroed counters into `buf`
 * (device, >= lowbit_gemv_chain_bytes(count, stages)) on `stream`; returns
 * after the copy completed.  spin_limit: polls of a dependency wait before it
 * gives up (0 = default, about seconds); a wait that gives up sets bit 0 of
 * the chain's error word (lowbit_gemv_chain_error) and the run's results are
 * undefined, but the launch still completes.  Fills *chain.
 */
int lowbit_gemv_chain_init(lowbit_gemv_chain *chain, int fmt, int M, int group_size, int count,
                           const lowbit_gemv_problem *problems, const int *stage_of,
                           unsigned spin_limit, void *buf, size_t buf_bytes, void *stream);

/* Enqueue one run of the chain on `stream`, as a cooperative launch: every
 * workgroup is resident at once, or the launch is refused (LOWBIT_E_HIP with
 * hipErrorCooperativeLaunchTooLarge, e.g. when other work holds the compute
 * units' resources) and nothing runs.  Capturable in a graph. */
int lowbit_gemv_chain_run(const lowbit_gemv_chain *chain, void *stream);

/* Read the chain's error word (0 = every wait so far was met) into *error;
 * synchronizes `stream`. */
int lowbit_gemv_chain_error(const lowbit_gemv_chain *chain, unsigned *error, void *stream);

/*
 * Prefill GEMM with W4 weights ("Low Bit ARM kernels": prefill is the same
 * product over many tokens; "Low Bit Metal Kernels": activation and weight
 * tiles staged on chip and multiplied):
 *   c[m][n] = sum_k a[m][k] * (q[n][k] - z) * s[n][k / group_size]
 * on the matrix cores with fp32 accumulation; weights are never rounded
 * (scales are applied in fp32 per group); the sum is rounded to nearest even
 * into c_dtype.
 *   fmt             : LOWBIT_W4_SYM or LOWBIT_W4_ASYM
 *   M               : any number of rows >= 0
 *   packed          : blob from lowbit_pack_weights(fmt, 1, N, K, group_size, ...)
 *   a / a_dtype     : [M][K] activations, LOWBIT_BF16 or LOWBIT_F16
 *   c / c_dtype     : [M][N] output, LOWBIT_BF16 or LOWBIT_F16 (must not overlap a)
 *   workspace       : >= lowbit_workspace_bytes(LOWBIT_OP_GEMM, fmt, M, N, K,
 *                     group_size) bytes (fp32 split-K partials for shapes whose
 *                     output tiles alone cannot fill the GPU; may be NULL when 0)
 * Scales must be finite; a zero scale contributes nothing (exactly).
 */
int lowbit_gemm(int fmt, int M, int N, int K, int group_size, const void *packed,
                const void *a, int a_dtype, void *c, int c_dtype,
                void *workspace, size_t ws_bytes, void *stream);

/*
 * Bucket routed token slots by expert ("vLLM PR #62759 analysis", section
 * "A gather": the grouped GEMM walks rows through sorted_token_ids built by
 * moe_align_block_size; a slot id below the number of routed slots is a real
 * row).  Slot sid = t * top_k + j is token t's j-th routed expert
 * topk_ids[t][j].  Output order: experts ascending by global id, slot ids
 * ascending within an expert; each expert's run is padded to a multiple of
 * block_m with the sentinel T * top_k; experts with no slot have no block.
 *   topk_ids       : i32 [T][top_k], values in [0, E) (other values are ignored)
 *   expert_map     : i32 [E] global -> local expert id or -1 (not on this
 *                    device); NULL = identity
 *   sorted_ids     : i32 [T*top_k + E*(block_m-1)] (output; entries past the
 *                    padded length hold the sentinel)
 *   expert_offsets : i32 [E+1] (output) start of each expert's padded run;
 *                    expert_offsets[E] = padded length
 *   block_expert   : i32 [(T*top_k + E*(block_m-1)) / block_m] (output) local
 *                    expert of each block (-1 if not local, and past the end)
 *   num_post_padded: i32 [1] (output) padded length
 * E <= 1024.  Deterministic: identical inputs give identical outputs.
 */
int lowbit_moe_align(const int32_t *topk_ids, int T, int top_k, int E, int block_m,
                     const int32_t *expert_map, int32_t *sorted_ids, int32_t *expert_offsets,
                     int32_t *block_expert, int32_t *num_post_padded, void *stream);

/*
 * Grouped expert GEMM with 3-bit LUT-codebook weights and MXFP8 activations
 * ("vLLM PR #62759 analysis": sections "Format", "A gather", "Expert
 * parallelism"; numerics of section "Emulation path"):
 *   out[sid][n] = RNE_bf16( sum_k a[row][k] * w_e[n][k] ),  row = sid / a_row_div
 *   a[row][k]   = E4M3(a_e4m3[row][k]) * 2^(a_ue8m0[row][k/32] - 127)
 *   w_e[n][k]   = E4M3(codebook of tile (n/8, k/64))[index] * 2^(tile exponent - 127)
 * for every slot sid < num_valid listed in sorted_ids, where e is the local
 * expert block_expert[] gives for the slot's block.  Slots of experts that are
 * not local (block_expert = -1) get zero rows.  Rows of out that no slot
 * names are not written.  Accumulation is fp32.
 *   fmt            : LOWBIT_LUT3_E4M3
 *   E_local, N, K  : packed blob from lowbit_pack_weights(LOWBIT_LUT3_E4M3,
 *                    E_local, N, K, ...); N % 8 == 0, K % 64 == 0
 *   E              : number of global experts (expert_offsets has E + 1 entries)
 *   a_e4m3/a_ue8m0 : u8 [a_rows][K] and u8 [a_rows][K/32]
 *   a_row_div      : top_k when every routed copy of a token reads the token's
 *                    row (gate/up), 1 when each slot has its own row (down)
 *   sorted_ids, expert_offsets, block_expert : from lowbit_moe_align with the
 *                    same block_m (a multiple of 16)
 *   out            : bf16 [num_valid][N]
 */
int lowbit_moe_gemm(int fmt, int E_local, int N, int K, const void *packed, int E,
                    const uint8_t *a_e4m3, const uint8_t *a_ue8m0, int a_rows, int a_row_div,
                    const int32_t *sorted_ids, const int32_t *expert_offsets,
                    const int32_t *block_expert, int num_valid, int block_m, void *out,
                    void *stream);

/*
 * MXFP8 quantization of bf16 rows (OCP MX as the "vLLM PR #62759 analysis"
 * uses it, section "Format"/"Emulation path": E4M3 elements with one UE8M0
 * scale per 32 consecutive elements).  Per 32-block of a row: e =
 * floor(log2(max |x|)) - 8 (8 = exponent of E4M3's largest value 448),
 * clamped to [-127, 127], 0 for an all-zero block; scale byte = e + 127;
 * element = round-to-nearest-even E4M3 of x / 2^e, saturated at +-448.
 *   x     : bf16 [R][K], 16-byte aligned, K % 32 == 0
 *   q     : u8 (E4M3) [R][K] (output), 8-byte aligned
 *   scale : u8 (UE8M0) [R][K/32] (output)
 * The hidden states go through this before the gate/up grouped GEMM.
 */
int lowbit_mxfp8_quant(const void *x, int R, int K, uint8_t *q, uint8_t *scale, void *stream);

/*
 * SiLU(gate) * up of the gate/up grouped GEMM output, re-quantized to MXFP8
 * for the down GEMM (the expert MLP of the MoE layer; the page's emulation
 * quantizes the activations before each expert GEMM).
 *   gate_up : bf16 [R][2I] (lowbit_moe_gemm output of the stacked gate and up
 *             projections: columns 0..I-1 gate, I..2I-1 up), 16-byte aligned
 *   q, scale: as lowbit_mxfp8_quant for K = I (I % 32 == 0)
 * act = RNE_bf16(SiLU(g) * u) in binary32, SiLU(g) = g / (1 + e^-g) with e^-g
 * evaluated as 2^t, t = -g * log2(e), by a fixed binary32 algorithm (n =
 * rint(t), 2^(t-n) by its Taylor polynomial through degree 7 in Horner form
 * with fused multiply-adds, t clamped to [-100, 100]), then MXFP8 of act.
 */
int lowbit_moe_silu_mul_quant(const void *gate_up, int R, int I, uint8_t *q, uint8_t *scale, void *stream);

/*
 * The gate/up grouped GEMM and the SiLU(gate) * up MXFP8 step in one launch
 * (the expert MLP of the "vLLM PR #62759 analysis", sections "Format" and
 * "Emulation path"): the bytes written equal those of lowbit_moe_gemm with
 * N = 2I into a bf16 [num_valid][2I] buffer followed by
 * lowbit_moe_silu_mul_quant on it, without that buffer.  Slots of experts
 * that are not local read as zero gate/up rows (q = 0, scale = 127).
 *   fmt, E_local, K, packed : as lowbit_moe_gemm with N = 2I (the stacked
 *                    gate and up projections, gate rows first)
 *   E, a_e4m3, a_ue8m0, a_rows, a_row_div, sorted_ids, expert_offsets,
 *   block_expert, num_valid, block_m : as lowbit_moe_gemm
 *   q, scale       : u8 [num_valid][I] and u8 [num_valid][I/32] (outputs),
 *                    rows indexed by slot id; rows no slot names are not written
 * I % 128 == 0 and K <= 4864 (16 activation rows of K bytes fit the 80 KB
 * staging area), else LOWBIT_E_UNSUPPORTED.
 */
int lowbit_moe_gemm_silu_quant(int fmt, int E_local, int I, int K, const void *packed, int E,
                               const uint8_t *a_e4m3, const uint8_t *a_ue8m0, int a_rows, int a_row_div,
                               const int32_t *sorted_ids, const int32_t *expert_offsets,
                               const int32_t *block_expert, int num_valid, int block_m, uint8_t *q,
                               uint8_t *scale, void *stream);

/*
 * Router-weighted combine of the routed experts' outputs:
 *   y[t][h] = RNE_bf16( sum_{j < top_k} topk_weights[t][j] * expert_out[t*top_k + j][h] )
 * in fp32, j ascending.  Slots of experts that are not local have zero rows
 * (lowbit_moe_gemm) and add nothing.
 *   expert_out   : bf16 [T*top_k][H], 16-byte aligned; H % 8 == 0
 *   topk_weights : f32 [T][top_k]
 *   y            : bf16 [T][H] (output), 16-byte aligned
 */
int lowbit_moe_combine(const void *expert_out, const float *topk_weights, int T, int top_k, int H, void *y,
                       void *stream);

/* Workspace bytes of lowbit_moe_layer (0 for an invalid shape). */
size_t lowbit_moe_layer_workspace_bytes(int T, int top_k, int E, int H, int I, int block_m);

/*
 * One whole MoE layer with 3-bit LUT-codebook experts and MXFP8 activations
 * ("vLLM PR #62759 analysis": format, A gather, expert parallelism, emulation
 * path), enqueued as six kernels: MXFP8 of x, routing alignment, gate/up
 * grouped GEMM, SiLU(gate) * up with MXFP8, down grouped GEMM, combine.
 *   w13      : lowbit_pack_weights(LOWBIT_LUT3_E4M3, E_local, 2I, H, ...) --
 *              each expert's gate (rows 0..I-1) and up (rows I..2I-1) stacked
 *   w2       : lowbit_pack_weights(LOWBIT_LUT3_E4M3, E_local, H, I, ...)
 *   E        : global experts (routing ids are in [0, E)); expert_map as in
 *              lowbit_moe_align (NULL = all local, which needs E <= E_local:
 *              else LOWBIT_E_INVALID_ARG, as slots would name experts that
 *              w13 and w2 do not hold)
 *   x        : bf16 [T][H] hidden states, 16-byte aligned; H % 64 == 0, I % 64 == 0
 *   topk_ids : i32 [T][top_k]; topk_weights: f32 [T][top_k]
 *   y        : bf16 [T][H] (output), 16-byte aligned
 *   workspace: >= lowbit_moe_layer_workspace_bytes(T, top_k, E, H, I, block_m),
 *              256-byte aligned; block_m a multiple of 16
 */
int lowbit_moe_layer(const void *w13, const void *w2, int E_local, int E, int H, int I, const void *x,
                     const int32_t *topk_ids, const float *topk_weights, int T, int top_k, const int32_t *expert_map,
                     int block_m, void *y, void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
