/*
 * moe_fp4: one block-scaled Mixture-of-Experts layer forward on an AMD MI355X
 * (gfx950), as a C ABI.
 *
 * What is computed (MegaMoE post, flashinfer.ai, "The problem" and "Our
 * approach"; FlashInfer PR #4366, "Description"; newruntime summary of
 * FlashInfer PR #5319, "Retrieval answer"):
 *
 *   S1 route     per token, the top-K of E router logits (descending, ties to
 *                the lower expert id) and weights p = softmax over the chosen K;
 *   S2 permute   routes r = t*K + k grouped by expert, tokens ascending inside a
 *                group (expert-contiguous grouped-GEMM order);
 *   S3 quantize  FC1 input: NVFP4 (E2M1 values, E4M3 scale per 16 elements,
 *                FP32 global scale per tensor or per token), MXFP8 (E4M3 values,
 *                E8M0 scale per 32) or none (W4A16: bf16 activations);
 *   S4 FC1       grouped GEMM h = x W1_e^T per route;
 *   S5           SwiGLU (silu(gate) * up) or ReLU2 (max(h,0)^2); with input-side
 *                placement the result is multiplied by p in FP32; then the FC2
 *                input is quantized (W4A4: NVFP4 per tensor or per route; MXFP8)
 *                or stored as bf16 (W4A16);
 *   S6 FC2       grouped GEMM o = a W2_e^T per route;
 *   S7 finalize  y[t] = sum_k w[t,k] o[route t*K+k] with w = p (output side) or
 *                1 (input side, the weight was applied before FC2), in fixed k
 *                order, either as its own kernel (deterministic) or fused into
 *                FC2 (the FC2 block completing a token's K routes for its
 *                columns reduces them; the same bits).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are device pointers (hipMalloc'd or equivalent), row-major,
 *    owned by the caller. The library never allocates device or host memory
 *    and keeps no per-call state, except the optional stage timing below.
 *  - Every call only enqueues work on `stream` and returns; no host<->device
 *    synchronisation except in moe_check_prepared, moe_forward_status and
 *    moe_stage_times (and in moe_forward while stage timing is on, see
 *    moe_stage_timing).
 *  - Argument checks all run before any launch; on failure nothing is
 *    enqueued and a moe_status other than MOE_OK is returned, with a message in
 *    moe_last_error().
 *  - Device pointers must be 256-byte aligned where noted, else 16-byte aligned.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_W4A4_TENSOR = 0, /* NVFP4 weights and activations, one activation global scale per tensor */
    MOE_W4A4_TOKEN = 1,  /* NVFP4 weights and activations, one activation global scale per row    */
    MOE_W4A16 = 2,       /* NVFP4 weights, bf16 activations                                         */
    MOE_MXFP8 = 3,       /* MXFP8 (E4M3 + E8M0 per 32) weights and activations                      */
    /* NVFP4 weights; activations per token under the "4-over-6" contract
     * (FlashInfer PR #4366, "Performance benchmark", named there by its
     * switches only; this library's reading): global scale amax / (6*256) per
     * row, and per 16-block the block max mapped to 6 or to 4, whichever gives
     * the smaller sum of squared errors (fp64, element order; ties to 6). The
     * GEMMs consume the result like any NVFP4 operand. */
    MOE_W4A4_TOKEN_4O6 = 4,
    /* NVFP4 W4A4 with per-token activation scales, GEMMs on the block-scaled
     * FP4 matrix cores: both operands re-blocked from NVFP4 (E4M3 per 16) to
     * MXFP4 (E8M0 per 32) by the OCP MX rule, which rounds each element a second
     * time (about 11-12 % relative Frobenius difference per GEMM operand against
     * the NVFP4 values); the FP32 global scales are applied in the epilogues.
     * Opt-in, for callers that accept that error; needs an MOE_FMT_MXFP4 blob. */
    MOE_W4A4_TOKEN_MXFP4 = 5
} moe_mode;

typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 } moe_act;
/* MOE_FMT_MXFP4: the weights NVFP4-quantized (per-expert FP32 global scale)
 * and re-blocked to MXFP4, in the FP4 matrix-core layout (mode 5 only). */
typedef enum { MOE_FMT_NVFP4 = 0, MOE_FMT_MXFP8 = 1, MOE_FMT_MXFP4 = 2 } moe_wfmt;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* null/misaligned pointer, bad size or enum                  */
    MOE_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (e.g. H % 128 != 0)       */
    MOE_ERR_WORKSPACE = 3,   /* workspace or prepared buffer too small                      */
    MOE_ERR_HIP = 4          /* a HIP call failed; moe_last_error() has hipGetErrorString */
} moe_status;

/* Layer geometry. N1 = 2*I for SwiGLU (rows [0,I) gate, [I,2I) up), I for
 * ReLU2. Limits: 1 <= E <= 1024; H and I positive multiples of 128 (the K
 * extent of one weight micro-tile); H, I <= 32768. */
typedef struct {
    int32_t E, H, I;
    int32_t act;  /* moe_act  */
    int32_t wfmt; /* moe_wfmt */
} moe_dims;

/* Size in bytes of the prepared-weight blob for `d` (0 if `d` is invalid). */
size_t moe_prepared_bytes(const moe_dims* d);

/* S0 (off the timed path): quantize and reorder the weights.
 * Weights arrive in the standard checkpoint layout and the library quantizes
 * and reorders them itself (MegaMoE post, "Usage"); one NVFP4 blob serves the
 * W4A4 and W4A16 modes (newruntime summary of PR #5319, title).
 *   w1: [E][N1][H] fp32, w2: [E][H][I] fp32 (device).
 *   prepared: device buffer of at least moe_prepared_bytes(d) bytes, 256-byte
 *   aligned; written entirely (header, per-expert FP32 global scales
 *   g = amax / (6*448) per expert per matrix for NVFP4, codes and scales in the
 *   kernel-native layout described in the design notes). Immutable afterwards;
 *   it may be shared by concurrent forwards. */
int moe_prepare_weights(const moe_dims* d, const float* w1, const float* w2, void* prepared,
                        size_t prepared_bytes, hipStream_t stream);

/* Synchronous check that a device blob's header matches `d` (reads 256 bytes
 * to the host; not for use under graph capture). */
int moe_check_prepared(const moe_dims* d, const void* prepared, hipStream_t stream);

/* Workspace bytes needed by moe_forward for up to T_max tokens and top-K. */
size_t moe_workspace_bytes(const moe_dims* d, int32_t T_max, int32_t K, int32_t mode);

/* S1..S7: one layer forward.
 *   prepared: blob from moe_prepare_weights with the same `d` (NVFP4 blob for
 *             modes 0..2, MXFP8 blob for mode 3), prepared_bytes its size in
 *             bytes (MOE_ERR_WORKSPACE below moe_prepared_bytes(d)). The blob's
 *             header is compared with `d` on the device by the forward's first
 *             kernel: on a difference (a blob prepared for other dimensions,
 *             activation or format) the forward reads no weights, leaves y
 *             unwritten and sets its status word to MOE_ERR_INVALID, which
 *             moe_forward_status returns.
 *   x:        [T][H] bf16 bit patterns.            logits: [T][E] fp32 (finite).
 *   T >= 1, 1 <= K <= min(E, 64), T*K*max(H, I)*2 < 4 GiB (MOE_ERR_UNSUPPORTED
 *   otherwise: the GEMMs address activation rows with 32-bit offsets).
 *   act must equal d->act. router_weight_on_input: 0 = output side (finalize
 *   weights p), 1 = input side (p applied to the FP32 activation output before
 *   the FC2-input quantization or bf16 store; finalize weights 1).
 *   deterministic_finalize: 1 = FC2 stores the permuted output O in fp32, then
 *   a fixed-order unpermute+reduce in fp32 (bit-identical run to run);
 *   0 = the finalize fused into the FC2 kernel: the FC2 block that completes
 *   a token's K routes for its output columns reduces them, in the same order
 *   and arithmetic, so the output is the same bits as with 1.
 *   MXFP8 quantizes the FC2 input in the FC1 epilogue (no fp32 copy).
 *   workspace: >= moe_workspace_bytes(d, T, K, mode) bytes, 256-byte aligned;
 *   afterwards it holds the forward's status word (first 4 bytes) and the
 *   intermediate views listed by moe_workspace_view.
 *   y: [T][H] bf16 bit patterns (output). */
int moe_forward(const moe_dims* d, const void* prepared, size_t prepared_bytes, const uint16_t* x,
                const float* logits, int32_t T, int32_t K, int32_t mode, int32_t act,
                int32_t router_weight_on_input, int32_t deterministic_finalize, void* workspace,
                size_t workspace_bytes, uint16_t* y, hipStream_t stream);

/* moe_forward for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same forward, on a
 * workspace that is a device array inside the library (64 MiB; each GPU the
 * library runs on holds its own copy until the process ends) instead of a
 * caller buffer; the caller still passes the inputs and y. Arguments, their
 * checks and error codes as for moe_forward; a shape whose workspace
 * (moe_workspace_bytes) exceeds 64 MiB returns MOE_ERR_WORKSPACE before any
 * launch. No call allocates memory; the first call on a device looks up the
 * array's device address (hipGetSymbolAddress) with that device current, so
 * `stream` must belong to the current device. All calls on one GPU share the
 * array, which keeps the last call's contents (every forward rewrites what it
 * reads): forwards that overlap in time on one GPU, on different streams or
 * host threads, race and must be serialised by the caller. The status word
 * of the device-side blob check lives in that array and is not readable. */
int moe_forward_noalloc(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                        const uint16_t* x, const float* logits, int32_t T, int32_t K,
                        int32_t mode, int32_t act, int32_t router_weight_on_input,
                        int32_t deterministic_finalize, uint16_t* y, hipStream_t stream);

/* Status word of the last forward enqueued on `workspace` (synchronous: waits
 * for `stream`, then reads 4 bytes): *status = 0 after a forward whose blob
 * header matched its dimensions, MOE_ERR_INVALID otherwise (y was then not
 * written). Not for use under graph capture. */
int moe_forward_status(const void* workspace, int32_t* status, hipStream_t stream);

/* S7 alone (unfused finalize, as in PR #5319): y[t][j] = sum_{k<K} w[t][k] *
 * permuted_out[route_to_row[t*K+k]][j], accumulated in fp32 in k order and
 * rounded once to bf16. Always the fixed-order (deterministic) reduction: the
 * fused variant exists only inside moe_forward, where it is the FC2
 * epilogue's scatter-add.
 *   permuted_out: [R][H] fp32 (out_is_bf16 = 0) or bf16 (1), R = T*K.
 *   route_to_row: [T*K] int32, each in [0, R).  weights: [T][K] fp32 or NULL
 *   for unit weights (input-side placement).  y: [T][H] bf16. */
int moe_finalize(const void* permuted_out, int32_t out_is_bf16, const int32_t* route_to_row,
                 const float* weights, int32_t T, int32_t K, int32_t H, uint16_t* y,
                 hipStream_t stream);

/* Standalone block quantizer (the S3/S5 quantizer as a library call).
 *   v: [rows][cols] fp32; kind: 0 = NVFP4 one global scale for the whole
 *   matrix, 1 = NVFP4 one global scale per row, 2 = MXFP8, 3 = NVFP4 per row
 *   with the 4-over-6 block choice (see MOE_W4A4_TOKEN_4O6).
 *   codes: NVFP4 [rows][cols/2] (two E2M1 codes per byte, even element in the
 *   low nibble); MXFP8 [rows][cols] E4M3.  scales: NVFP4 [rows][cols/16] E4M3;
 *   MXFP8 [rows][cols/32] E8M0.  g: NVFP4 [1] or [rows] fp32 (unused for MXFP8).
 *   scratch: 256 bytes of device memory (cleared by the call).
 *   cols % 32 == 0. */
int moe_quantize(const float* v, int32_t rows, int32_t cols, int32_t kind, uint8_t* codes,
                 uint8_t* scales, float* g, void* scratch, hipStream_t stream);

/* Location of an intermediate inside the workspace (for inspection/parity):
 *   0 topk_ids [T][K] i32        1 topk_w [T][K] f32
 *   2 counts [E] i32             3 offsets [E+1] i32
 *   4 row_to_route [R] i32       5 route_to_row [R] i32
 *   6 x codes                    7 x scales               8 x global scale(s) f32
 *   9 FC2 input, fp32 before quantization [R][I] (W4A4) or bf16 (W4A16)
 *   10 FC2-input codes           11 FC2-input scales      12 FC2-input global scale(s)
 *   13 permuted FC2 output O [R][H] f32 (either finalize)
 *   14/15 x re-blocked to MXFP4: codes [T][H/2], E8M0 scales [T][H/32] (mode 5)
 *   16/17 FC2 input re-blocked to MXFP4: codes [R][I/2], scales [R][I/32] (mode 5)
 * Returns MOE_ERR_INVALID for a view the mode does not produce. */
int moe_workspace_view(const moe_dims* d, int32_t T, int32_t K, int32_t mode, int32_t view_id,
                       size_t* offset, size_t* bytes);

/* Optional per-stage timing with HIP events recorded on the forward's stream
 * around each stage (not to be enabled under graph capture). While it is on,
 * forwards take a process-wide lock for their launches (forwards from several
 * host threads serialise), and a forward waits for the events of the oldest
 * of the last 128 timed forwards before reusing them. moe_stage_times
 * synchronises, returns the summed milliseconds per stage since the last
 * reset in ms[0..n) and the number of timed forwards, and resets. Stage ids:
 * 0 route, 1 permute, 2 quantize x, 3 FC1, 4 FC2-input quantize, 5 FC2,
 * 6 finalize. */
int moe_stage_timing(int32_t enable);
int moe_stage_times(float* ms, int32_t n, int32_t* forwards);

/* Message for the last non-OK status returned on this thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP4_H */
