// Host-side launchers of the HIP kernels (each defined in the .hip file that
// holds its kernels). All launches are asynchronous on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_fp4.h"

namespace moe {

struct BlobHeader;
// Routing; block 0 also clears `misc` and writes the forward's status word
// (0, or MOE_ERR_INVALID when the blob's header differs from `expect`).
hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* ids, float* topw,
                        uint32_t* misc, const void* blob, const BlobHeader& expect,
                        uint32_t* status, hipStream_t s);
bool small_route_permute(int R, int E);
hipError_t launch_permute_small(const int32_t* ids, int R, int E, int32_t* counts,
                                int32_t* offsets, int32_t* tiles, int32_t* r2r, int32_t* rt2row,
                                hipStream_t s);
hipError_t launch_permute(const int32_t* ids, int R, int E, int nblk, int32_t* bhist,
                          int32_t* bbase, int32_t* counts, int32_t* offsets, int32_t* tiles,
                          int32_t* r2r, int32_t* rt2row, hipStream_t s);

// Row quantizers. kind: 0 NVFP4 one global scale (from the amax: the largest
// of amax_slots words amax_stride apart from amax_slot, each the bits of a
// non-negative partial maximum), 1 NVFP4 one global scale per row, 2 MXFP8. in_bf16: input
// rows are bf16 (else fp32). deq (NVFP4 only, may be null): fp16 [rows][cols]
// of code * sf.
// QK_NV_ROW_4O6: one global scale amax / (6 * 256) per row and the 4-over-6
// block choice (nvfp4_block_4o6).
enum QuantKind { QK_NV_TENSOR = 0, QK_NV_ROW = 1, QK_MX = 2, QK_NV_ROW_4O6 = 3 };
// Max |v| into the nslots words stride apart from amax_slot (already cleared).
hipError_t launch_amax(const void* v, int in_bf16, size_t n, uint32_t* amax_slot, int nslots,
                       int stride, hipStream_t s);
hipError_t launch_quant_rows(const void* v, int in_bf16, int rows, int cols, int kind,
                             const uint32_t* amax_slot, int amax_slots, int amax_stride, uint8_t* codes,
                             uint8_t* scales, float* g, uint16_t* deq, hipStream_t s);

// NVFP4 (packed codes, E4M3 per 16) of n consecutive elements re-blocked to
// MXFP4 (packed codes, E8M0 per 32); status: skip when it points to non-zero.
hipError_t launch_reblock_mxfp4(const uint8_t* nv_codes, const uint8_t* nv_scales, size_t n,
                                uint8_t* mx_codes, uint8_t* mx_scales, const uint32_t* status,
                                hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
// status: the forward's status word (skip all work when not 0), or null.
hipError_t launch_finalize(const void* O, int is_bf16, const int32_t* rt2row, const float* w,
                           int T, int K, int H, uint16_t* y, const uint32_t* status,
                           hipStream_t s);

// Weight preparation (one matrix family W[E][N][K] at a time).
hipError_t launch_prep_amax(const float* w, int E, size_t per_expert, uint32_t* amax, hipStream_t s);
hipError_t launch_prep_nvfp4(const float* w, int E, int N, int K, int swiglu_I,
                             const uint32_t* amax, float* g, uint8_t* codes, uint8_t* scales,
                             hipStream_t s);
// NVFP4-quantized with the expert's global scale, then re-blocked to MXFP4.
hipError_t launch_prep_mxfp4(const float* w, int E, int N, int K, int swiglu_I,
                             const uint32_t* amax, float* g, uint8_t* codes, uint8_t* scales,
                             hipStream_t s);
hipError_t launch_prep_mxfp8(const float* w, int E, int N, int K, int swiglu_I, uint8_t* codes,
                             uint8_t* scales, hipStream_t s);

// Grouped GEMMs.
// AB_FP4: MXFP4 operands (re-blocked NVFP4) on the block-scaled matrix cores.
enum GemmAB { AB_F16_NV = 0, AB_BF16_NV = 1, AB_FP8 = 2, AB_FP4 = 3 };
enum GemmEpi { EPI_FC1 = 0, EPI_FC2 = 1 };
// How FC2 finishes the layer: store O for the finalize kernel, or store O and
// let the block that completes a token's K routes for its columns reduce them
// into y (arrival counts).
enum GemmFuse { FUSE_NONE = 0, FUSE_ARRIVE = 1 };

struct GemmArgs {
    // A: activations. gather != 0: A row of permuted row r is row_to_route[r] / topk.
    const void* a;
    const uint8_t* a_scales;  // MXFP8 / MXFP4 E8M0 [rows][Kdim/32]
    const float* a_g;         // NVFP4 activation global scale(s), null for W4A16
    int a_g_per_row;
    int gather;
    const int32_t* row_to_route;
    int topk;
    // B: prepared weights of this GEMM
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* b_g;  // per-expert NVFP4 global scale, null for MXFP8
    int N, Kdim;
    // tile list
    const int32_t* offsets;
    const int32_t* tiles;  // [E+1] for this BM
    int E;
    int mt_max;
    int resident;  // set by the launcher: blocks of this kernel the device holds at once
    // epilogue
    int act, on_input, I;
    const float* topw;
    float* out_f32;      // FC1 NVFP4: fp32 [R][I] before quantization; FC2: O [R][N]
    uint16_t* out_bf16;  // FC1 W4A16: bf16 [R][I]
    uint8_t* a2_codes;   // FC1 MXFP8: FC2-input E4M3 codes [R][I], quantized here
    uint8_t* a2_scales;  //            and their E8M0 block scales [R][I/32]
    uint32_t* amax_slot; // FC1: kAmaxSlots partial maxima of the FC2 input, kAmaxStride apart (NVFP4 per-tensor)
    int fused;           // FC2: FUSE_NONE or FUSE_ARRIVE
    uint32_t* arrive;    // FC2 fused by arrival counts: [T][N / block columns] counters, zero on entry
    const int32_t* rt2row;  //   route (t, k) -> its row of O
    uint16_t* y;         //   bf16 output [T][N]
    const uint32_t* status;  // the forward's status word: blocks exit when it is not 0
};

// The forward as the C ABI runs it (moe_api.cpp): argument checks other than
// the workspace's, the workspace a shape needs, and the launch sequence on a
// workspace of at least that size. report_error sets moe_last_error().
int forward_checked(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                    const uint16_t* x, const float* logits, int32_t T, int32_t K, int32_t mode,
                    int32_t act, int32_t router_weight_on_input, int32_t deterministic_finalize,
                    const uint16_t* y);
size_t forward_workspace_bytes(const moe_dims* d, int32_t T, int32_t K, int32_t mode);
int enqueue_forward(const moe_dims* d, const void* prepared, const uint16_t* x,
                    const float* logits, int32_t T, int32_t K, int32_t mode, int32_t act,
                    int32_t router_weight_on_input, int32_t deterministic_finalize,
                    void* workspace, uint16_t* y, hipStream_t stream);
int report_error(int code, const char* msg);

// t0/t1: optional events recorded at the kernel's start and end.
hipError_t launch_gemm(int ab, int epi, int bm_index, const GemmArgs& a, hipStream_t s,
                       hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

}  // namespace moe
