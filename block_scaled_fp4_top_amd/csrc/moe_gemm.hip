// S4/S6 grouped GEMMs with fused epilogues.
//
// C[r][n] = sum_k A[row(r)][k] * W_e[n][k] for the rows r of one expert e.
// A block of NW waves (4, or 8 for wide tiles) owns an M-tile of BM rows of
// one expert (from the device tile list built by the permutation) and NW*WN
// strips of 16 output columns; wave w owns strips [w*WN, w*WN + WN) and all
// rows of the tile.
//  - A (activations) is staged through LDS per 128-deep K step by direct
//    global->LDS loads: f16/bf16 as 8 rows x one 128-byte line per load, in an
//    XOR-swizzled layout whose operand reads are free of bank conflicts; fp8
//    in the operand's own order (16 rows x 64 bytes per load).
//  - B (weights) is read straight from HBM into registers: the prepared blob
//    stores every 16 x 128 micro-tile as the register image of a 64-lane wave,
//    so each load is a contiguous 1 KB (NVFP4) or 2 KB (MXFP8) per wave.
//  - P-stage software pipeline: the loads of the next P-1 steps are in flight
//    while one step is multiplied (P LDS buffers for A, P register sets for B).
//  - Small tiles (decode): one contiguous range of tiles per XCD, and, when
//    every block is resident at once, wave priorities that let the blocks
//    furthest behind in their K loop issue first.
//  - NVFP4: exact dequantization code * sf in registers (hardware fp4
//    converter at unit scale, then the E4M3 block scale: a packed fp16 multiply
//    for fp16 operands, an fp32 multiply for bf16; the product has at most 6
//    significant bits, so it is exact), then v_mfma_f32_16x16x32_{f16,bf16}.
//    The E4M3 block-16 scales do not fit the matrix cores' E8M0 block-32
//    scaling, so the scale is applied on the VALU.
//  - MXFP8: v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0 block scales as
//    the per-lane scale operands; no dequantization at all.
//  - Epilogue: global scales (g_a * g_w), then FC1: SwiGLU/ReLU2, optional
//    input-side router weight in FP32, then the FC2 input: fp32 (+ partial
//    maxima of |value| for the per-tensor global scale) for
//    NVFP4, bf16 for W4A16, or MXFP8 codes and scales quantized in place;
//    FC2: store of the permuted output O, and for the fused finalize the
//    reduction of every token whose K routes this block completes.
#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "moe_internal.h"
#include "moe_kernels.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_pair(float lo, float hi, bool bf16) {
    if (bf16) return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// SiLU(g) * u with the hardware exp2 and reciprocal (a few ulp in fp32).
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Epilogue: acc[ms][s][i] holds C for row ms*16 + 4*(lane/16) + i of the
// tile and column strip gs0 + s, lane % 16.
// Max over the 16 lanes of each DPP row (lanes with equal lane/16), by
// rotations within the row: every lane ends with the row's max.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
    return v;
}

template <int AB, int MS, int WN, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, f32x4 (&acc)[MS][WN], int e,
                                              int row0, int rows, const int* s_arow, int gs0,
                                              int lane) {
    const float gw = p.b_g ? p.b_g[e] : 1.0f;
    const int c16 = lane & 15;
    if constexpr (EPI == EPI_FC1 && AB == AB_FP8) {
        // MXFP8: the wave holds 32 consecutive FC2-input columns of each row
        // per pair of output strips (lanes with equal lane/16 share a row), so
        // it quantizes whole 32-element blocks: block max over the 16 lanes of
        // the row group, E8M0 exponent, E4M3 codes. All lanes compute (rows
        // past the group hold finite values of a re-read row); stores are
        // guarded.
        constexpr int OS = WN / 2;  // SwiGLU output strips; ReLU2 has WN
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ms * 16 + 4 * (lane >> 4) + i;
                const int row = row0 + min(m, rows - 1);
                const float pw = p.on_input ? p.topw[p.row_to_route[row]] : 1.0f;
                float a[WN];
                int nout;
                if (p.act == MOE_ACT_SWIGLU) {
                    nout = OS;
#pragma unroll
                    for (int u = 0; u < OS; ++u) {
                        a[u] = silu_mul(acc[ms][2 * u][i] * gw, acc[ms][2 * u + 1][i] * gw);
                        if (p.on_input) a[u] = a[u] * pw;
                    }
                } else {
                    nout = WN;
#pragma unroll
                    for (int u = 0; u < WN; ++u) {
                        const float h = acc[ms][u][i] * gw;
                        a[u] = h > 0.0f ? h * h : 0.0f;
                        if (p.on_input) a[u] = a[u] * pw;
                    }
                }
                const int col0 = (p.act == MOE_ACT_SWIGLU ? gs0 >> 1 : gs0) * 16;
#pragma unroll
                for (int b = 0; b < WN / 2; ++b) {
                    if (2 * b + 1 >= nout) break;  // the host launches whole blocks only
                    float ab = fmaxf(fabsf(a[2 * b]), fabsf(a[2 * b + 1]));
                    ab = row16_max(ab);
                    const int X = mxfp8_exponent(ab);
                    const float inv = mxfp8_inv_scale(X);
                    if (m < rows) {
                        const size_t o = (size_t)(row0 + m) * p.I + col0 + 32 * b + c16;
                        const uint32_t c = e4m3_code2(__fmul_rn(a[2 * b], inv), __fmul_rn(a[2 * b + 1], inv));
                        p.a2_codes[o] = (uint8_t)c;
                        p.a2_codes[o + 16] = (uint8_t)(c >> 8);
                        if (c16 == 0)
                            p.a2_scales[(size_t)(row0 + m) * (p.I / 32) + (col0 >> 5) + b] = (uint8_t)(X + 127);
                    }
                }
            }
        }
    } else {
    float amax = 0.0f;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = ms * 16 + 4 * (lane >> 4) + i;
            if (m >= rows) continue;
            const int row = row0 + m;
            const float ga = p.a_g ? p.a_g[p.a_g_per_row ? s_arow[m] : 0] : 1.0f;
            const float sc = ga * gw;
            if (EPI == EPI_FC1) {
                const float pw = p.on_input ? p.topw[p.row_to_route[row]] : 1.0f;
                if (p.act == MOE_ACT_SWIGLU) {
#pragma unroll
                    for (int u = 0; u < WN / 2; ++u) {
                        float a = silu_mul(acc[ms][2 * u][i] * sc, acc[ms][2 * u + 1][i] * sc);
                        if (p.on_input) a = a * pw;
                        const int col = ((gs0 + 2 * u) >> 1) * 16 + c16;
                        if (p.out_bf16) p.out_bf16[(size_t)row * p.I + col] = bf16_rne(a);
                        else p.out_f32[(size_t)row * p.I + col] = a;
                        amax = fmaxf(amax, fabsf(a));
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < WN; ++s) {
                        const float h = acc[ms][s][i] * sc;
                        float a = h > 0.0f ? h * h : 0.0f;
                        if (p.on_input) a = a * pw;
                        const int col = (gs0 + s) * 16 + c16;
                        if (p.out_bf16) p.out_bf16[(size_t)row * p.I + col] = bf16_rne(a);
                        else p.out_f32[(size_t)row * p.I + col] = a;
                        amax = fmaxf(amax, fabsf(a));
                    }
                }
            } else {
                if (p.fused == FUSE_ARRIVE) {
                    // device scope: rows are read back by a block on any XCD
                    float* o = p.out_f32 + (size_t)row * p.N + gs0 * 16 + c16;
#pragma unroll
                    for (int s = 0; s < WN; ++s)
                        __hip_atomic_store(o + s * 16, acc[ms][s][i] * sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
#pragma unroll
                    for (int s = 0; s < WN; ++s)
                        p.out_f32[(size_t)row * p.N + (gs0 + s) * 16 + c16] = acc[ms][s][i] * sc;
                }
            }
        }
    }
    if (EPI == EPI_FC1 && p.amax_slot) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const int slot = (blockIdx.x * 4 + (threadIdx.x >> 6)) % kAmaxSlots;
        if (lane == 0) atomicMax(p.amax_slot + slot * kAmaxStride, f2u(amax));
    }
    }
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 l (lds_base is uniform across the wave).
__device__ __forceinline__ void lds_load16(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)gsrc,
        (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)gsrc,
        (void __attribute__((address_space(3)))*)lds_base, 4, 0, 0);
}

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding and all LDS operations are done (export counter not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Orders the first use of a loaded register after the preceding wait: the
// empty volatile asm "redefines" the value, so no instruction reading it can
// be scheduled above the asm (and volatile asm keeps its order).
__device__ __forceinline__ void reg_fence(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void reg_fence(u32x4& v) { asm volatile("" : "+v"(v)); }

// f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time indexes,
// e.g. for instruction operands that must be immediates).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier without the fence __syncthreads() carries (that fence
// drains every outstanding load, which would serialise the pipeline). The
// caller waits for the loads that must have landed; the memory clobber keeps
// the compiler from moving memory accesses across.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Fused finalize by arrival counts, after a block has stored its O tile
// (rows of one expert's M-tile, the BN columns of N-block nb). Each route of
// the tile counts itself in on its token's counter for this N-block; the
// route whose increment completes the count (the K-th) hands its token to the
// block, which then reduces the token's K rows of O over these BN columns in
// the order k = 0..K-1, each term weighted by the router weight (output side),
// in fp32 with one rounding to bf16 at the end. That is the deterministic
// finalize's arithmetic in its order, so both variants give the same bits, and
// no fp32 atomics touch the output: a token's columns are written once, by
// whichever block arrives last.
// The wide tiles keep their block order, which gives each XCD a contiguous
// range of (N-block, M-tile) pairs: an N-block-major order over the whole
// chip ran this FC2 1.5x slower at 16k tokens (5.57 against 3.79 ms).
// Visibility across XCDs (each has its own L2) uses device-scope accesses on
// the O rows themselves rather than device-scope fences, which write back or
// invalidate a whole L2 (measured: 3x slower FC2 at 16k tokens, 9x on the
// decode tiles): the epilogue stores O with device scope, so each store is
// complete only once it is visible device-wide; every wave waits for its
// stores before the barrier that precedes the block's counter increments; and
// the block that completes a count reads the rows back with device-scope
// loads, issued after its increment has returned.
template <int NW, int BN>
__device__ __forceinline__ void arrive_finalize(const GemmArgs& p, int nb, int row0, int rows,
                                                int* s_list, int* s_n) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.topk, NB = p.N / BN;
    wait_vmcnt<0>();  // this wave's O stores are complete
    __syncthreads();  // ... and every wave's; s_n was zeroed before the main loop
    for (int m = tid; m < rows; m += NW * 64) {
        const int t = p.row_to_route[row0 + m] / K;
        const uint32_t old = __hip_atomic_fetch_add(p.arrive + (size_t)t * NB + nb, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(K - 1)) s_list[atomicAdd(s_n, 1)] = t;
    }
    __syncthreads();
    const int n = *s_n;
    constexpr int CPL = BN / 64;  // columns per lane: lane + 64 j, coalesced per load
    const float* ob = p.out_f32 + (size_t)nb * BN + lane;  // this N-block's columns of O
    const int c0 = nb * BN + lane;
    // two tokens per round when K <= 32 (lanes 32 + k hold the second one's
    // routes): the loads of up to 8 routes of both tokens are issued
    // together, then each token is summed in k order (on the decode tiles,
    // whose blocks all run at once, this tail is latency)
    const int TB = K <= 32 ? 2 : 1;
    for (int j = TB * wave; j < n; j += TB * NW) {
        const bool two = TB == 2 && j + 1 < n;
        const int t0 = s_list[j], t1 = two ? s_list[j + 1] : t0;
        const int k = TB == 2 ? (lane & 31) : lane;  // route of this lane
        const int tl = lane < 32 ? t0 : t1;
        int my_row = 0;
        float my_w = 1.0f;
        if (k < K && (TB == 1 || lane < 32 || two)) {
            my_row = p.rt2row[(size_t)tl * K + k];
            if (!p.on_input) my_w = p.topw[(size_t)tl * K + k];
        }
        float a0[CPL], a1[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) a0[c] = a1[c] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            float q0[8][CPL], q1[8][CPL];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k0 + u < K) {
                    const float* o = ob + (size_t)__builtin_amdgcn_readlane(my_row, k0 + u) * p.N;
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        q0[u][c] = __hip_atomic_load(o + 64 * c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (two) {
                        const float* o1 = ob + (size_t)__builtin_amdgcn_readlane(my_row, 32 + k0 + u) * p.N;
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            q1[u][c] = __hip_atomic_load(o1 + 64 * c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k0 + u < K) {
                    const float w0 = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), k0 + u));
#pragma unroll
                    for (int c = 0; c < CPL; ++c) a0[c] = __fmaf_rn(w0, q0[u][c], a0[c]);
                    if (two) {
                        const float w1 = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), 32 + k0 + u));
#pragma unroll
                        for (int c = 0; c < CPL; ++c) a1[c] = __fmaf_rn(w1, q1[u][c], a1[c]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) p.y[(size_t)t0 * p.N + c0 + 64 * c] = bf16_rne(a0[c]);
        if (two) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) p.y[(size_t)t1 * p.N + c0 + 64 * c] = bf16_rne(a1[c]);
        }
    }
}

// Grouped GEMM tile kernel. P-stage software pipeline over 128-deep K steps:
// while step kt is multiplied, the loads of steps kt+1 .. kt+P-1 are in
// flight (A into P rotating LDS buffers by direct loads, B into P rotating
// register sets). Every wave issues the same number L of loads per step
// (padding loads target a scratch LDS area), so "step kt has landed" is the
// wait vmcnt <= L*(P-2) followed by a barrier.
template <int AB, int BM, int WN, int EPI, int P, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs p) {
    constexpr bool F8 = AB == AB_FP8;
    constexpr bool F4 = AB == AB_FP4;
    constexpr bool SC = F8 || F4;  // block-scaled matrix core (E8M0 scale per 32)
    constexpr int A_ROW = F8 ? 128 : (F4 ? 64 : 256);  // bytes of one A row per K step
    constexpr int A_TILE = BM * A_ROW;
    __shared__ __attribute__((aligned(1024))) uint8_t sA[P][A_TILE];
    // A scales (fp8, fp4): one wave-wide 4-byte direct load per step writes 64
    // words, so each buffer holds at least 64 rows' words even for BM < 64.
    __shared__ __attribute__((aligned(256))) uint32_t sAsc[P][SC ? (BM > 64 ? BM : 64) : 1];
    __shared__ __attribute__((aligned(1024))) uint8_t sJunk[1024];
    __shared__ int s_arow[BM];
    __shared__ int s_narrive;  // fused finalize by arrival counts: tokens this block completes

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    // the forward's status word, loaded here and tested after the tile lookup
    // so that its latency overlaps the lookup's loads
    const uint32_t status = p.status ? *p.status : 0u;
    // Block order. Blocks are dealt round-robin over the 8 XCDs (each with its
    // own L2) and the grid is a multiple of 8, so blockIdx % 8 names the XCD.
    //  - Wide tiles: M-tile fastest (across experts), then N-block, in
    //    consecutive positions per XCD. Each XCD sweeps all M-tiles for its own
    //    N-blocks: the blocks it runs at a time share one N-block's weight
    //    columns in its L2 (re-read by the M-tiles of an expert), and the eight
    //    XCDs walk the A rows in step, so the last-level cache serves most A
    //    re-reads.
    //  - Small tiles (every weight is read once): the active (M-tile, N-block)
    //    pairs, N-block fastest, are cut into 8 contiguous ranges, one per XCD.
    //    All N-blocks of an M-tile then run on one XCD, so its A rows come into
    //    one L2 once instead of into all eight.
    int mt, nb;
    bool fair = false;  // see the wave priorities in the K loop
    if constexpr (BM <= 32) {
        const int NB = p.N / (16 * NW * WN);
        const int work = p.tiles[p.E] * NB;  // <= the grid: tiles[E] <= mt_max
        const int per = (work + 7) >> 3;
        const int j = blockIdx.x >> 3;
        const int w = (blockIdx.x & 7) * per + j;
        if (j >= per || w >= work) return;
        mt = w / NB;
        nb = w % NB;
        fair = work <= p.resident;
    } else {
        const int id = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
        mt = id % p.mt_max;
        nb = id / p.mt_max;
        if (nb >= p.N / (16 * NW * WN) || mt >= p.tiles[p.E]) return;
    }
    // Expert of M-tile mt: the last e with tiles[e] <= mt (tiles[] is the
    // exclusive prefix of the experts' tile counts, so empty experts repeat
    // their successor's entry and are skipped).
    int e;
    if constexpr (BM <= 32) {
        // one wave-wide load and ballot per 64 experts instead of a chain of
        // dependent loads: these blocks are all resident at once, so their
        // start-up latency is on the kernel's critical path
        int cnt = 0;
        for (int base = 0; base < p.E; base += 64) {
            const int ee = base + lane;
            cnt += __popcll(__ballot(ee < p.E && p.tiles[ee] <= mt));
        }
        e = cnt - 1;
    } else {
        int lo = 0, hi = p.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
        }
        e = lo;
    }
    const int mt_local = mt - p.tiles[e];
    const int row0 = p.offsets[e] + mt_local * BM;
    const int rows = min(BM, p.offsets[e + 1] - row0);
    if (status) return;  // blob prepared for other dimensions: no weight reads, no stores
    for (int m = tid; m < BM; m += NW * 64)
        s_arow[m] = m < rows ? (p.gather ? p.row_to_route[row0 + m] / p.topk : row0 + m) : -1;
    if (tid == 0) s_narrive = 0;
    __syncthreads();

    // Main loop and epilogue of one tile whose rows fit in MS 16-row groups
    // (MS <= the kernel's BM / 16): the launch picks the smallest MS that covers
    // the tile, so an expert's last, partly filled tile runs fewer matrix-core
    // operations and loads.
    auto body = [&](auto ms_tag) {
        constexpr int MS = decltype(ms_tag)::value;
        constexpr bool BF = AB == AB_BF16_NV;
        const int KT = p.Kdim / kTileK;
        const size_t tiles_e = (size_t)(p.N / kStrip) * KT;
        const int gs0 = nb * (NW * WN) + wave * WN;  // first global strip of this wave
        const uint8_t* abase = static_cast<const uint8_t*>(p.a);
        const size_t a_row_bytes = F4 ? (size_t)p.Kdim / 2 : (size_t)p.Kdim * (F8 ? 1 : 2);
        const int r_any = s_arow[0];                 // rows past the group re-read a valid row

        // A staging: every 1 KB of the LDS tile is one wave-wide direct load
        // (lane l lands at byte 16 l).
        //  f16/bf16: block blk = 4 ms + 2 h + g holds rows ms*16 + 8 g + [0, 8),
        //    bytes 128 h + [0, 128) of the 256-byte K step: each row's request is
        //    one full 128-byte line. Row r (0..15 in its group) puts its 16-byte
        //    chunk c at slot (r % 8) * 8 + (c ^ (r % 8) ^ 7 (r / 8)): the 64
        //    addresses of one matrix-core operand read (16 rows, one chunk each)
        //    then differ modulo 1 KB and, within every 8-lane group, modulo 128
        //    bytes, which keeps the read free of bank conflicts (checked with the
        //    LDS conflict counter; without the factor 7 the reads conflicted).
        //  fp8: block blk = 2 ms + h holds lane l' = row ms*16 + l'%16,
        //    k = 64 h + 16 (l'/16) + [0, 16), the operand's own order (the
        //    128-byte-row form measured 3 % slower here).
        //  fp4: block blk = ms holds lane l' = row ms*16 + l'%16, packed
        //    k = 32 (l'/16) + [0, 32) (bytes 16 (l'/16) + [0, 16) of the row's
        //    64-byte step): the lane's 32 values are the one 32-block whose
        //    E8M0 scale that lane supplies (probed on gfx950).
        // Wave w loads the blocks w, w + NW, w + 2 NW, ...
        constexpr int JB = F8 ? 2 : (F4 ? 1 : 4);
        constexpr int AB_PER_WAVE = (MS * JB + NW - 1) / NW;
        uint32_t aoff[AB_PER_WAVE];  // byte offset of the lane's A row chunk (A < 4 GiB)
        int adst[AB_PER_WAVE];
#pragma unroll
        for (int i = 0; i < AB_PER_WAVE; ++i) {
            const int blk = wave + NW * i;
            const int ms = blk / JB, g = blk & 1, h = (blk % JB) >> 1;
            const int r8 = lane >> 3;  // row within the 8-row half
            const int koff = F4 ? 16 * (lane >> 4)
                                : (F8 ? g * 64 + 16 * (lane >> 4) : h * 128 + (((lane & 7) ^ r8 ^ (7 * g)) << 4));
            int r = r_any;
            if (ms < MS) {
                const int rr = s_arow[ms * 16 + (SC ? (lane & 15) : 8 * g + r8)];
                r = rr >= 0 ? rr : r_any;
            }
            aoff[i] = (uint32_t)((size_t)r * a_row_bytes + koff);
            adst[i] = (ms < MS) ? blk * 1024 : -1;   // -1: padding load into sJunk
        }
        const uint8_t* ascsrc = nullptr;
        if (SC) {
            const int m = wave * 64 + lane;
            const int rr = m < MS * 16 ? s_arow[m] : -1;
            ascsrc = p.a_scales + (size_t)(rr >= 0 ? rr : r_any) * (p.Kdim / 32);
        }
        // loads per step per wave: A, A scales, the strips' weight codes and
        // one load of all their weight scales
        static_assert(WN == 2 || WN == 4, "weight scales are read as 2 or 4 strips of a group of 4");
        constexpr int L = AB_PER_WAVE + (SC ? 1 : 0) + WN * (F8 ? 2 : 1) + 1;

        // Weight loads: small M tiles read each weight once, so they stream past
    // the caches (non-temporal); wide tiles rely on L2 hits across the M-tiles
    // of one expert and load normally.
    auto load_b = [](const u32x4* q) -> u32x4 {
        if constexpr (BM <= 32) return __builtin_nontemporal_load(q);
        else return *q;
    };
    // one step's loads; ks >= KT issues the same number of loads as padding
        auto issue = [&](int ks, int buf, u32x4* c1, u32x4* c2, uint32_t* sc) {
            const bool real = ks < KT;
            const int kk = real ? ks : KT - 1;
#pragma unroll
            for (int i = 0; i < AB_PER_WAVE; ++i)
                lds_load16(abase + aoff[i] + (size_t)kk * A_ROW, (real && adst[i] >= 0) ? (void*)&sA[buf][adst[i]] : (void*)sJunk);
            if (SC) lds_load4(ascsrc + kk * 4, (real && wave * 64 < MS * 16) ? (void*)&sAsc[buf][wave * 64] : (void*)sJunk);
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                const size_t tile = (size_t)e * tiles_e + (size_t)(gs0 + s) * KT + kk;
                if (F8) {
                    const u32x4* q = reinterpret_cast<const u32x4*>(p.b_codes + tile * kF8TileBytes + lane * 32);
                    c1[s] = load_b(q);
                    c2[s] = load_b(q + 1);
                } else if (F4) {
                    c1[s] = load_b(reinterpret_cast<const u32x4*>(p.b_codes + tile * kF4TileBytes + lane * 16));
                } else {
                    c1[s] = load_b(reinterpret_cast<const u32x4*>(p.b_codes + tile * kNvTileBytes + lane * 16));
                }
            }
            // the WN strips' scales of this step, side by side in one load:
            // fp8/fp4 the lane's E8M0 bytes (sc[0], byte s for strip s),
            // NVFP4 the lane's E4M3 dwords (sc[s])
            if (SC) {
                const uint8_t* sp = p.b_scales + wscale_offset(tiles_e, e, gs0, kk, KT, F8 ? kF8TileScale : kF4TileScale,
                                                               lane, 1);
                if constexpr (WN == 4) sc[0] = *reinterpret_cast<const uint32_t*>(sp);
                else sc[0] = *reinterpret_cast<const uint16_t*>(sp);
            } else {
                const uint8_t* sp = p.b_scales + wscale_offset(tiles_e, e, gs0, kk, KT, kNvTileScale,
                                                               (lane >> 5) * 16 + (lane & 15), 4);
                if constexpr (WN == 4) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(sp);
                    sc[0] = v.x; sc[1] = v.y; sc[2] = v.z; sc[3] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(sp);
                    sc[0] = v.x; sc[1] = v.y;
                }
            }
        };

        f32x4 acc[MS][WN];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int s = 0; s < WN; ++s) acc[ms][s] = f32x4{0.f, 0.f, 0.f, 0.f};

        // f16/bf16: this lane's operand chunk in the staged A tile: row lane % 16,
        // chunk lane / 16 (+ 4 for the second 64 bytes of a 128-byte half).
        const int a_r7 = lane & 7, a_g = (lane >> 3) & 1;
        const int a_slot0 = a_g * 1024 + a_r7 * 128 + (((lane >> 4) ^ a_r7 ^ (7 * a_g)) << 4);
        const int a_slot1 = a_slot0 ^ 64;
        auto compute = [&](int buf, const u32x4* bc, const u32x4* bc2, const uint32_t* bs) {
            if (F4) {
                // E2M1 operands, four VGPRs each (the instruction reads no more
                // for fp4), E8M0 scales of the lane's 32-block
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const uint4 a0 = *reinterpret_cast<const uint4*>(&sA[buf][ms * 1024 + lane * 16]);
                    const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
                    const int asc = (int)((sAsc[buf][ms * 16 + (lane & 15)] >> (8 * (lane >> 4))) & 0xFFu);
                    static_for<WN>([&](auto S) {
                        constexpr int s = decltype(S)::value;
                        const i32x8 bv = {(int)bc[s].x, (int)bc[s].y, (int)bc[s].z, (int)bc[s].w, 0, 0, 0, 0};
                        // byte s of the packed weight scales (operand select)
                        acc[ms][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc[ms][s], 4, 4, 0, asc, s, (int)bs[0]);
                    });
                }
            } else if (F8) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const uint4 a0 = *reinterpret_cast<const uint4*>(&sA[buf][ms * 2048 + lane * 16]);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(&sA[buf][ms * 2048 + 1024 + lane * 16]);
                    const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    const int asc = (int)((sAsc[buf][ms * 16 + (lane & 15)] >> (8 * (lane >> 4))) & 0xFFu);
                    static_for<WN>([&](auto S) {
                        constexpr int s = decltype(S)::value;
                        const i32x8 bv = {(int)bc[s].x, (int)bc[s].y, (int)bc[s].z, (int)bc[s].w,
                                          (int)bc2[s].x, (int)bc2[s].y, (int)bc2[s].z, (int)bc2[s].w};
                        acc[ms][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc[ms][s], 0, 0, 0, asc, s, (int)bs[0]);
                    });
                }
            } else if (!BF) {
                // fp16 operands: each E2M1 pair converts to two fp16 values, then
                // one packed multiply by the block scale (E4M3, exact in fp16);
                // code * scale has at most 6 significant bits and lies in
                // [2^-10, 2688], so the product is exact.
                h2 sfp[WN][2];
#pragma unroll
                for (int s = 0; s < WN; ++s) {
                    sfp[s][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[s], 1.0f, false);
                    sfp[s][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[s], 1.0f, true);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x4 bq[WN];
#pragma unroll
                    for (int s = 0; s < WN; ++s) {
                        const uint32_t w = bc[s][j];
                        const h2 f = (j & 1) ? sfp[s][j >> 1].yy : sfp[s][j >> 1].xx;
                        const h2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * f;
                        const h2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * f;
                        const h2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * f;
                        const h2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * f;
                        bq[s] = u32x4{__builtin_bit_cast(uint32_t, c0), __builtin_bit_cast(uint32_t, c1),
                                      __builtin_bit_cast(uint32_t, c2), __builtin_bit_cast(uint32_t, c3)};
                    }
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms) {
                        const uint4 a = *reinterpret_cast<const uint4*>(
                            &sA[buf][(ms * 4 + (j >> 1) * 2) * 1024 + ((j & 1) ? a_slot1 : a_slot0)]);
#pragma unroll
                        for (int s = 0; s < WN; ++s)
                            acc[ms][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, bq[s]), acc[ms][s], 0, 0, 0);
                    }
                    // keep each 32-deep slice's weights short-lived (no hoisting
                    // of later slices' conversions, which spills at 256 registers)
                    if constexpr (NW == 8) __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // bf16 operands: code * scale in fp32 (exact), then the top half
                // of each fp32 is the bf16 value (at most 6 significant bits).
                float sj[WN][4];
#pragma unroll
                for (int s = 0; s < WN; ++s) {
                    const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bs[s], 1.0f, false);
                    const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bs[s], 1.0f, true);
                    sj[s][0] = s01[0]; sj[s][1] = s01[1]; sj[s][2] = s23[0]; sj[s][3] = s23[1];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint4 bq[WN];
#pragma unroll
                    for (int s = 0; s < WN; ++s) {
                        const uint32_t w = j == 0 ? bc[s].x : (j == 1 ? bc[s].y : (j == 2 ? bc[s].z : bc[s].w));
                        float c[8];
                        e2m1x8_to_f32(w, c);
                        const float f = sj[s][j];
                        bq[s] = make_uint4(pack_pair(c[0] * f, c[1] * f, true), pack_pair(c[2] * f, c[3] * f, true),
                                           pack_pair(c[4] * f, c[5] * f, true), pack_pair(c[6] * f, c[7] * f, true));
                    }
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms) {
                        const uint4 a = *reinterpret_cast<const uint4*>(
                            &sA[buf][(ms * 4 + (j >> 1) * 2) * 1024 + ((j & 1) ? a_slot1 : a_slot0)]);
#pragma unroll
                        for (int s = 0; s < WN; ++s)
                            acc[ms][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bq[s]), acc[ms][s], 0, 0, 0);
                    }
                }
            }
        };

        u32x4 rc[P][WN], rc2[P][F8 ? WN : 1];
        uint32_t rs[P][WN];
#pragma unroll
        for (int u = 0; u < P - 1; ++u) {
            issue(u, u, rc[u], rc2[F8 ? u : 0], rs[u]);
            asm volatile("" ::: "memory");  // keep each step's loads together, in step order
        }
        // Step kt waits until only the loads of the P - 2 later steps are in
        // flight, then refills the buffer freed by step kt - 1. Full groups of P
        // steps run without branches between them, so every buffer keeps its
        // registers across the loop; the remaining steps follow after it.
        // Wave priorities (small tiles whose blocks are all resident at once):
        // the instruction arbiter favours older waves, so the blocks a CU
        // received first would stream ahead and the last ones would finish
        // late, with the chip's loads thinning out meanwhile. Each block's
        // waves instead run at priority 3, 2, 1, 0 over the four quarters of
        // their K loop, so blocks that are behind issue first.
        auto set_prio = [&](int kt) {
            const int q = (4 * kt) / KT;
            if (kt != 0 && q == (4 * (kt - 1)) / KT) return;
            if (q == 0) __builtin_amdgcn_s_setprio(3);
            else if (q == 1) __builtin_amdgcn_s_setprio(2);
            else if (q == 2) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        };
        auto step = [&](int kt, int u) {
            wait_vmcnt<L * (P - 2)>();
            bare_barrier();
            if (BM <= 32 && fair) set_prio(kt);
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                reg_fence(rc[u][s]);
                if (!SC || s == 0) reg_fence(rs[u][s]);
                if (F8) reg_fence(rc2[F8 ? u : 0][s]);
            }
            const int nxt = (u + P - 1) % P;  // static once the loops are unrolled
            issue(kt + P - 1, nxt, rc[nxt], rc2[F8 ? nxt : 0], rs[nxt]);
            compute(u, rc[u], rc2[F8 ? u : 0], rs[u]);
        };
        int kt0 = 0;
        for (; kt0 + P <= KT; kt0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) step(kt0 + u, u);
        }
#pragma unroll
        for (int u = 0; u < P - 1; ++u)
            if (kt0 + u < KT) step(kt0 + u, u);
        wait_vmcnt<0>();
        gemm_epilogue<AB, MS, WN, EPI>(p, acc, e, row0, rows, s_arow, gs0, lane);
    };
    if constexpr (BM >= 64) {
        if (rows > BM / 2) body(std::integral_constant<int, BM / 16>{});
        else if (BM == 128 && rows > 32) body(std::integral_constant<int, 4>{});
        else if (rows > 16) body(std::integral_constant<int, 2>{});
        else body(std::integral_constant<int, 1>{});
    } else {
        body(std::integral_constant<int, BM / 16>{});
    }
    if constexpr (EPI == EPI_FC2) {
        if (p.fused == FUSE_ARRIVE) {
            __syncthreads();  // s_arow is the list of completed tokens from here on
            arrive_finalize<NW, 16 * NW * WN>(p, nb, row0, rows, s_arow, &s_narrive);
        }
    }
}

// ---- host launchers (device code above) ----
// With timing events, hipExtLaunchKernelGGL records them at the kernel's own
// start and end, so the measured interval is the kernel alone.
template <typename K>
static void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t t0,
                         hipEvent_t t1, const GemmArgs& a) {
    if (t0) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, a);
    else hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
}

// Blocks of one kernel configuration the current device holds at once
// (occupancy x CUs), cached per configuration and device (every configuration
// has a cache of its own: all instantiations share one function type); 0 if
// the runtime cannot say.
template <int AB, int BM, int WN, int EPI, int P, int NW>
static int resident_blocks() {
    static std::atomic<int> cache[64];  // value + 1; 0 = not yet asked
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_kernel<AB, BM, WN, EPI, P, NW>,
                                                         NW * 64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = per_cu * cus + 1;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c - 1;
}

template <int AB, int EPI, int BM, int WN, int P, int NW>
static void launch_cfg(const GemmArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const long long blocks = (long long)(a.N / (16 * NW * WN)) * a.mt_max;
    const dim3 grid((unsigned)((blocks + 7) / 8 * 8)), block(NW * 64);
    GemmArgs b = a;
    b.resident = resident_blocks<AB, BM, WN, EPI, P, NW>();
    launch_timed(gemm_kernel<AB, BM, WN, EPI, P, NW>, grid, block, s, t0, t1, b);
}

template <int AB, int EPI>
static hipError_t launch_bm(int bm_index, const GemmArgs& a, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1) {
    // Small M tiles (few rows per expert, weight streaming): three-stage
    // pipeline, two strips per wave. Wide M tiles: four strips per wave, so
    // each A fragment read from LDS feeds four matrix-core operations; with
    // 512 columns per block, eight waves (two per SIMD) share one A tile,
    // which halves the A re-reads against 256-column blocks.
    constexpr bool SCL = AB == AB_FP8 || AB == AB_FP4;
    constexpr int PW = SCL ? 3 : 4;   // pipeline depth, four-wave wide tiles
    constexpr int PW8 = SCL ? 3 : 2;  // eight waves: what fits in 256 registers
    // MXFP8 FC1 quantizes whole 32-column blocks in its epilogue: a wave must
    // own 32 consecutive FC2-input columns, i.e. four strips under SwiGLU
    // (2I is always a multiple of 256) and two under ReLU2.
    constexpr bool QF = AB == AB_FP8 && EPI == EPI_FC1;
    if constexpr (QF) {
        if (bm_index <= 1 && a.N % 256 == 0) {
            if (bm_index == 0) launch_cfg<AB, EPI, 16, 4, 3, 4>(a, s, t0, t1);
            else launch_cfg<AB, EPI, 32, 4, 3, 4>(a, s, t0, t1);
            return hipGetLastError();
        }
    }
    switch (bm_index) {
        case 0: launch_cfg<AB, EPI, 16, 2, 3, 4>(a, s, t0, t1); break;
        case 1: launch_cfg<AB, EPI, 32, 2, 3, 4>(a, s, t0, t1); break;
        case 2:
            if (a.N % 256 == 0) launch_cfg<AB, EPI, 64, 4, 2, 4>(a, s, t0, t1);
            else launch_cfg<AB, EPI, 64, 2, 2, 4>(a, s, t0, t1);
            break;
        default:
            if (a.N % 256 != 0) {
                launch_cfg<AB, EPI, 128, 2, 2, 4>(a, s, t0, t1);
            } else if (a.N % 512 == 0) {
                // (not instantiated for bf16 operands: that variant spills)
                if constexpr (AB != AB_BF16_NV) launch_cfg<AB, EPI, 128, 4, PW8, 8>(a, s, t0, t1);
                else launch_cfg<AB, EPI, 128, 4, PW, 4>(a, s, t0, t1);
            } else {
                launch_cfg<AB, EPI, 128, 4, PW, 4>(a, s, t0, t1);
            }
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int ab, int epi, int bm_index, const GemmArgs& a, hipStream_t s,
                       hipEvent_t t0, hipEvent_t t1) {
    if (ab == AB_F16_NV) return epi == EPI_FC1 ? launch_bm<AB_F16_NV, EPI_FC1>(bm_index, a, s, t0, t1)
                                               : launch_bm<AB_F16_NV, EPI_FC2>(bm_index, a, s, t0, t1);
    if (ab == AB_BF16_NV) return epi == EPI_FC1 ? launch_bm<AB_BF16_NV, EPI_FC1>(bm_index, a, s, t0, t1)
                                                : launch_bm<AB_BF16_NV, EPI_FC2>(bm_index, a, s, t0, t1);
    if (ab == AB_FP4) return epi == EPI_FC1 ? launch_bm<AB_FP4, EPI_FC1>(bm_index, a, s, t0, t1)
                                            : launch_bm<AB_FP4, EPI_FC2>(bm_index, a, s, t0, t1);
    return epi == EPI_FC1 ? launch_bm<AB_FP8, EPI_FC1>(bm_index, a, s, t0, t1)
                          : launch_bm<AB_FP8, EPI_FC2>(bm_index, a, s, t0, t1);
}

}  // namespace moe
