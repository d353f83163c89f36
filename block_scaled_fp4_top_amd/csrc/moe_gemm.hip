// S4/S6 grouped GEMMs with fused epilogues.
//
// C[r][n] = sum_k A[row(r)][k] * W_e[n][k] for the rows r of one expert e.
// A block of 256 threads (4 waves) owns an M-tile of BM rows of one expert
// (from the device tile list built by the permutation) and 4*WN strips of 16
// output columns; wave w owns strips [w*WN, w*WN + WN).
//  - A (activations) is staged through LDS per 128-wide K step, double
//    buffered, in the exact order the matrix cores read it, so every wave's
//    fragment read is 1 KB (f16/bf16) or 2 KB (fp8) of contiguous LDS.
//  - B (weights) is read straight from HBM into registers: the prepared blob
//    stores every 16 x 128 micro-tile as the register image of a 64-lane wave,
//    so each load is a contiguous 1 KB (NVFP4) or 2 KB (MXFP8) per wave.
//  - NVFP4: exact dequantization code * sf in registers (hardware fp4 -> f32
//    convert at unit scale, one fp32 multiply by the E4M3 scale; the product
//    has at most 6 significant bits so the f16/bf16 pack is exact), then
//    v_mfma_f32_16x16x32_{f16,bf16}. The E4M3 block-16 scales do not fit the
//    matrix cores' E8M0 block-32 scaling, so the scale is applied on the VALU.
//  - MXFP8: v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0 block scales as
//    the per-lane scale operands; no dequantization at all.
//  - Epilogue: global scales (g_a * g_w), then FC1: SwiGLU/ReLU2, optional
//    input-side router weight in FP32, store of the FC2 input (fp32 + amax, or
//    bf16); FC2: store of the permuted output or fp32 atomic scatter-add into
//    the token accumulator (fused finalize).
#include "moe_internal.h"
#include "moe_kernels.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t pack_pair(float lo, float hi, bool bf16) {
    if (bf16) return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int AB, int BM, int WN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
    constexpr bool F8 = AB == AB_FP8;
    constexpr bool BF = AB == AB_BF16_NV;
    constexpr int MS = BM / 16;
    constexpr int A_ROW = F8 ? 128 : 256;            // bytes of one A row per K step
    constexpr int A_TILE = BM * A_ROW;
    constexpr int CHUNKS = A_TILE / 16;
    constexpr int CPT = (CHUNKS + 255) / 256;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][A_TILE];
    __shared__ uint32_t sAsc[2][F8 ? BM : 1];
    __shared__ int s_arow[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Block order: M-tile fastest (across experts), then N-block; consecutive
    // positions go to the same XCD (blocks are dealt round-robin over the 8
    // XCDs and the grid is a multiple of 8), so concurrently running blocks of
    // one XCD share an N-block's weight columns.
    const int total = gridDim.x;
    const int id = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int mt = id % p.mt_max, nb = id / p.mt_max;
    if (nb >= p.N / (64 * WN) || mt >= p.tiles[p.E]) return;
    int lo = 0, hi = p.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mt_local = mt - p.tiles[e];
    const int row0 = p.offsets[e] + mt_local * BM;
    const int rows = min(BM, p.offsets[e + 1] - row0);
    for (int m = tid; m < BM; m += 256)
        s_arow[m] = m < rows ? (p.gather ? p.row_to_route[row0 + m] / p.topk : row0 + m) : -1;
    __syncthreads();

    const int KT = p.Kdim / kTileK;
    const size_t tiles_e = (size_t)(p.N / kStrip) * KT;
    const int gs0 = nb * (4 * WN) + wave * WN;  // first global strip of this wave
    const uint8_t* abase = static_cast<const uint8_t*>(p.a);
    const size_t a_row_bytes = (size_t)p.Kdim * (F8 ? 1 : 2);

    uint4 areg[CPT];
    uint32_t ascreg = 0x7F7F7F7Fu;
    auto load_a = [&](int kt) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int cid = tid + 256 * i;
            if (cid < CHUNKS) {
                const int c = F8 ? (cid & 7) : (cid & 15);
                const int m = F8 ? (cid >> 3) : (cid >> 4);
                const int r = s_arow[m];
                areg[i] = r >= 0 ? *reinterpret_cast<const uint4*>(abase + (size_t)r * a_row_bytes +
                                                                   (size_t)kt * A_ROW + c * 16)
                                 : make_uint4(0, 0, 0, 0);
            }
        }
        if (F8 && tid < BM) {
            const int r = s_arow[tid];
            ascreg = r >= 0 ? *reinterpret_cast<const uint32_t*>(p.a_scales + (size_t)r * (p.Kdim / 32) + kt * 4)
                            : 0x7F7F7F7Fu;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int cid = tid + 256 * i;
            if (cid < CHUNKS) {
                int off;
                if (F8) {
                    const int c = cid & 7, m = cid >> 3;
                    off = ((m >> 4) * 64 + (m & 15) + 16 * (c & 3)) * 32 + (c >> 2) * 16;
                } else {
                    const int c = cid & 15, m = cid >> 4;
                    off = (((m >> 4) * 4 + (c >> 2)) * 64 + (m & 15) + 16 * (c & 3)) * 16;
                }
                *reinterpret_cast<uint4*>(&sA[buf][off]) = areg[i];
            }
        }
        if (F8 && tid < BM) sAsc[buf][tid] = ascreg;
    };

    uint4 bc[WN], bc2[WN], nc[WN], nc2[WN];
    uint32_t bs[WN], ns[WN];
    auto load_b = [&](int kt, uint4* c1, uint4* c2, uint32_t* sc) {
#pragma unroll
        for (int s = 0; s < WN; ++s) {
            const size_t tile = (size_t)e * tiles_e + (size_t)(gs0 + s) * KT + kt;
            if (F8) {
                const uint4* q = reinterpret_cast<const uint4*>(p.b_codes + tile * kF8TileBytes + lane * 32);
                c1[s] = q[0];
                c2[s] = q[1];
                sc[s] = p.b_scales[tile * kF8TileScale + lane];
            } else {
                c1[s] = *reinterpret_cast<const uint4*>(p.b_codes + tile * kNvTileBytes + lane * 16);
                sc[s] = *reinterpret_cast<const uint32_t*>(
                    p.b_scales + tile * kNvTileScale + ((lane >> 5) * 16 + (lane & 15)) * 4);
            }
        }
    };

    f32x4 acc[MS][WN];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int s = 0; s < WN; ++s) acc[ms][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    store_a(0);
    load_b(0, bc, bc2, bs);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            load_a(kt + 1);
            load_b(kt + 1, nc, nc2, ns);
        }
        if (F8) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const uint4* ap = reinterpret_cast<const uint4*>(&sA[buf][(ms * 64 + lane) * 32]);
                const uint4 a0 = ap[0], a1 = ap[1];
                const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                  (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                const int asc = (int)((sAsc[buf][ms * 16 + (lane & 15)] >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
                for (int s = 0; s < WN; ++s) {
                    const i32x8 bv = {(int)bc[s].x, (int)bc[s].y, (int)bc[s].z, (int)bc[s].w,
                                      (int)bc2[s].x, (int)bc2[s].y, (int)bc2[s].z, (int)bc2[s].w};
                    acc[ms][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, acc[ms][s], 0, 0, 0, asc, 0, (int)bs[s]);
                }
            }
        } else {
            uint32_t bfr[WN][4][4];
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bs[s], 1.0f, false);
                const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bs[s], 1.0f, true);
                const float sj[4] = {s01[0], s01[1], s23[0], s23[1]};
                const uint32_t wj[4] = {bc[s].x, bc[s].y, bc[s].z, bc[s].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float c[8];
                    e2m1x8_to_f32(wj[j], c);
#pragma unroll
                    for (int i = 0; i < 4; ++i) bfr[s][j][i] = pack_pair(c[2 * i] * sj[j], c[2 * i + 1] * sj[j], BF);
                }
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 a = *reinterpret_cast<const uint4*>(&sA[buf][((ms * 4 + j) * 64 + lane) * 16]);
#pragma unroll
                    for (int s = 0; s < WN; ++s) {
                        const uint4 b = make_uint4(bfr[s][j][0], bfr[s][j][1], bfr[s][j][2], bfr[s][j][3]);
                        if (BF)
                            acc[ms][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[ms][s], 0, 0, 0);
                        else
                            acc[ms][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc[ms][s], 0, 0, 0);
                    }
                }
        }
        if (more) {
            store_a(buf ^ 1);
#pragma unroll
            for (int s = 0; s < WN; ++s) { bc[s] = nc[s]; bc2[s] = nc2[s]; bs[s] = ns[s]; }
        }
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    const float gw = p.b_g ? p.b_g[e] : 1.0f;
    const int c16 = lane & 15;
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
                        const float hg = acc[ms][2 * u][i] * sc, hu = acc[ms][2 * u + 1][i] * sc;
                        float a = hg / (1.0f + expf(-hg)) * hu;
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
                if (p.fused) {
                    const int route = p.row_to_route[row];
                    const int t = route / p.topk;
                    const float w = p.on_input ? 1.0f : p.topw[route];
#pragma unroll
                    for (int s = 0; s < WN; ++s)
                        atomicAdd(&p.yacc[(size_t)t * p.N + (gs0 + s) * 16 + c16], w * (acc[ms][s][i] * sc));
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
        if (lane == 0) atomicMax(p.amax_slot, f2u(amax));
    }
}

template <int AB, int EPI>
static hipError_t launch_bm(int bm_index, const GemmArgs& a, hipStream_t s) {
    constexpr int WN = 2;
    const int nbn = a.N / (64 * WN);
    const long long blocks = (long long)nbn * a.mt_max;
    const dim3 grid((unsigned)((blocks + 7) / 8 * 8)), block(256);
    switch (bm_index) {
        case 0: hipLaunchKernelGGL((gemm_kernel<AB, 16, WN, EPI>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((gemm_kernel<AB, 32, WN, EPI>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<AB, 64, WN, EPI>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((gemm_kernel<AB, 128, WN, EPI>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int ab, int epi, int bm_index, const GemmArgs& a, hipStream_t s) {
    if (ab == AB_F16_NV) return epi == EPI_FC1 ? launch_bm<AB_F16_NV, EPI_FC1>(bm_index, a, s)
                                               : launch_bm<AB_F16_NV, EPI_FC2>(bm_index, a, s);
    if (ab == AB_BF16_NV) return epi == EPI_FC1 ? launch_bm<AB_BF16_NV, EPI_FC1>(bm_index, a, s)
                                                : launch_bm<AB_BF16_NV, EPI_FC2>(bm_index, a, s);
    return epi == EPI_FC1 ? launch_bm<AB_FP8, EPI_FC1>(bm_index, a, s)
                          : launch_bm<AB_FP8, EPI_FC2>(bm_index, a, s);
}

}  // namespace moe
