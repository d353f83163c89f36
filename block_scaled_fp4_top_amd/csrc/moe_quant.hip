// Block quantizers (S3 FC1 input, S5 FC2 input, S0 weights), the finalize
// (S7) and small helper kernels.
#include "moe_internal.h"
#include "moe_kernels.h"
#include "moe_quant_dev.h"

namespace moe {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// WPR waves per row: 1 (four rows per block) or 4 (one row per block, for
// few wide rows). With a tensor-wide or no global scale the blocks of a row
// are independent, and gridDim.y > 1 splits each row into chunks of
// 64 * WPR quantization blocks (few rows: more blocks in flight).
template <int KIND, bool BF16, int WPR>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ v, int rows,
                                                         int cols,
                                                         const uint32_t* __restrict__ amax_slot,
                                                         int amax_slots, int amax_stride,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         float* __restrict__ g,
                                                         uint16_t* __restrict__ deq) {
    constexpr int TPR = 64 * WPR;  // threads per row
    const int tid = threadIdx.x;
    const int lt = tid % TPR;      // thread index within the row
    const int row = blockIdx.x * (4 / WPR) + tid / TPR;
    if (row >= rows) return;
    const size_t base = (size_t)row * cols;
    if (KIND == QK_MX) {
        const int nb = cols / 32;
        const int b_end = gridDim.y == 1 ? nb : min(nb, ((int)blockIdx.y + 1) * TPR);
        for (int b = blockIdx.y * TPR + lt; b < b_end; b += TPR) {
            float vv[32];
            load16<BF16>(v, base + (size_t)b * 32, vv);
            load16<BF16>(v, base + (size_t)b * 32 + 16, vv + 16);
            uint8_t c[32];
            const uint32_t e8 = mxfp8_block(vv, c);
            uint4* dst = reinterpret_cast<uint4*>(codes + base + (size_t)b * 32);
            dst[0] = *reinterpret_cast<const uint4*>(c);
            dst[1] = *reinterpret_cast<const uint4*>(c + 16);
            scales[(size_t)row * nb + b] = (uint8_t)e8;
        }
        return;
    }
    float gg;
    if (KIND == QK_NV_TENSOR) {
        // the partial maxima (amax_slots <= 64), one per lane, then the wave's max
        const int ln = tid & 63;
        const float am = wave_max(ln < amax_slots ? u2f(amax_slot[(size_t)ln * amax_stride]) : 0.0f);
        gg = __fdiv_rn(am, 2688.0f);
        if (row == 0 && lt == 0 && blockIdx.y == 0) g[0] = gg;
    } else {
        float m = 0.0f;
        for (int i = lt; i < cols; i += TPR) m = fmaxf(m, fabsf(load1<BF16>(v, base + i)));
        m = wave_max(m);
        if (WPR > 1) {
            __shared__ float red[4];
            if ((tid & 63) == 0) red[tid >> 6] = m;
            __syncthreads();
            m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        }
        gg = __fdiv_rn(m, KIND == QK_NV_ROW_4O6 ? 1536.0f : 2688.0f);
        if (lt == 0) g[row] = gg;
    }
    const int nb = cols / 16;
    const int b_end = gridDim.y == 1 ? nb : min(nb, ((int)blockIdx.y + 1) * TPR);
    for (int b = blockIdx.y * TPR + lt; b < b_end; b += TPR) {
        float vv[16];
        load16<BF16>(v, base + (size_t)b * 16, vv);
        uint32_t packed[2], sf;
        if (KIND == QK_NV_ROW_4O6) nvfp4_block_4o6(vv, gg, packed, &sf);
        else nvfp4_block(vv, gg, packed, &sf);
        *reinterpret_cast<uint2*>(codes + base / 2 + (size_t)b * 8) = make_uint2(packed[0], packed[1]);
        scales[(size_t)row * nb + b] = (uint8_t)sf;
        if (deq) {
            uint32_t h[8];
            nvfp4_deq_f16(packed, sf, h);
            uint4* dst = reinterpret_cast<uint4*>(deq + base + (size_t)b * 16);
            dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
            dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
        }
    }
}

// NVFP4 with one global scale per row, rows of at most 64 * 16 * NBL values:
// one wave per row holds its row in registers (lane l owns the 16-element
// blocks l, l + 64, ...), so the row max and the quantization read HBM once.
template <bool BF16, int NBL, bool F46>
__global__ __launch_bounds__(256) void quant_rows_nvrow_kernel(const void* __restrict__ v, int rows,
                                                               int cols,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               float* __restrict__ g,
                                                               uint16_t* __restrict__ deq) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const size_t base = (size_t)row * cols;
    const int nb = cols / 16;
    float vv[NBL][16];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
        const int b = lane + 64 * j;
        if (b < nb) {
            load16<BF16>(v, base + (size_t)b * 16, vv[j]);
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(vv[j][i]));
        }
    }
    m = wave_max(m);
    const float gg = __fdiv_rn(m, F46 ? 1536.0f : 2688.0f);
    if (lane == 0) g[row] = gg;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
        const int b = lane + 64 * j;
        if (b >= nb) break;
        uint32_t packed[2], sf;
        if (F46) nvfp4_block_4o6(vv[j], gg, packed, &sf);
        else nvfp4_block(vv[j], gg, packed, &sf);
        *reinterpret_cast<uint2*>(codes + base / 2 + (size_t)b * 8) = make_uint2(packed[0], packed[1]);
        scales[(size_t)row * nb + b] = (uint8_t)sf;
        if (deq) {
            uint32_t h[8];
            nvfp4_deq_f16(packed, sf, h);
            uint4* dst = reinterpret_cast<uint4*>(deq + base + (size_t)b * 16);
            dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
            dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
        }
    }
}

// NVFP4 rows (packed codes [rows][cols/2], E4M3 scales [rows][cols/16]) re-blocked
// to MXFP4 (packed codes [rows][cols/2], E8M0 scales [rows][cols/32]): one
// thread per 32-element block (16-byte loads and stores).
__global__ __launch_bounds__(256) void reblock_mxfp4_kernel(const uint8_t* __restrict__ nv_codes,
                                                            const uint8_t* __restrict__ nv_scales,
                                                            size_t nblocks, uint8_t* __restrict__ mx_codes,
                                                            uint8_t* __restrict__ mx_scales,
                                                            const uint32_t* __restrict__ status) {
    if (status && *status) return;
    for (size_t b = (size_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (size_t)gridDim.x * 256) {
        const uint4 c = reinterpret_cast<const uint4*>(nv_codes)[b];
        const uint32_t nv[4] = {c.x, c.y, c.z, c.w};
        const uint16_t sc = reinterpret_cast<const uint16_t*>(nv_scales)[b];
        uint32_t mx[4];
        const uint32_t e8 = mxfp4_reblock32(nv, sc & 0xFFu, sc >> 8, mx);
        reinterpret_cast<uint4*>(mx_codes)[b] = make_uint4(mx[0], mx[1], mx[2], mx[3]);
        mx_scales[b] = (uint8_t)e8;
    }
}

// Max |v| over n elements as fp32 bits (order-free atomicMax on non-negative
// floats compared as unsigned integers). Block b folds its maximum into word
// (b % nslots) * stride of slot: spreading the atomics over words on separate
// lines avoids the serialisation of many atomics on one address.
template <bool BF16>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ v, size_t n,
                                                   uint32_t* __restrict__ slot, int nslots,
                                                   int stride) {
    float m = 0.0f;
    const size_t n16 = n / 16;  // 16-element chunks (v is 16-byte aligned)
    for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < n16; c += (size_t)gridDim.x * 256) {
        float q[16];
        load16<BF16>(v, c * 16, q);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(q[i]));
    }
    for (size_t i = n16 * 16 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(load1<BF16>(v, i)));
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        atomicMax(slot + (size_t)(blockIdx.x % nslots) * stride, f2u(m));
    }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = v;
}

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu2 __attribute__((ext_vector_type(2)));

// Deterministic finalize: one block per token and column chunk (blockIdx.y;
// the whole row when gridDim.y == 1); the token's K route rows and weights are
// staged in LDS, each thread reduces 4 columns over k = 0..K-1 in order in
// fp32 and rounds once to bf16. Every O element is read once: its
// loads are non-temporal (the kernel ran 11-16 % faster with them on the
// prefill workloads).
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const void* __restrict__ O,
                                                       const int32_t* __restrict__ rt2row,
                                                       const float* __restrict__ w, int K, int H,
                                                       uint16_t* __restrict__ y,
                                                       const uint32_t* __restrict__ status) {
    __shared__ int32_t s_row[kMaxK];
    __shared__ float s_w[kMaxK];
    const int t = blockIdx.x;
    const uint32_t st = status ? *status : 0u;  // issued beside the route loads
    if ((int)threadIdx.x < K) {
        s_row[threadIdx.x] = rt2row[(size_t)t * K + threadIdx.x];
        s_w[threadIdx.x] = w ? w[(size_t)t * K + threadIdx.x] : 1.0f;
    }
    if (st) return;  // uniform over the block
    __syncthreads();
    const int c_end = gridDim.y == 1 ? H : min(H, ((int)blockIdx.y + 1) * 1024);
    for (int c = blockIdx.y * 1024 + threadIdx.x * 4; c < c_end; c += 1024) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        // the loads of up to 8 routes are issued together, then reduced in k order
        for (int k0 = 0; k0 < K; k0 += 8) {
            float4 q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k0 + u < K) {
                    const size_t off = (size_t)s_row[k0 + u] * H + c;
                    if (BF16) {
                        const vu2 b = __builtin_nontemporal_load(
                            reinterpret_cast<const vu2*>(static_cast<const uint16_t*>(O) + off));
                        q[u] = make_float4(u2f(b.x << 16), u2f(b.x & 0xFFFF0000u), u2f(b.y << 16),
                                           u2f(b.y & 0xFFFF0000u));
                    } else {
                        const vf4 v = __builtin_nontemporal_load(
                            reinterpret_cast<const vf4*>(static_cast<const float*>(O) + off));
                        q[u] = make_float4(v.x, v.y, v.z, v.w);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k0 + u < K) {
                    const float wk = s_w[k0 + u];
                    a0 = __fmaf_rn(wk, q[u].x, a0); a1 = __fmaf_rn(wk, q[u].y, a1);
                    a2 = __fmaf_rn(wk, q[u].z, a2); a3 = __fmaf_rn(wk, q[u].w, a3);
                }
            }
        }
        const uint32_t lo = (uint32_t)bf16_rne(a0) | ((uint32_t)bf16_rne(a1) << 16);
        const uint32_t hi = (uint32_t)bf16_rne(a2) | ((uint32_t)bf16_rne(a3) << 16);
        *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = make_uint2(lo, hi);
    }
}

// ---------------------------------------------------------------------------
// Weight preparation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_amax_kernel(const float* __restrict__ w,
                                                        size_t per_expert,
                                                        uint32_t* __restrict__ amax) {
    const int e = blockIdx.y;
    const float* we = w + (size_t)e * per_expert;
    float m = 0.0f;
    for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < per_expert;
         i += (size_t)gridDim.x * 256 * 4) {
        const float4 q = *reinterpret_cast<const float4*>(we + i);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))));
    }
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(amax + e, f2u(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// Logical row of prepared row p (SwiGLU strip interleave when swiglu_I > 0).
__device__ __forceinline__ int logical_row(int p, int swiglu_I) {
    if (!swiglu_I) return p;
    const int st = p >> 4;
    return (st & 1) * swiglu_I + (st >> 1) * 16 + (p & 15);
}

// One thread per (expert, prepared row, 16-block): quantize with the expert's
// global scale and scatter into the micro-tile register image.
__global__ __launch_bounds__(256) void prep_nvfp4_kernel(const float* __restrict__ w, int E, int N,
                                                         int K, int swiglu_I,
                                                         const uint32_t* __restrict__ amax,
                                                         float* __restrict__ gout,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
    const int nkb = K / 16;
    const size_t total = (size_t)E * N * nkb;
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int e = (int)(id / ((size_t)N * nkb));
    const int rem = (int)(id % ((size_t)N * nkb));
    const int p = rem / nkb, kb = rem % nkb;
    const float g = __fdiv_rn(u2f(amax[e]), 2688.0f);
    if (p == 0 && kb == 0) gout[e] = g;
    const int n = logical_row(p, swiglu_I);
    float v[16];
    const float4* src = reinterpret_cast<const float4*>(w + ((size_t)e * N + n) * K + (size_t)kb * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = src[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    uint32_t packed[2], sf;
    nvfp4_block(v, g, packed, &sf);
    const int k0 = kb * 16, kt = k0 / kTileK, j = (k0 % kTileK) / 32, half = (k0 % 32) / 16;
    const size_t tiles_e = (size_t)(N / kStrip) * (K / kTileK);
    const size_t tile = (size_t)e * tiles_e + (size_t)(p / kStrip) * (K / kTileK) + kt;
    uint8_t* cb = codes + tile * kNvTileBytes;
    const int l1 = (p & 15) + 16 * (2 * half), l2 = l1 + 16;
    *reinterpret_cast<uint32_t*>(cb + l1 * 16 + j * 4) = packed[0];
    *reinterpret_cast<uint32_t*>(cb + l2 * 16 + j * 4) = packed[1];
    scales[wscale_offset(tiles_e, e, p / kStrip, kt, K / kTileK, kNvTileScale, half * 16 + (p & 15), 4) + j] =
        (uint8_t)sf;
}

// One thread per (expert, prepared row, 32-block).
__global__ __launch_bounds__(256) void prep_mxfp8_kernel(const float* __restrict__ w, int E, int N,
                                                         int K, int swiglu_I,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
    const int nkb = K / 32;
    const size_t total = (size_t)E * N * nkb;
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int e = (int)(id / ((size_t)N * nkb));
    const int rem = (int)(id % ((size_t)N * nkb));
    const int p = rem / nkb, kb = rem % nkb;
    const int n = logical_row(p, swiglu_I);
    float v[32];
    const float4* src = reinterpret_cast<const float4*>(w + ((size_t)e * N + n) * K + (size_t)kb * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 q = src[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    uint8_t c[32];
    const uint32_t e8 = mxfp8_block(v, c);
    const int k0 = kb * 32, kt = k0 / kTileK, kb4 = (k0 % kTileK) / 32;
    const size_t tiles_e = (size_t)(N / kStrip) * (K / kTileK);
    const size_t tile = (size_t)e * tiles_e + (size_t)(p / kStrip) * (K / kTileK) + kt;
    uint8_t* cb = codes + tile * kF8TileBytes;
    // block kb4 covers tile k in [32 kb4, 32 kb4 + 32): its first 16 values
    // live in lane q = (32 kb4 mod 64)/16, byte offset (kb4 >= 2 ? 16 : 0), the
    // next 16 in lane q + 1 at the same byte offset.
    const int q0 = ((32 * kb4) % 64) / 16, boff = kb4 >= 2 ? 16 : 0;
    const int la = (p & 15) + 16 * q0, lb = la + 16;
    *reinterpret_cast<uint4*>(cb + la * 32 + boff) = *reinterpret_cast<const uint4*>(c);
    *reinterpret_cast<uint4*>(cb + lb * 32 + boff) = *reinterpret_cast<const uint4*>(c + 16);
    scales[wscale_offset(tiles_e, e, p / kStrip, kt, K / kTileK, kF8TileScale, (p & 15) + 16 * kb4, 1)] =
        (uint8_t)e8;
}

// One thread per (expert, prepared row, 32-block): the two 16-blocks NVFP4-
// quantized with the expert's global scale (as prep_nvfp4_kernel), then
// re-blocked to MXFP4 and stored in the fp4 micro-tile register image: lane
// (p % 16) + 16 q of tile (p / 16, k / 128) holds row p's 32-block q of the
// tile (16 packed bytes, even element in the low nibble), scale byte at the
// same lane index.
__global__ __launch_bounds__(256) void prep_mxfp4_kernel(const float* __restrict__ w, int E, int N,
                                                         int K, int swiglu_I,
                                                         const uint32_t* __restrict__ amax,
                                                         float* __restrict__ gout,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
    const int nkb = K / 32;
    const size_t total = (size_t)E * N * nkb;
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int e = (int)(id / ((size_t)N * nkb));
    const int rem = (int)(id % ((size_t)N * nkb));
    const int p = rem / nkb, kb = rem % nkb;
    const float g = __fdiv_rn(u2f(amax[e]), 2688.0f);
    if (p == 0 && kb == 0) gout[e] = g;
    const int n = logical_row(p, swiglu_I);
    const float4* src = reinterpret_cast<const float4*>(w + ((size_t)e * N + n) * K + (size_t)kb * 32);
    uint32_t nv[4], sf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = src[4 * h + i];
            v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
        nvfp4_block(v, g, nv + 2 * h, sf + h);
    }
    uint32_t mx[4];
    const uint32_t e8 = mxfp4_reblock32(nv, sf[0], sf[1], mx);
    const int kt = (kb * 32) / kTileK, q = kb % 4;
    const size_t tiles_e = (size_t)(N / kStrip) * (K / kTileK);
    const size_t tile = (size_t)e * tiles_e + (size_t)(p / kStrip) * (K / kTileK) + kt;
    const int lane = (p & 15) + 16 * q;
    *reinterpret_cast<uint4*>(codes + tile * kF4TileBytes + lane * 16) = make_uint4(mx[0], mx[1], mx[2], mx[3]);
    scales[wscale_offset(tiles_e, e, p / kStrip, kt, K / kTileK, kF4TileScale, lane, 1)] = (uint8_t)e8;
}

__global__ void write_header_kernel(BlobHeader h, uint32_t* __restrict__ dst) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&h);
    if (threadIdx.x < sizeof(BlobHeader) / 4) dst[threadIdx.x] = w[threadIdx.x];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for(size_t n, unsigned cap = 4096) {
    size_t g = (n + 255) / 256;
    if (g > cap) g = cap;
    return g ? (unsigned)g : 1u;
}

hipError_t launch_write_header(const BlobHeader& h, void* dst, hipStream_t s) {
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, s, h, static_cast<uint32_t*>(dst));
    return hipGetLastError();
}

hipError_t launch_amax(const void* v, int in_bf16, size_t n, uint32_t* slot, int nslots, int stride,
                       hipStream_t s) {
    const dim3 grid(grid_for((n + 15) / 16, 1024)), block(256);
    if (in_bf16) hipLaunchKernelGGL(amax_kernel<true>, grid, block, 0, s, v, n, slot, nslots, stride);
    else hipLaunchKernelGGL(amax_kernel<false>, grid, block, 0, s, v, n, slot, nslots, stride);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const void* v, int in_bf16, int rows, int cols, int kind,
                             const uint32_t* amax_slot, int amax_slots, int amax_stride, uint8_t* codes,
                             uint8_t* scales, float* g, uint16_t* deq, hipStream_t s) {
    const bool per_row = kind == QK_NV_ROW || kind == QK_NV_ROW_4O6;
    if (per_row && !(rows < 2048 && cols >= 1024) && cols <= 64 * 16 * 8) {
        // single pass with the row in registers
        const int nbl = (cols / 16 + 63) / 64;
        const dim3 grid4((rows + 3) / 4), block4(256);
#define QN(BF, N, F) hipLaunchKernelGGL((quant_rows_nvrow_kernel<BF, N, F>), grid4, block4, 0, s, v, rows, cols, codes, scales, g, deq)
#define QNB(BF, F) do { if (nbl <= 1) QN(BF, 1, F); else if (nbl <= 2) QN(BF, 2, F); else if (nbl <= 4) QN(BF, 4, F); else QN(BF, 8, F); } while (0)
        if (in_bf16) {
            if (kind == QK_NV_ROW_4O6) QNB(true, true); else QNB(true, false);
        } else {
            if (kind == QK_NV_ROW_4O6) QNB(false, true); else QNB(false, false);
        }
#undef QNB
#undef QN
        return hipGetLastError();
    }
    const bool wide = rows < 2048 && cols >= 1024;  // few long rows: a block per row
    // very few rows: also split each row (not for per-row scales, whose row
    // maximum needs the whole row in one block)
    const int qb = kind == QK_MX ? 32 : 16;
    const unsigned chunks = (wide && rows < 256 && !per_row) ? (unsigned)((cols / qb + 255) / 256) : 1u;
    const dim3 grid(wide ? rows : (rows + 3) / 4, chunks), block(256);
#define QR(KD, BF, W) hipLaunchKernelGGL((quant_rows_kernel<KD, BF, W>), grid, block, 0, s, v, rows, cols, amax_slot, amax_slots, amax_stride, codes, scales, g, deq)
#define QRW(KD, BF) do { if (wide) QR(KD, BF, 4); else QR(KD, BF, 1); } while (0)
    if (in_bf16) {
        if (kind == QK_NV_TENSOR) QRW(QK_NV_TENSOR, true);
        else if (kind == QK_NV_ROW) QRW(QK_NV_ROW, true);
        else if (kind == QK_NV_ROW_4O6) QRW(QK_NV_ROW_4O6, true);
        else QRW(QK_MX, true);
    } else {
        if (kind == QK_NV_TENSOR) QRW(QK_NV_TENSOR, false);
        else if (kind == QK_NV_ROW) QRW(QK_NV_ROW, false);
        else if (kind == QK_NV_ROW_4O6) QRW(QK_NV_ROW_4O6, false);
        else QRW(QK_MX, false);
    }
#undef QRW
#undef QR
    return hipGetLastError();
}

hipError_t launch_reblock_mxfp4(const uint8_t* nv_codes, const uint8_t* nv_scales, size_t n,
                                uint8_t* mx_codes, uint8_t* mx_scales, const uint32_t* status,
                                hipStream_t s) {
    // n (elements) is a multiple of 32; codes 16-byte aligned
    const size_t nb = n / 32;
    hipLaunchKernelGGL(reblock_mxfp4_kernel, dim3(grid_for(nb, 8192)), dim3(256), 0, s, nv_codes, nv_scales,
                       nb, mx_codes, mx_scales, status);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n, 8192)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_finalize(const void* O, int is_bf16, const int32_t* rt2row, const float* w,
                           int T, int K, int H, uint16_t* y, const uint32_t* status,
                           hipStream_t s) {
    // few tokens: one block per 1024 columns as well, so the reads of O keep
    // enough blocks in flight (64 tokens of 7168 columns: the finalize stage
    // went from 14 to 7 us)
    const dim3 grid(T, T < 2048 ? (H + 1023) / 1024 : 1);
    if (is_bf16) hipLaunchKernelGGL(finalize_kernel<true>, grid, dim3(256), 0, s, O, rt2row, w, K, H, y, status);
    else hipLaunchKernelGGL(finalize_kernel<false>, grid, dim3(256), 0, s, O, rt2row, w, K, H, y, status);
    return hipGetLastError();
}

hipError_t launch_prep_amax(const float* w, int E, size_t per_expert, uint32_t* amax, hipStream_t s) {
    unsigned gx = (unsigned)((per_expert / 4 + 255) / 256);
    if (gx > 256) gx = 256;
    if (gx == 0) gx = 1;
    hipLaunchKernelGGL(prep_amax_kernel, dim3(gx, E), dim3(256), 0, s, w, per_expert, amax);
    return hipGetLastError();
}

hipError_t launch_prep_nvfp4(const float* w, int E, int N, int K, int swiglu_I,
                             const uint32_t* amax, float* g, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
    const size_t total = (size_t)E * N * (K / 16);
    hipLaunchKernelGGL(prep_nvfp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       w, E, N, K, swiglu_I, amax, g, codes, scales);
    return hipGetLastError();
}

hipError_t launch_prep_mxfp4(const float* w, int E, int N, int K, int swiglu_I,
                             const uint32_t* amax, float* g, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
    const size_t total = (size_t)E * N * (K / 32);
    hipLaunchKernelGGL(prep_mxfp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       w, E, N, K, swiglu_I, amax, g, codes, scales);
    return hipGetLastError();
}

hipError_t launch_prep_mxfp8(const float* w, int E, int N, int K, int swiglu_I, uint8_t* codes,
                             uint8_t* scales, hipStream_t s) {
    const size_t total = (size_t)E * N * (K / 32);
    hipLaunchKernelGGL(prep_mxfp8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       w, E, N, K, swiglu_I, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
