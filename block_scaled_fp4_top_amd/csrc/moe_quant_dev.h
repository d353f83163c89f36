// Device helpers of the block quantizers (loads of 16 values, wave maximum,
// fp16 copies of NVFP4 blocks).
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    return m;
}

// 16 consecutive values starting at element `idx` of a bf16 or fp32 row.
template <bool BF16>
__device__ __forceinline__ void load16(const void* base, size_t idx, float* v) {
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        const uint4 q0 = p[0], q1 = p[1];
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = u2f(w[i] << 16);
            v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = p[i];
            v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
    if (BF16) return u2f((uint32_t)static_cast<const uint16_t*>(base)[idx] << 16);
    return static_cast<const float*>(base)[idx];
}

// fp16 values code * sf of one NVFP4 block (exact: at most 6 significant bits
// in [2^-10, 2688]) into 8 dwords.
__device__ __forceinline__ void nvfp4_deq_f16(const uint32_t* packed, uint32_t sf, uint32_t* out) {
    const float s = e4m3_value(sf);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        float c[8];
        e2m1x8_to_f32(packed[w], c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[w * 4 + i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(c[2 * i] * s, c[2 * i + 1] * s));
    }
}

}  // namespace moe
