// Device code of S1 routing (top-K of one token by one wave) and the DPP
// wave scan of the permutation.
#pragma once

#include "moe_internal.h"

namespace moe {

// Top-K of one token by one wave. Each lane holds E/64 logits; K
// rounds of a wave-wide maximum of the key (value, then lower id) pick the
// experts in descending order with ties to the lower id. The key is the
// logit's order-preserving integer image in the high word and ~id in the low
// word, so one 64-bit maximum decides both; it is reduced by DPP rotations
// inside each 16-lane row and across the four rows by lane reads (no LDS
// round trips). p_k = exp(l_k - l_max) / sum_j exp(l_j - l_max), summed in k
// order.
__device__ __forceinline__ uint32_t orderable(float f) {
    const uint32_t u = f2u(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t dpp_ror(uint64_t k, int ctrl_sel) {
    const int lo = (int)(uint32_t)k, hi = (int)(uint32_t)(k >> 32);
    int lo2, hi2;
    switch (ctrl_sel) {  // row_ror:1, 2, 4, 8
        case 1: lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x121, 0xF, 0xF, false);
                hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x121, 0xF, 0xF, false); break;
        case 2: lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x122, 0xF, 0xF, false);
                hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x122, 0xF, 0xF, false); break;
        case 4: lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x124, 0xF, 0xF, false);
                hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x124, 0xF, 0xF, false); break;
        default: lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x128, 0xF, 0xF, false);
                 hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x128, 0xF, 0xF, false); break;
    }
    return ((uint64_t)(uint32_t)hi2 << 32) | (uint32_t)lo2;
}
__device__ __forceinline__ uint64_t wave_key_max(uint64_t k) {
    k = key_max(k, dpp_ror(k, 8));
    k = key_max(k, dpp_ror(k, 4));
    k = key_max(k, dpp_ror(k, 2));
    k = key_max(k, dpp_ror(k, 1));
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 16 * r);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * r);
        best = key_max(best, ((uint64_t)hi << 32) | lo);
    }
    return best;
}

__device__ __forceinline__ float from_orderable(uint32_t o) {
    return u2f((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int EPL>
__device__ __forceinline__ void route_one_token(const float* __restrict__ lt, int E, int K,
                                                int lane, int32_t* __restrict__ ids_t,
                                                float* __restrict__ w_t) {
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const float v = e < E ? lt[e] + 0.0f : 0.0f;  // -0 -> +0: equal logits tie
        key[i] = e < E ? ((uint64_t)orderable(v) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    float my_v = 0.0f;
    int my_e = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t kb = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) kb = key_max(kb, key[i]);
        const uint64_t best = wave_key_max(kb);  // wave-uniform
        const int be = (int)~(uint32_t)best;
        if ((be & 63) == lane) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (be >> 6)) key[i] = 0;  // taken
        }
        if (lane == k) { my_v = from_orderable((uint32_t)(best >> 32)); my_e = be; }
    }
    const float m = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, my_v)));
    const float ex = lane < K ? expf(my_v - m) : 0.0f;
    float s = 0.0f;
    for (int k = 0; k < K; ++k)
        s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), k));
    if (lane < K) {
        ids_t[lane] = my_e;
        w_t[lane] = __fdiv_rn(ex, s);
    }
}

// Inclusive scan over the 64 lanes of a wave with DPP moves: row_shr 1, 2, 4,
// 8 inside each 16-lane row (lanes shifted in from outside the row read 0),
// then row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds the total of rows 0-1 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
    return v;
}

}  // namespace moe
