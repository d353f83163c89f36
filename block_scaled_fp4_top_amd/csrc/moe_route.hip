// S1 routing (top-K + renormalised softmax) and S2 expert-contiguous
// permutation (MegaMoE post, "The problem": tokens go to a top-K subset of
// experts and the grouped GEMMs consume them expert by expert).
#include "moe_internal.h"
#include "moe_kernels.h"
#include "moe_route_dev.h"

namespace moe {

// One wave per token, 4 tokens per block. Each lane holds E/64 logits; K
// rounds of a wave-wide (max value, min index) reduction pick the experts in
// descending order with ties to the lower id. Lane k keeps the k-th pick.
// p_k = exp(l_k - l_max) / sum_j exp(l_j - l_max), summed in k order.
// Block 0 also clears the misc words of the forward and compares the
// prepared blob's header with the one the call's dimensions imply (one word
// per lane of its first wave): the status word becomes MOE_ERR_INVALID on any
// difference, 0 otherwise, so the later kernels of the forward skip a blob
// prepared for other dimensions, activation or format.
template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int K, int32_t* __restrict__ ids,
                                                         float* __restrict__ topw,
                                                         uint32_t* __restrict__ misc,
                                                         const uint32_t* __restrict__ blob,
                                                         BlobHeader expect,
                                                         uint32_t* __restrict__ status) {
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < kMiscWords; i += blockDim.x) misc[i] = 0u;
        if (threadIdx.x < 64) {
            constexpr int kWords = sizeof(BlobHeader) / 4;
            static_assert(kWords <= 64, "one header word per lane");
            const uint32_t* ew = reinterpret_cast<const uint32_t*>(&expect);
            const int l = threadIdx.x;
            const bool differs = l < kWords && blob[l] != ew[l];
            const uint64_t any = __ballot(differs);
            if (l == 0) *status = any ? (uint32_t)MOE_ERR_INVALID : 0u;
        }
    }
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_one_token<EPL>(logits + (size_t)t * E, E, K, lane, ids + (size_t)t * K,
                         topw + (size_t)t * K);
}

// Per-block expert histogram of kPermChunk consecutive routes (LDS atomics;
// counts do not depend on the order of the increments).
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ ids, int R,
                                                        int E, int32_t* __restrict__ bhist) {
    __shared__ int32_t h[kMaxE];
    for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kPermChunk;
    for (int i = threadIdx.x; i < kPermChunk; i += 256) {
        const int r = base + i;
        if (r < R) atomicAdd(&h[ids[r]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) bhist[(size_t)blockIdx.x * E + e] = h[e];
}

// Exclusive scan over the threads of a 1024-thread block: a DPP scan inside
// each wave, the 16 wave totals scanned by wave 0, two barriers. The totals
// (buf[0, 16)) and the wave prefixes (buf[16, 32)) are separate, so a second
// scan may reuse buf right away.
__device__ __forceinline__ int block1024_exclusive_scan(int v, int* buf /*>= 32 ints*/) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) buf[w] = x;
    __syncthreads();
    if (w == 0) {
        const int a = lane < 16 ? buf[lane] : 0;
        const int ia = wave_incl_scan(a);
        if (lane < 16) buf[16 + lane] = ia - a;
    }
    __syncthreads();
    return buf[16 + w] + x - v;
}

// Three independent exclusive scans at once (same scheme, two barriers;
// totals in buf[0, 48), wave prefixes in buf[48, 96)).
__device__ __forceinline__ int3 block1024_exclusive_scan3(int3 v, int* buf /*>= 96 ints*/) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int3 x = make_int3(wave_incl_scan(v.x), wave_incl_scan(v.y), wave_incl_scan(v.z));
    if (lane == 63) { buf[3 * w] = x.x; buf[3 * w + 1] = x.y; buf[3 * w + 2] = x.z; }
    __syncthreads();
    if (w == 0) {
        const int a = lane < 16 ? buf[3 * lane] : 0;
        const int b = lane < 16 ? buf[3 * lane + 1] : 0;
        const int c = lane < 16 ? buf[3 * lane + 2] : 0;
        const int ia = wave_incl_scan(a), ib = wave_incl_scan(b), ic = wave_incl_scan(c);
        if (lane < 16) {
            buf[48 + 3 * lane] = ia - a;
            buf[48 + 3 * lane + 1] = ib - b;
            buf[48 + 3 * lane + 2] = ic - c;
        }
    }
    __syncthreads();
    return make_int3(buf[48 + 3 * w] + x.x - v.x, buf[48 + 3 * w + 1] + x.y - v.y,
                     buf[48 + 3 * w + 2] + x.z - v.z);
}

// One block of 1024 threads: per-block bases by a column scan over the block
// histograms (each expert's block list split among up to 1024 / E threads,
// whose loads are issued eight at a time), expert counts and offsets, and the
// exclusive scans of ceil(count / BM) that list the grouped-GEMM M-tiles.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ bhist,
                                                         int nblk, int E, int R,
                                                         int32_t* __restrict__ bbase,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tiles) {
    __shared__ int buf[2 * 1024];
    __shared__ int part[1024];  // [q][e]: sum, then exclusive prefix over q, of split q
    __shared__ int s_off[kMaxE];
    const int t = threadIdx.x;
    int tpe = 1;
    while (tpe * 2 * E <= 1024) tpe *= 2;
    const int q = t / E, ec = t - q * E;
    const bool active = q < tpe;
    const int cb = (nblk + tpe - 1) / tpe;
    const int b0 = min(nblk, q * cb), b1 = min(nblk, b0 + cb);
    if (active) {
        int sum = 0;
        for (int b = b0; b < b1; b += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? bhist[(size_t)(b + u) * E + ec] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        part[q * E + ec] = sum;
    }
    __syncthreads();
    const int e = t;
    int run = 0;
    if (e < E) {
        for (int qq = 0; qq < tpe; ++qq) {
            const int v = part[qq * E + e];
            part[qq * E + e] = run;
            run += v;
        }
    }
    const int off = block1024_exclusive_scan(e < E ? run : 0, buf);
    if (e < E) {
        counts[e] = run;
        offsets[e] = off;
        s_off[e] = off;
    }
    if (e == 0) offsets[E] = R;
    __syncthreads();
    if (active) {
        int base = s_off[ec] + part[q * E + ec];
        for (int b = b0; b < b1; b += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? bhist[(size_t)(b + u) * E + ec] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (b + u < b1) bbase[(size_t)(b + u) * E + ec] = base;
                base += v[u];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kNumBM; ++i) {
        const int bm = bm_of(i);
        const int nt = e < E ? (run + bm - 1) / bm : 0;
        const int toff = block1024_exclusive_scan(nt, buf);
        if (e < E) tiles[i * (E + 1) + e] = toff;
        if (e == E - 1) tiles[i * (E + 1) + E] = toff + nt;
    }
}

// Scatter: route r gets row bbase[block][e] + (routes of expert e earlier in
// this block). Sub-chunks of 256 routes are processed in order; inside a wave
// the rank comes from ballots matching the expert id bit by bit; across the
// block's waves from per-wave counts in LDS. No atomics decide any position.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, int R,
                                                           int E, const int32_t* __restrict__ bbase,
                                                           int32_t* __restrict__ r2r,
                                                           int32_t* __restrict__ rt2row) {
    __shared__ int32_t cnt[kMaxE];
    __shared__ int32_t wh[4][kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int e = tid; e < E; e += 256) {
        cnt[e] = bbase[(size_t)blockIdx.x * E + e];
        wh[0][e] = wh[1][e] = wh[2][e] = wh[3][e] = 0;
    }
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int sub = 0; sub < kPermChunk / 256; ++sub) {
        const int r = blockIdx.x * kPermChunk + sub * 256 + tid;
        const bool valid = r < R;
        const int x = valid ? ids[r] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (x >> b) & 1;
            const uint64_t bal = __ballot(valid && bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid && rank == 0) wh[w][x] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int prior = 0;
            for (int ww = 0; ww < w; ++ww) prior += wh[ww][x];
            const int row = cnt[x] + prior + rank;
            if (row >= 0 && row < R) {
                r2r[row] = r;
                rt2row[r] = row;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += 256) {
            cnt[e] += wh[0][e] + wh[1][e] + wh[2][e] + wh[3][e];
            wh[0][e] = wh[1][e] = wh[2][e] = wh[3][e] = 0;
        }
        __syncthreads();
    }
}


// Small batches (R <= 4096 routes, E <= 256): histogram, scans and the
// stable scatter in one block of 1024 threads (16 waves), saving two
// launches. Same results as the multi-block path: the scatter walks the
// routes in order, 1024 at a time, with in-wave ballot ranks and per-wave
// counts in LDS.
constexpr int kSmallMaxE = 256;
constexpr int kSmallMaxR = 4096;

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles, int32_t* __restrict__ r2r,
    int32_t* __restrict__ rt2row) {
    __shared__ int buf[2 * 1024];
    __shared__ int32_t cnt[kSmallMaxE];
    __shared__ int32_t wh[16][kSmallMaxE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int kPer = kSmallMaxR / 1024;  // routes per thread, kept in registers
    int xs[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int r = tid + 1024 * i;
        xs[i] = r < R ? ids[r] : -1;
    }
    for (int e = tid; e < kSmallMaxE; e += 1024) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (xs[i] >= 0) atomicAdd(&cnt[xs[i]], 1);
    __syncthreads();
    const int run = tid < E ? cnt[tid] : 0;
    // expert offsets and the four tile-list offsets in one pass: all prefix
    // sums stay below 2^16 here (R <= kSmallMaxR, tiles <= R/16 + E), so two
    // scans share each 32-bit word
    int nt[kNumBM];
#pragma unroll
    for (int i = 0; i < kNumBM; ++i) nt[i] = tid < E ? (run + bm_of(i) - 1) / bm_of(i) : 0;
    static_assert(kNumBM == 4, "packing below assumes four tile sizes");
    const int3 pk = block1024_exclusive_scan3(
        make_int3(run | (nt[0] << 16), nt[1] | (nt[2] << 16), nt[3]), buf);
    const int off = pk.x & 0xFFFF;
    const int toff[kNumBM] = {pk.x >> 16, pk.y & 0xFFFF, pk.y >> 16, pk.z};
    if (tid < E) {
        counts[tid] = run;
        offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = R;
#pragma unroll
    for (int i = 0; i < kNumBM; ++i) {
        if (tid < E) tiles[i * (E + 1) + tid] = toff[i];
        if (tid == E - 1) tiles[i * (E + 1) + E] = toff[i] + nt[i];
    }
    if (tid < E) cnt[tid] = off;
    for (int e = tid; e < kSmallMaxE; e += 1024)
        for (int ww = 0; ww < 16; ++ww) wh[ww][e] = 0;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int base = 1024 * i;
        if (base >= R) break;
        const int r = base + tid;
        const bool valid = r < R;
        const int x = valid ? xs[i] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (x >> b) & 1;
            const uint64_t bal = __ballot(valid && bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid && rank == 0) wh[w][x] = __popcll(peers);
        __syncthreads();
        if (valid) {
            // routes of expert x in the earlier waves: all 15 reads issued
            // together, the later waves' counts masked out
            int prior = 0;
#pragma unroll
            for (int ww = 0; ww < 15; ++ww) {
                const int c = wh[ww][x];
                prior += ww < w ? c : 0;
            }
            const int row = cnt[x] + prior + rank;
            if (row >= 0 && row < R) {
                r2r[row] = r;
                rt2row[r] = row;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += 1024) {
            int sum = 0;
            for (int ww = 0; ww < 16; ++ww) { sum += wh[ww][e]; wh[ww][e] = 0; }
            cnt[e] += sum;
        }
        __syncthreads();
    }
}

hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* ids, float* topw,
                        uint32_t* misc, const void* blob, const BlobHeader& expect,
                        uint32_t* status, hipStream_t s) {
    const dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + 63) / 64;
    const uint32_t* bw = static_cast<const uint32_t*>(blob);
#define RT(N) hipLaunchKernelGGL(route_topk_kernel<N>, grid, block, 0, s, logits, T, E, K, ids, topw, misc, bw, expect, status)
    if (epl <= 1) RT(1);
    else if (epl <= 2) RT(2);
    else if (epl <= 4) RT(4);
    else if (epl <= 8) RT(8);
    else RT(16);
#undef RT
    return hipGetLastError();
}

bool small_route_permute(int R, int E) { return R <= kSmallMaxR && E <= kSmallMaxE; }

hipError_t launch_permute_small(const int32_t* ids, int R, int E, int32_t* counts,
                                int32_t* offsets, int32_t* tiles, int32_t* r2r, int32_t* rt2row,
                                hipStream_t s) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, s, ids, R, E, counts, offsets,
                       tiles, r2r, rt2row);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int R, int E, int nblk, int32_t* bhist,
                          int32_t* bbase, int32_t* counts, int32_t* offsets, int32_t* tiles,
                          int32_t* r2r, int32_t* rt2row, hipStream_t s) {
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nblk), dim3(256), 0, s, ids, R, E, bhist);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, bhist, nblk, E, R, bbase,
                       counts, offsets, tiles);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblk), dim3(256), 0, s, ids, R, E, bbase, r2r,
                       rt2row);
    return hipGetLastError();
}

}  // namespace moe
