// Single-launch MoE layer for small batches: routing (S1), permutation (S2),
// FC1-input quantization (S3), FC1 with its epilogue (S4, S5), FC2-input
// quantization (S5), FC2 (S6) and the finalize (S7) in one persistent launch
// (MegaMoE post, "Our approach": one persistent kernel per forward pass, with
// the FC2 of a group of rows starting as soon as its FC1 is done).
//
// Work is a sequence of items taken from device queues by whichever block is
// free; an item waits only for items that were handed out before it, so the
// launch drains without any assumption about which blocks run at once (every
// wait is also bounded, see ls_wait):
//  - phase 1, one queue: route items (4 tokens each); the block finishing the
//    last one builds the permutation in place and publishes it. FC1-input
//    quantization items (4 rows each; per-tensor NVFP4 first takes partial
//    maxima of x in amax items).
//  - phase 2, 8 queues, one per XCD (blockIdx % 8, as the hardware deals
//    blocks out round-robin), each over a contiguous range of M-tiles: the
//    FC1 tiles (M-tile-major, N-block fastest), then for NVFP4 one FC2-input
//    quantization item per M-tile, then the FC2 tiles. A block drains its own
//    queue first, then helps the others. An FC2 tile waits until every FC1
//    N-block of its M-tile is done (NVFP4: until its M-tile is quantized; the
//    per-tensor scale waits for all of FC1). Keeping an M-tile's FC1, its
//    quantization and its FC2 on one XCD keeps its FC2 input in that XCD's L2.
//  - finalize: after its epilogue stores, an FC2 tile counts, per token of its
//    rows, the route contributions to its column block; the tile that brings
//    a token's count to K sums that token's K route rows for those columns in
//    route order (fp32, one bf16 rounding), exactly as the standalone
//    deterministic finalize does. The result is deterministic for either
//    finalize setting.
// Cross-block data passes through agent-scope release (writer: every wave
// fences its own stores, then one counter update) and acquire (reader: one
// poll that sees the count, then an acquire fence) so it is visible across
// the XCDs' separate L2 caches.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>

#include "moe_gemm_tile.h"
#include "moe_quant_dev.h"
#include "moe_route_dev.h"

namespace moe {

namespace {

constexpr int kXAmaxChunk = 256 * 64;  // x elements per amax item

// One thread waits until *ctr >= target, then acquires at agent scope. The
// polls back off (sleeps of 64 to 1024 cycles) to keep the pressure of many
// waiting blocks on one counter low. Gives up when the forward's status turns
// non-zero (another wait gave up, or the blob header did not match), or after
// `ticks` of the constant-rate wall clock (or 2^24 polls), recording
// MOE_ERR_TIMEOUT as the status if none is set yet, with the counter's word
// index, its target and the value last seen in status words 1..3.
__device__ bool ls_wait(const uint32_t* ctr, uint32_t target, uint32_t* status, const uint32_t* sync,
                        long long ticks) {
    const long long t0 = wall_clock64();
    int sleep = 1;
    for (long n = 0;; ++n) {
        const uint32_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= target) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            return true;
        }
        if ((n & 15) == 15) {
            if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
            if (wall_clock64() - t0 > ticks || n >= (1L << 24)) {
                uint32_t zero = 0u;
                if (__hip_atomic_compare_exchange_strong(status, &zero, (uint32_t)MOE_ERR_TIMEOUT,
                                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)) {
                    status[1] = (uint32_t)(ctr - sync);
                    status[2] = target;
                    status[3] = v;
                }
                return false;
            }
        }
        if (sleep == 1) __builtin_amdgcn_s_sleep(1);
        else if (sleep == 2) __builtin_amdgcn_s_sleep(2);
        else if (sleep == 4) __builtin_amdgcn_s_sleep(4);
        else if (sleep == 8) __builtin_amdgcn_s_sleep(8);
        else __builtin_amdgcn_s_sleep(16);
        if (sleep < 16) sleep <<= 1;
    }
}

// threadIdx.x behind an empty asm: values the GEMM tile derives from it are
// recomputed per item instead of being kept live across the item loop.
__device__ __forceinline__ int fresh_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

struct LayerShared {
    int item, flag, old, nlist, nt;
    int list[32];  // tokens whose column block this FC2 tile completes
    float red[4];
};

// The block waits for *ctr >= target (thread 0 polls); false: give up. Every
// wave then acquires at agent scope itself before it reads what the counter
// guards.
__device__ __forceinline__ bool block_wait(const uint32_t* ctr, uint32_t target, const LayerArgs& a,
                                           LayerShared& ls) {
    if (threadIdx.x == 0) ls.flag = ls_wait(ctr, target, a.status, a.sync, a.wait_ticks) ? 1 : 0;
    __syncthreads();
    const bool ok = ls.flag != 0;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    return ok;
}

// Every wave releases its stores at agent scope; then thread 0 adds 1 to *ctr
// (release) and, with want_old, hands the previous value to the whole block
// (then an acquire: every wave, as in block_wait).
__device__ __forceinline__ int block_signal(uint32_t* ctr, LayerShared& ls, bool want_old) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t o = __hip_atomic_fetch_add(ctr, 1u, want_old ? __ATOMIC_ACQ_REL : __ATOMIC_RELEASE,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        ls.old = (int)o;
    }
    if (!want_old) return 0;
    __syncthreads();
    const int o = ls.old;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every wave, as in block_wait
    __syncthreads();
    return o;
}

// Next item of a queue for the whole block.
__device__ __forceinline__ int block_ticket(uint32_t* head, LayerShared& ls) {
    if (threadIdx.x == 0)
        ls.item = (int)__hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = ls.item;
    __syncthreads();
    return it;
}

// LDS of the permutation (256 threads, E <= 256, R <= kLayerMaxR).
struct PermShared {
    int32_t cnt[256];
    int32_t wh[4][256];
    int buf[16];
};

// Exclusive scan of three values over a 256-thread block.
__device__ __forceinline__ int3 block256_exclusive_scan3(int3 v, int* buf /*>= 12*/) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int3 x = make_int3(wave_incl_scan(v.x), wave_incl_scan(v.y), wave_incl_scan(v.z));
    if (lane == 63) { buf[3 * w] = x.x; buf[3 * w + 1] = x.y; buf[3 * w + 2] = x.z; }
    __syncthreads();
    int3 pre = make_int3(0, 0, 0);
    for (int ww = 0; ww < w; ++ww) { pre.x += buf[3 * ww]; pre.y += buf[3 * ww + 1]; pre.z += buf[3 * ww + 2]; }
    __syncthreads();
    return make_int3(pre.x + x.x - v.x, pre.y + x.y - v.y, pre.z + x.z - v.z);
}

// Expert counts, offsets, the four tile lists and the stable scatter of the
// routes, by one block of 256 threads: the same results as the permutation
// kernels (routes of an expert keep their route order).
__device__ void permute_block256(const int32_t* __restrict__ ids, int R, int E,
                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                 int32_t* __restrict__ tiles, int32_t* __restrict__ r2r,
                                 int32_t* __restrict__ rt2row, PermShared& s) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int kPer = kLayerMaxR / 256;
    int xs[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int r = tid + 256 * i;
        xs[i] = r < R ? ids[r] : -1;
    }
    s.cnt[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (xs[i] >= 0) atomicAdd(&s.cnt[xs[i]], 1);
    __syncthreads();
    const int run = tid < E ? s.cnt[tid] : 0;
    int nt[kNumBM];
#pragma unroll
    for (int i = 0; i < kNumBM; ++i) nt[i] = tid < E ? (run + bm_of(i) - 1) / bm_of(i) : 0;
    // all prefix sums stay below 2^16 (R <= 4096, tiles <= R/16 + E): two
    // scans share each word
    static_assert(kNumBM == 4, "packing below assumes four tile sizes");
    const int3 pk = block256_exclusive_scan3(make_int3(run | (nt[0] << 16), nt[1] | (nt[2] << 16), nt[3]), s.buf);
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
    s.cnt[tid] = tid < E ? off : 0;
    s.wh[0][tid] = s.wh[1][tid] = s.wh[2][tid] = s.wh[3][tid] = 0;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (256 * i >= R) break;
        const int r = 256 * i + tid;
        const bool valid = r < R;
        const int x = valid ? xs[i] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (x >> b) & 1;
            const uint64_t bal = __ballot(valid && bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid && rank == 0) s.wh[w][x] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int prior = 0;
            for (int ww = 0; ww < w; ++ww) prior += s.wh[ww][x];
            const int row = s.cnt[x] + prior + rank;
            if (row >= 0 && row < R) {
                r2r[row] = r;
                rt2row[r] = row;
            }
        }
        __syncthreads();
        s.cnt[tid] += s.wh[0][tid] + s.wh[1][tid] + s.wh[2][tid] + s.wh[3][tid];
        s.wh[0][tid] = s.wh[1][tid] = s.wh[2][tid] = s.wh[3][tid] = 0;
        __syncthreads();
    }
}

// NVFP4 of one row by one wave (lane l takes the 16-blocks l, l + 64, ...):
// global scale gg, or with gg < 0 the row's own amax / (6 * 448), or
// amax / (6 * 256) with F46 (then the 4-over-6 block choice); the scale goes
// to *g_out. Same arithmetic as the row quantization kernels.
template <bool BF16, bool F46>
__device__ void nv_row_wave(const void* v, size_t base, int cols, float gg, float* g_out,
                            uint8_t* codes, uint8_t* scales, uint16_t* deq, int lane) {
    const int nb = cols / 16;
    if (gg < 0.0f) {
        float m = 0.0f;
        for (int b = lane; b < nb; b += 64) {
            float vv[16];
            load16<BF16>(v, base + (size_t)b * 16, vv);
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(vv[i]));
        }
        m = wave_max(m);
        gg = __fdiv_rn(m, F46 ? 1536.0f : 2688.0f);
    }
    if (lane == 0) *g_out = gg;
    const size_t row = base / cols;
    for (int b = lane; b < nb; b += 64) {
        float vv[16];
        load16<BF16>(v, base + (size_t)b * 16, vv);
        uint32_t packed[2], sf;
        if (F46) nvfp4_block_4o6(vv, gg, packed, &sf);
        else nvfp4_block(vv, gg, packed, &sf);
        *reinterpret_cast<uint2*>(codes + base / 2 + (size_t)b * 8) = make_uint2(packed[0], packed[1]);
        scales[row * nb + b] = (uint8_t)sf;
        uint32_t h[8];
        nvfp4_deq_f16(packed, sf, h);
        uint4* dst = reinterpret_cast<uint4*>(deq + base + (size_t)b * 16);
        dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
}

// MXFP8 of one bf16 row by one wave.
__device__ void mx8_row_wave(const uint16_t* x, int row, int cols, uint8_t* codes, uint8_t* scales,
                             int lane) {
    const size_t base = (size_t)row * cols;
    const int nb = cols / 32;
    for (int b = lane; b < nb; b += 64) {
        float vv[32];
        load16<true>(x, base + (size_t)b * 32, vv);
        load16<true>(x, base + (size_t)b * 32 + 16, vv + 16);
        uint8_t c[32];
        const uint32_t e8 = mxfp8_block(vv, c);
        uint4* dst = reinterpret_cast<uint4*>(codes + base + (size_t)b * 32);
        dst[0] = *reinterpret_cast<const uint4*>(c);
        dst[1] = *reinterpret_cast<const uint4*>(c + 16);
        scales[(size_t)row * nb + b] = (uint8_t)e8;
    }
}

// The per-tensor global scale from the partial maxima (one per lane).
__device__ __forceinline__ float tensor_scale(const uint32_t* slot, int lane) {
    const float am = wave_max(lane < kAmaxSlots ? u2f(slot[(size_t)lane * kAmaxStride]) : 0.0f);
    return __fdiv_rn(am, 2688.0f);
}

}  // namespace

// XQ (a LayerXq) is a template argument, so each kernel holds only the
// quantization code its mode runs (fewer registers).
template <int AB, int BM, int WN1, int XQ>
__global__ __launch_bounds__(256) void layer_kernel(LayerArgs args) {
    constexpr int P = 3, NW = 4;
    union Smem {
        GemmSmem<AB, BM, P> g;
        PermShared perm;
    };
    __shared__ Smem sm;
    __shared__ LayerShared ls;
    // The arguments live in LDS for the whole launch: the item loop then
    // reloads what it needs per item instead of holding every argument in
    // scalar registers across it (which spilled).
    __shared__ LayerArgs a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        a = args;
        ls.flag = __hip_atomic_load(args.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
    }
    __syncthreads();
    if (!ls.flag) return;  // blob header mismatch found by the prologue
    __syncthreads();
    uint32_t* const sync = a.sync;
    const int T = a.T, H = a.H, E = a.E, K = a.K, R = T * K;
    constexpr bool nv = XQ >= LX_NV_ROW;
    constexpr bool tensor = XQ == LX_NV_TENSOR;

    // ---- phase 1: routing + permutation, FC1-input quantization ----
    const int n_route = (T + 3) / 4;
    const int n_xamax = tensor ? (int)(((size_t)T * H + kXAmaxChunk - 1) / kXAmaxChunk) : 0;
    const int n_xq = XQ != LX_NONE ? (T + 3) / 4 : 0;
    const int n1 = n_route + n_xamax + n_xq;
    for (;;) {
        const int it = block_ticket(&sync[kLsQueue1], ls);
        if (it >= n1) break;
        if (it < n_route) {
            const int t = it * 4 + wave;
            if (t < T)
                route_one_token<4>(a.logits + (size_t)t * E, E, K, lane, a.ids + (size_t)t * K,
                                   a.topw + (size_t)t * K);
            const int done = block_signal(&sync[kLsRouted], ls, true);
            if (done == n_route - 1) {  // every route is in: permute, then publish
                permute_block256(a.ids, R, E, a.counts, a.offsets, a.tiles, a.r2r, a.rt2row, sm.perm);
                block_signal(&sync[kLsPlan], ls, false);
            }
        } else if (it < n_route + n_xamax) {
            const size_t n = (size_t)T * H;
            const size_t c0 = (size_t)(it - n_route) * kXAmaxChunk;
            float m = 0.0f;
#pragma unroll
            for (int u = 0; u < kXAmaxChunk / 256 / 16; ++u) {
                const size_t i = c0 + ((size_t)u * 256 + tid) * 16;
                if (i < n) {  // T * H is a multiple of 16
                    float q[16];
                    load16<true>(a.x, i, q);
#pragma unroll
                    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(q[j]));
                }
            }
            m = wave_max(m);
            if (lane == 0) ls.red[wave] = m;
            __syncthreads();
            if (tid == 0)
                atomicMax(a.misc + kMiscXAmax + (size_t)((it - n_route) % kAmaxSlots) * kAmaxStride,
                          f2u(fmaxf(fmaxf(ls.red[0], ls.red[1]), fmaxf(ls.red[2], ls.red[3]))));
            block_signal(&sync[kLsXAmax], ls, false);
        } else {
            if (tensor && !block_wait(&sync[kLsXAmax], (uint32_t)n_xamax, a, ls)) return;
            const int row = (it - n_route - n_xamax) * 4 + wave;
            if (row < T) {
                if constexpr (XQ == LX_MX8) {
                    mx8_row_wave(a.x, row, H, a.xcodes, a.xscales, lane);
                } else if constexpr (nv) {
                    const float gg = tensor ? tensor_scale(a.misc + kMiscXAmax, lane) : -1.0f;
                    nv_row_wave<true, XQ == LX_NV_ROW_4O6>(a.x, (size_t)row * H, H, gg, a.xg + row,
                                                            a.xcodes, a.xscales, a.xdeq, lane);
                }
            }
            block_signal(&sync[kLsXDone], ls, false);
        }
    }

    // ---- phase 2: FC1, FC2-input quantization, FC2 + finalize ----
    if (!block_wait(&sync[kLsPlan], 1u, a, ls)) return;
    if (n_xq && !block_wait(&sync[kLsXDone], (uint32_t)n_xq, a, ls)) return;
    const GemmArgs& g1 = a.g1;
    const GemmArgs& g2 = a.g2;
    const int nb1 = g1.N / (16 * NW * WN1);
    const int nb2 = H / (16 * NW * 2);
    // M-tiles of this forward: read once and broadcast, so that every wave
    // walks the queues (and their barriers) alike
    if (tid == 0) ls.nt = g1.tiles[E];
    __syncthreads();
    const int nt = ls.nt;
    const int per = (nt + 7) >> 3;
    uint32_t* const fc1_done = sync + kLsFixed;
    uint32_t* const a2q_done = fc1_done + a.mt_max;
    uint32_t* const tok_cnt = a2q_done + a.mt_max;
    const int n_a2q = nv ? 1 : 0;
    for (int qi = 0; qi < 8; ++qi) {
        const int q = (int)((blockIdx.x + qi) & 7);
        const int mt0 = q * per;
        const int mtn = max(0, min(nt, mt0 + per) - mt0);
        const int n_fc1 = mtn * nb1, n_q = mtn * n_a2q;
        const int nq = n_fc1 + n_q + mtn * nb2;
        if (nq == 0) continue;
        for (;;) {
            const int it = block_ticket(&sync[kLsHeads + q * kLsLine], ls);
            if (it >= nq) break;
            if (it < n_fc1) {
                const int mt = mt0 + it / nb1;
                const TileLoc loc = tile_locate<BM>(g1, mt, lane);
                gemm_tile_run<AB, BM, WN1, EPI_FC1, P, NW>(g1, sm.g, loc, it % nb1, false, fresh_tid());
                block_signal(&fc1_done[mt], ls, false);
                if (tensor) block_signal(&sync[kLsFc1All], ls, false);
            } else if (nv && it < n_fc1 + n_q) {
                // FC2-input quantization of one M-tile's rows (NVFP4)
                const int mt = mt0 + (it - n_fc1);
                if (tensor) {
                    if (!block_wait(&sync[kLsFc1All], (uint32_t)(nt * nb1), a, ls)) return;
                } else if (!block_wait(&fc1_done[mt], (uint32_t)nb1, a, ls)) {
                    return;
                }
                const TileLoc loc = tile_locate<BM>(g1, mt, lane);
                const float gg = tensor ? tensor_scale(a.misc + kMiscA2Amax, lane) : -1.0f;
                for (int m = wave; m < loc.rows; m += NW) {
                    const int row = loc.row0 + m;
                    nv_row_wave<false, XQ == LX_NV_ROW_4O6>(a.a2f, (size_t)row * a.I, a.I, gg, a.a2g + row,
                                                            a.a2codes, a.a2scales, a.a2deq, lane);
                }
                block_signal(&a2q_done[mt], ls, false);
            } else {
                const int j = it - n_fc1 - n_q;
                const int mt = mt0 + j / nb2, nb = j % nb2;
                if (!block_wait(nv ? &a2q_done[mt] : &fc1_done[mt], nv ? 1u : (uint32_t)nb1, a, ls))
                    return;
                const TileLoc loc = tile_locate<BM>(g2, mt, lane);
                gemm_tile_run<AB, BM, 2, EPI_FC2, P, NW>(g2, sm.g, loc, nb, false, fresh_tid());
                // count this column block's contributions per token
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                if (tid == 0) ls.nlist = 0;
                __syncthreads();
                if (tid < loc.rows) {
                    const int t = a.r2r[loc.row0 + tid] / K;
                    const uint32_t o = __hip_atomic_fetch_add(&tok_cnt[(size_t)t * nb2 + nb], 1u,
                                                              __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                    if (o == (uint32_t)K - 1u) ls.list[atomicAdd(&ls.nlist, 1)] = t;
                }
                __syncthreads();
                const int nl = ls.nlist;
                if (nl) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    const int col = nb * 128 + (tid & 127);
                    for (int i = tid >> 7; i < nl; i += 2) {
                        const int t = ls.list[i];
                        float acc = 0.0f;
                        for (int k = 0; k < K; ++k) {
                            const int row = a.rt2row[(size_t)t * K + k];
                            const float wk = g2.on_input ? 1.0f : a.topw[(size_t)t * K + k];
                            acc = __fmaf_rn(wk, g2.out_f32[(size_t)row * H + col], acc);
                        }
                        a.y[(size_t)t * H + col] = bf16_rne(acc);
                    }
                }
                __syncthreads();
            }
        }
    }
}

// Header check and clearing of the sync words and of the misc words (amax
// slots) before the layer kernel (a kernel cannot clear counters that its
// own blocks may already be using).
__global__ __launch_bounds__(256) void layer_prologue_kernel(uint32_t* __restrict__ sync, size_t nsync,
                                                             uint32_t* __restrict__ misc,
                                                             const uint32_t* __restrict__ blob,
                                                             BlobHeader expect,
                                                             uint32_t* __restrict__ status) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nsync; i += (size_t)gridDim.x * 256)
        sync[i] = 0u;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < (size_t)kMiscWords; i += (size_t)gridDim.x * 256)
        misc[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x < 64) {
        constexpr int kWords = sizeof(BlobHeader) / 4;
        static_assert(kWords <= 64, "one header word per lane");
        const uint32_t* ew = reinterpret_cast<const uint32_t*>(&expect);
        const int l = threadIdx.x;
        const bool differs = l < kWords && blob[l] != ew[l];
        const uint64_t any = __ballot(differs);
        if (l == 0) *status = any ? (uint32_t)MOE_ERR_INVALID : 0u;
    }
}

// Blocks of one layer-kernel configuration the current device holds at once,
// cached per configuration and device.
template <int AB, int BM, int WN1, int XQ>
static int layer_resident_blocks() {
    static std::atomic<int> cache[64];  // value + 1; 0 = not yet asked
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, layer_kernel<AB, BM, WN1, XQ>, 256, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = per_cu * cus + 1;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c - 1;
}

template <int AB, int BM, int WN1, int XQ>
static hipError_t launch_layer_cfg(const LayerArgs& a, int max_items, hipStream_t s, hipEvent_t t0,
                                   hipEvent_t t1) {
    auto kern = layer_kernel<AB, BM, WN1, XQ>;
    int grid = layer_resident_blocks<AB, BM, WN1, XQ>();
    if (grid <= 0) grid = 256;
    grid = std::min(grid, max_items);  // no more blocks than work items
    grid = std::max(8, grid / 8 * 8);  // every XCD queue has home blocks
    if (t0) hipExtLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, t0, t1, 0, a);
    else hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

bool layer_supported(int R, int E, int bm_index, int mode) {
    // Switched off for every shape. On the GPU the kernel completed in the
    // per-tensor NVFP4 mode (bit-identical to the multi-launch forward), but
    // it did not finish in the per-row NVFP4 mode and then in the W4A16 mode,
    // the two runs in which FC2 (or the FC2-input quantization) waits on a
    // per-M-tile FC1 counter while other FC1 tiles still run. The hang
    // outlasted every bounded wait of the kernel, so it is not a lost counter
    // update; its cause is not found. The shape test stays for when it is.
    (void)R; (void)E; (void)bm_index; (void)mode;
    return false;
}

hipError_t launch_layer(const LayerArgs& args, int ab, const void* blob, const BlobHeader& expect,
                        size_t sync_words, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    LayerArgs a = args;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        khz = 100000;
    a.wait_ticks = (long long)khz * 250;  // a quarter of a second per wait
    const int pro_grid = (int)std::min<size_t>(64, (sync_words + kMiscWords + 4095) / 4096);
    hipLaunchKernelGGL(layer_prologue_kernel, dim3(pro_grid), dim3(256), 0, s, a.sync, sync_words,
                       a.misc, static_cast<const uint32_t*>(blob), expect, a.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool bm16 = a.bmi == 0;
    const int N1 = a.g1.N;
    const bool qf = N1 % 256 == 0;  // MXFP8 FC1 quantizes whole 32-column blocks per wave
    // work items at most: phase 1, then per M-tile the FC1 and FC2 tiles and
    // one quantization item
    const int nb1 = N1 / (ab == AB_FP8 && qf ? 256 : 128), nb2 = a.H / 128;
    const long long items = 3LL * ((a.T + 3) / 4) + (long long)a.mt_max * (nb1 + nb2 + 1) +
                            ((long long)a.T * a.H + 16383) / 16384;
    const int max_items = (int)std::min<long long>(items, 1 << 20);
#define LL(AB_, WN_, XQ_) (bm16 ? launch_layer_cfg<AB_, 16, WN_, XQ_>(a, max_items, s, t0, t1) \
                                : launch_layer_cfg<AB_, 32, WN_, XQ_>(a, max_items, s, t0, t1))
    if (ab == AB_BF16_NV) return LL(AB_BF16_NV, 2, LX_NONE);
    if (ab == AB_FP8) return qf ? LL(AB_FP8, 4, LX_MX8) : LL(AB_FP8, 2, LX_MX8);
    if (a.xq == LX_NV_TENSOR) return LL(AB_F16_NV, 2, LX_NV_TENSOR);
    return hipErrorInvalidValue;  // per-row NVFP4 modes take the multi-launch sequence
#undef LL
}

}  // namespace moe
