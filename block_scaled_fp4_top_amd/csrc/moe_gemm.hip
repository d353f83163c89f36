// S4/S6 grouped GEMMs: the standalone kernels (one launch per GEMM) and their
// host launchers. The tile itself (K loop, operand formats, epilogues) is in
// moe_gemm_tile.h.
#include <hip/hip_ext.h>

#include <atomic>

#include "moe_gemm_tile.h"

namespace moe {

// Standalone grouped-GEMM kernel: block blockIdx.x -> (M-tile, N-block) in an
// XCD-aware order, then one tile.
template <int AB, int BM, int WN, int EPI, int P, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs p) {
    __shared__ GemmSmem<AB, BM, P> sm;
    const int lane = threadIdx.x & 63;
    const int vb = blockIdx.x, nvb = gridDim.x;
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
    //  - Wide tiles, FC2 with the fused finalize into a token accumulator larger
    //    than the last-level cache: N-block slowest for the whole chip (every
    //    XCD takes one contiguous range of M-tiles per N-block), so the
    //    atomics of a phase land on one N-block's columns of the accumulator
    //    (T x 512 x 4 bytes), which stay cache-resident; an expert's M-tiles
    //    still share one XCD's L2 for their weights.
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
        const int j = vb >> 3;
        const int w = (vb & 7) * per + j;
        if (j >= per || w >= work) return;
        mt = w / NB;
        nb = w % NB;
        fair = work <= p.resident;
    } else if (EPI == EPI_FC2 && p.phased) {
        const int NB = p.N / (16 * NW * WN);
        const int act = p.tiles[p.E];
        const int per = (act + 7) >> 3;
        if (per == 0) return;  // no rows (a forward always has some)
        const int j = vb >> 3;
        nb = j / per;
        mt = (vb & 7) * per + j % per;
        if (nb >= NB || mt >= act) return;
    } else {
        const int id = (vb & 7) * (nvb >> 3) + (vb >> 3);
        mt = id % p.mt_max;
        nb = id / p.mt_max;
        if (nb >= p.N / (16 * NW * WN) || mt >= p.tiles[p.E]) return;
    }
    const TileLoc loc = tile_locate<BM>(p, mt, lane);
    if (status) return;  // blob prepared for other dimensions: no weight reads, no stores
    gemm_tile_run<AB, BM, WN, EPI, P, NW>(p, sm, loc, nb, fair, threadIdx.x);
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
    long long blocks = (long long)(a.N / (16 * NW * WN)) * a.mt_max;
    if (BM > 32 && EPI == EPI_FC2 && a.phased)  // room for 8 ranges of ceil(mt_max / 8) per N-block
        blocks = 8LL * (a.N / (16 * NW * WN)) * ((a.mt_max + 7) / 8);
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
