// Internal layout definitions and device codecs of the HIP path.
//
// Element formats follow the OCP Microscaling Formats (MX) v1.0 definitions
// (E2M1, E4M3 "FN", E8M0). NVFP4 = E2M1 elements with an E4M3 scale per 16
// elements and an FP32 global scale g = amax / (6 * 448); MXFP8 = E4M3
// elements with an E8M0 scale per 32 elements (MegaMoE post, "Our approach":
// block-16 and block-32 scaling).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_fp4.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kTileK = 128;         // K extent of one weight micro-tile
constexpr int kStrip = 16;          // N rows of one weight micro-tile
constexpr int kNvTileBytes = 1024;  // NVFP4 codes of a 16 x 128 micro-tile
constexpr int kNvTileScale = 128;   // its 16 x 8 E4M3 scales
constexpr int kF8TileBytes = 2048;  // MXFP8 codes of a 16 x 128 micro-tile
constexpr int kF8TileScale = 64;    // its 16 x 4 E8M0 scales
constexpr int kF4TileBytes = 1024;  // MXFP4 codes of a 16 x 128 micro-tile
constexpr int kF4TileScale = 64;    // its 16 x 4 E8M0 scales
constexpr int kPermChunk = 1024;    // routes per block in the permutation kernels
constexpr int kNumBM = 4;           // M-tile sizes with a device tile list
__host__ __device__ constexpr int bm_of(int i) { return 16 << i; }  // 16, 32, 64, 128
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr uint32_t kBlobMagic0 = 0x5746454Du;  // "MEFW"
constexpr uint32_t kBlobMagic1 = 0x34504634u;  // "4FP4"
constexpr uint32_t kBlobVersion = 2;
constexpr size_t kBlobHeader = 4096;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Prepared weight blob
// ---------------------------------------------------------------------------
// [header 4096 B][g1: E f32][g2: E f32][amax scratch: 2E u32]
// [W1 codes][W1 scales][W2 codes][W2 scales]
// Each weight matrix W[N][K] (N1 x H for W1, H x I for W2) is cut into
// micro-tiles of 16 rows x 128 k stored tile-row-major: tile (nt, kt) at
// (nt * K/128 + kt) * tile_bytes. Inside a tile the bytes are the exact
// register image a 64-lane wave feeds to the matrix cores:
//  NVFP4 (16x16x32 bf16/f16 MFMA after dequantization): lane l owns 16 bytes at
//    l*16; row n = l % 16; dword j (0..3) holds the 8 codes
//    k = 32 j + 8 (l / 16) + [0, 8), element i in nibble i (low nibble first).
//    Scales: 32 dwords; dword (l >> 5) * 16 + (l & 15) holds, in byte j, the
//    E4M3 scale of row l % 16 for 16-block 2 j + (l >> 5) of the tile.
//  MXFP8 (16x16x128 scaled f8f6f4 MFMA): lane l owns 32 bytes at l*32; row
//    n = l % 16, q = l / 16; byte b < 16 is k = 16 q + b, byte b >= 16 is
//    k = 64 + 16 q + (b - 16). Scales: byte l is the E8M0 scale of row l % 16
//    for 32-block l / 16 of the tile.
// Scales are not stored per micro-tile but per group of four strips
// (kScaleGroup) and K step: one block of 4 x (a micro-tile's scale bytes) in
// which each lane's scale units of the four strips lie side by side (unit:
// the lane's E8M0 byte for MXFP8 and MXFP4, its dword of four E4M3 bytes for
// NVFP4), so a wave reads the scales of its 2 or 4 strips for one K step with
// one load (wscale_offset).
// SwiGLU W1 rows are interleaved by strips of 16: prepared strip 2s holds gate
// rows [16 s, 16 s + 16) and strip 2s + 1 the up rows I + [16 s, 16 s + 16), so
// one wave sees matching gate/up accumulators in the same lanes.
struct BlobHeader {
    uint32_t magic0, magic1, version, wfmt;
    int32_t E, H, I, N1, act, pad0;
    uint64_t off_g1, off_g2, off_amax, off_w1, off_s1, off_w2, off_s2, total;
};

constexpr int kScaleGroup = 4;
// Byte offset of scale unit `unit_index` (tile-local numbering as above) of
// strip nt, K step kt, expert e, in one matrix family's scale array
// (expert_tiles micro-tiles per expert, KT steps, tile_scale_bytes per tile).
__host__ __device__ inline size_t wscale_offset(size_t expert_tiles, int e, int nt, int kt, int KT,
                                                int tile_scale_bytes, int unit_index, int unit_bytes) {
    return (size_t)e * expert_tiles * tile_scale_bytes +
           ((size_t)(nt / kScaleGroup) * KT + kt) * (size_t)(kScaleGroup * tile_scale_bytes) +
           (size_t)unit_index * (kScaleGroup * unit_bytes) + (size_t)(nt % kScaleGroup) * unit_bytes;
}

struct BlobLayout {
    BlobHeader h;
    size_t w_tile_bytes, s_tile_bytes;
};

inline bool make_blob_layout(const moe_dims& d, BlobLayout* L) {
    BlobHeader& h = L->h;
    h.magic0 = kBlobMagic0;
    h.magic1 = kBlobMagic1;
    h.version = kBlobVersion;
    h.wfmt = (uint32_t)d.wfmt;
    h.E = d.E;
    h.H = d.H;
    h.I = d.I;
    h.N1 = d.act == MOE_ACT_SWIGLU ? 2 * d.I : d.I;
    h.act = d.act;
    h.pad0 = 0;
    const bool nv = d.wfmt == MOE_FMT_NVFP4;
    const bool mx4 = d.wfmt == MOE_FMT_MXFP4;
    L->w_tile_bytes = nv ? kNvTileBytes : (mx4 ? kF4TileBytes : kF8TileBytes);
    L->s_tile_bytes = nv ? kNvTileScale : (mx4 ? kF4TileScale : kF8TileScale);
    const size_t E = (size_t)d.E;
    const size_t t1 = (size_t)(h.N1 / kStrip) * (size_t)(d.H / kTileK);  // tiles per expert
    const size_t t2 = (size_t)(d.H / kStrip) * (size_t)(d.I / kTileK);
    size_t off = kBlobHeader;
    h.off_g1 = off; off = align256(off + E * 4);
    h.off_g2 = off; off = align256(off + E * 4);
    h.off_amax = off; off = align256(off + 2 * E * 4);
    h.off_w1 = off; off = align256(off + E * t1 * L->w_tile_bytes);
    h.off_s1 = off; off = align256(off + E * t1 * L->s_tile_bytes);
    h.off_w2 = off; off = align256(off + E * t2 * L->w_tile_bytes);
    h.off_s2 = off; off = align256(off + E * t2 * L->s_tile_bytes);
    h.total = off;
    return true;
}

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------
// misc region (u32 words), cleared by the routing kernel of every forward:
// the x amax and the FC2-input amax, each as kAmaxSlots partial maxima on
// separate 128-byte lines (kAmaxStride words apart), from words kMiscXAmax
// and kMiscA2Amax. Writers spread their atomics over the slots (one shared
// word made the per-tensor decode FC1 14 % slower and the x amax pass 20 us
// long from atomic contention); readers take the max.
constexpr int kAmaxSlots = 32, kAmaxStride = 32;
constexpr int kMiscXAmax = 0, kMiscA2Amax = kAmaxSlots * kAmaxStride;
constexpr int kMiscWords = 2 * kAmaxSlots * kAmaxStride;

// The first kWsStatusBytes of a forward's workspace hold its status word:
// the routing kernel writes 0, or MOE_ERR_INVALID when the prepared blob's
// header does not match the dimensions of the call; the kernels that read the
// weights or write the output skip their work when it is not 0.
constexpr size_t kWsStatusBytes = 256;

enum WsView {
    V_IDS = 0, V_TOPW, V_COUNTS, V_OFFSETS, V_R2R, V_RT2ROW,
    V_XCODES, V_XSCALES, V_XG, V_A2F, V_A2CODES, V_A2SCALES, V_A2G, V_O,
    V_XMXCODES, V_XMXSCALES, V_A2MXCODES, V_A2MXSCALES,  // MXFP4 re-blocked operands
    V_NUM_PUBLIC,
    V_TILES = V_NUM_PUBLIC, V_BHIST, V_MISC, V_XDEQ, V_A2DEQ, V_ARRIVE, V_NUM
};

struct WsPlan {
    size_t off[V_NUM];
    size_t bytes[V_NUM];
    size_t total;
    int nblk;  // permutation blocks
};

inline void plan_workspace(const moe_dims& d, int T, int K, int mode, WsPlan* p) {
    const size_t R = (size_t)T * K, E = (size_t)d.E, H = (size_t)d.H, I = (size_t)d.I;
    const bool mx4 = mode == MOE_W4A4_TOKEN_MXFP4;
    const bool nv4 = mode == MOE_W4A4_TENSOR || mode == MOE_W4A4_TOKEN || mode == MOE_W4A4_TOKEN_4O6 || mx4;
    const bool f8 = mode == MOE_MXFP8;
    p->nblk = (int)((R + kPermChunk - 1) / kPermChunk);
    for (int v = 0; v < V_NUM; ++v) p->bytes[v] = 0;
    p->bytes[V_IDS] = R * 4;
    p->bytes[V_TOPW] = R * 4;
    p->bytes[V_COUNTS] = E * 4;
    p->bytes[V_OFFSETS] = (E + 1) * 4;
    p->bytes[V_R2R] = R * 4;
    p->bytes[V_RT2ROW] = R * 4;
    p->bytes[V_TILES] = (size_t)kNumBM * (E + 1) * 4;
    p->bytes[V_BHIST] = (size_t)p->nblk * E * 4 * 2;
    p->bytes[V_MISC] = kMiscWords * 4;
    if (nv4) {
        p->bytes[V_XCODES] = (size_t)T * H / 2;
        p->bytes[V_XSCALES] = (size_t)T * H / 16;
        p->bytes[V_XG] = (size_t)T * 4;
        p->bytes[V_XDEQ] = (size_t)T * H * 2;
        p->bytes[V_A2F] = R * I * 4;
        p->bytes[V_A2CODES] = R * I / 2;
        p->bytes[V_A2SCALES] = R * I / 16;
        p->bytes[V_A2G] = R * 4;
        p->bytes[V_A2DEQ] = R * I * 2;
        if (mx4) {  // the GEMMs read the re-blocked MXFP4 operands, no fp16 copies
            p->bytes[V_XDEQ] = p->bytes[V_A2DEQ] = 0;
            p->bytes[V_XMXCODES] = (size_t)T * H / 2;
            p->bytes[V_XMXSCALES] = (size_t)T * H / 32;
            p->bytes[V_A2MXCODES] = R * I / 2;
            p->bytes[V_A2MXSCALES] = R * I / 32;
        }
    } else if (f8) {
        p->bytes[V_XCODES] = (size_t)T * H;
        p->bytes[V_XSCALES] = (size_t)T * H / 32;
        // the FC2 input is quantized in the FC1 epilogue: no fp32 copy
        p->bytes[V_A2CODES] = R * I;
        p->bytes[V_A2SCALES] = R * I / 32;
    } else {
        p->bytes[V_A2F] = R * I * 2;  // bf16 FC2 input
    }
    p->bytes[V_O] = R * H * 4;
    // fused finalize: one arrival counter per token and FC2 N-block (N-blocks
    // are at least 128 columns wide)
    p->bytes[V_ARRIVE] = (size_t)T * (H / 128) * 4;
    size_t off = kWsStatusBytes;
    for (int v = 0; v < V_NUM; ++v) {
        p->off[v] = off;
        off = align256(off + p->bytes[v]);
    }
    p->total = off;
}

// ---------------------------------------------------------------------------
// Device codecs (written independently of any reference implementation)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// E2M1 round-to-nearest-even with saturation (the midpoints 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5 go to the neighbour whose mantissa bit is 0; above 6 the
// code saturates to 6; the sign is kept, also for zero) by the hardware
// converter at unit scale: two values into the byte `sel` of `old`, the first
// in the low nibble. Checked on the GPU against the threshold form of that
// rule on every fp32 in [2^-3, 8) of both signs, zeros, subnormals and values
// up to 3.4e38: no difference.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, float u0, float u1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, u0, u1, 1.0f, SEL);
}

// E4M3 "FN" round-to-nearest-even, saturating to +-448, from the fp32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t s = (f2u(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a < 448.0f)) return s | 0x7Eu;
    if (a < 0.015625f) {                      // below 2^-6: subnormal grid m * 2^-9
        const float q = a * 512.0f;           // exact
        return s | (uint32_t)__builtin_rintf(q);  // 0..8; 8 is the first normal (0x08)
    }
    const uint32_t u = f2u(a);
    int e = (int)((u >> 23) & 0xFF) - 127;     // -6 .. 8
    uint32_t keep = (u >> 20) & 7u;
    const uint32_t rem = u & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) { keep = 0; ++e; }
    uint32_t c = ((uint32_t)(e + 7) << 3) | keep;
    if (c > 0x7Eu) c = 0x7Eu;
    return s | c;
}

// Two E4M3 codes (x0 in bits 0..7, x1 in bits 8..15) by the hardware
// converter, which rounds to nearest even; clamping to +-448 first gives the
// saturating result of e4m3_code for every finite input.
__device__ __forceinline__ uint32_t e4m3_code2(float x0, float x1) {
    x0 = fminf(fmaxf(x0, -448.0f), 448.0f);
    x1 = fminf(fmaxf(x1, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
}

// Value of a non-NaN E4M3 code.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t ef = (c >> 3) & 15u, m = c & 7u;
    float v = ef ? u2f(((ef + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -v : v;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The 8 E2M1 values of one 32-bit word (element i in nibble i) as fp32, by the
// hardware converter at unit scale (exact for every code).
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float* out) {
    const f32x2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    out[0] = c0[0]; out[1] = c0[1]; out[2] = c1[0]; out[3] = c1[1];
    out[4] = c2[0]; out[5] = c2[1]; out[6] = c3[0]; out[7] = c3[1];
}

// floor(log2(a)) for a finite a > 0, exactly, from the fp32 bits.
__device__ __forceinline__ int floor_log2(float a) {
    const uint32_t u = f2u(a);
    const int e = (int)((u >> 23) & 0xFF);
    if (e) return e - 127;
    return (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;
}

// bf16 round-to-nearest-even of a finite fp32.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = f2u(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// NVFP4 quantization of one 16-element block with global scale g:
//   s = a_b / (6 g), sf = E4M3(s), d = float(sf) * g, code_i = E2M1(v_i / d);
// every operation is one IEEE fp32 operation in this order. g == 0 or d == 0
// leaves only the sign bit of each code. Writes 8 packed bytes (even element in
// the low nibble) to `codes`, the scale byte, and returns the codes' block as
// two u32 for callers that dequantize.
__device__ __forceinline__ void nvfp4_block(const float* v, float g, uint32_t* packed /*[2]*/,
                                            uint32_t* sf_out) {
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
    uint32_t sf = 0;
    float d = 0.0f;
    if (g != 0.0f) {
        const float six_g = __fmul_rn(6.0f, g);
        sf = e4m3_code(__fdiv_rn(ab, six_g));
        d = __fmul_rn(e4m3_value(sf), g);
    }
    uint32_t w0 = 0, w1 = 0;
    if (d != 0.0f) {
        float u[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) u[i] = __fdiv_rn(v[i], d);
        w0 = e2m1_pair<0>(w0, u[0], u[1]);
        w0 = e2m1_pair<1>(w0, u[2], u[3]);
        w0 = e2m1_pair<2>(w0, u[4], u[5]);
        w0 = e2m1_pair<3>(w0, u[6], u[7]);
        w1 = e2m1_pair<0>(w1, u[8], u[9]);
        w1 = e2m1_pair<1>(w1, u[10], u[11]);
        w1 = e2m1_pair<2>(w1, u[12], u[13]);
        w1 = e2m1_pair<3>(w1, u[14], u[15]);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t c = (f2u(v[i]) >> 28) & 8u;  // only the sign survives
            if (i < 8) w0 |= c << (4 * i); else w1 |= c << (4 * (i - 8));
        }
    }
    packed[0] = w0;
    packed[1] = w1;
    *sf_out = sf;
}

// One NVFP4 candidate for a 16-element block with block max `ab` mapped to
// `top` (6: the usual mapping, 4: the alternative of the 4-over-6 choice):
// s = ab / (top g), sf = E4M3(s), d = float(sf) g, codes E2M1(v / d), each one
// IEEE fp32 operation in this order (d == 0: sign-only codes). Returns the
// block's sum of squared errors sum_i (v_i - code_i d)^2, accumulated in fp64
// in element order with every operation rounded once (no contraction), so the
// choice between candidates is reproducible bit for bit.
__device__ __forceinline__ double nvfp4_candidate(const float* v, float g, float ab, float top,
                                                  uint32_t* packed, uint32_t* sf_out) {
    const uint32_t sf = e4m3_code(__fdiv_rn(ab, __fmul_rn(top, g)));
    const float d = __fmul_rn(e4m3_value(sf), g);
    uint32_t w0 = 0, w1 = 0;
    if (d != 0.0f) {
        float u[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) u[i] = __fdiv_rn(v[i], d);
        w0 = e2m1_pair<0>(w0, u[0], u[1]);
        w0 = e2m1_pair<1>(w0, u[2], u[3]);
        w0 = e2m1_pair<2>(w0, u[4], u[5]);
        w0 = e2m1_pair<3>(w0, u[6], u[7]);
        w1 = e2m1_pair<0>(w1, u[8], u[9]);
        w1 = e2m1_pair<1>(w1, u[10], u[11]);
        w1 = e2m1_pair<2>(w1, u[12], u[13]);
        w1 = e2m1_pair<3>(w1, u[14], u[15]);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t c = (f2u(v[i]) >> 28) & 8u;
            if (i < 8) w0 |= c << (4 * i); else w1 |= c << (4 * (i - 8));
        }
    }
    float c[16];
    e2m1x8_to_f32(w0, c);
    e2m1x8_to_f32(w1, c + 8);
    double e = 0.0;
    const double dd = (double)d;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double diff = __dsub_rn((double)v[i], __dmul_rn((double)c[i], dd));
        e = __dadd_rn(e, __dmul_rn(diff, diff));
    }
    packed[0] = w0;
    packed[1] = w1;
    *sf_out = sf;
    return e;
}

// NVFP4 "4-over-6" quantization of one 16-element block with the global scale
// g = amax / (6 * 256) of its row: the max-to-6 and the max-to-4 candidates,
// and the one with the smaller squared error (ties to max-to-6). g == 0 gives
// scale 0 and sign-only codes.
__device__ __forceinline__ void nvfp4_block_4o6(const float* v, float g, uint32_t* packed,
                                                uint32_t* sf_out) {
    if (g == 0.0f) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t c = (f2u(v[i]) >> 28) & 8u;
            if (i < 8) w0 |= c << (4 * i); else w1 |= c << (4 * (i - 8));
        }
        packed[0] = w0;
        packed[1] = w1;
        *sf_out = 0;
        return;
    }
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
    uint32_t p6[2], s6, p4[2], s4;
    const double e6 = nvfp4_candidate(v, g, ab, 6.0f, p6, &s6);
    const double e4 = nvfp4_candidate(v, g, ab, 4.0f, p4, &s4);
    const bool four = e4 < e6;
    packed[0] = four ? p4[0] : p6[0];
    packed[1] = four ? p4[1] : p6[1];
    *sf_out = four ? s4 : s6;
}

// Re-blocking of one NVFP4 32-element block (two 16-blocks: 16 bytes of packed
// codes, two E4M3 scale codes) to MXFP4 (OCP MX v1.0 rule for E2M1 elements):
// the local values w = E2M1(code) * E4M3(sf) (at most 6 significant bits: exact
// in fp32), X = floor(log2 max|w|) - 2, codes E2M1_RNE(w * 2^-X) (exact
// product; the hardware converter rounds to nearest even, saturates and keeps
// the sign, also of zeros); an all-zero block gets X = -127 and sign-only
// codes. Writes the 16 packed MXFP4 bytes and returns the E8M0 code X + 127.
// The NVFP4 global scale is not involved (w spans [2^-10, 2688], so
// X lies in [-12, 9]).
__device__ __forceinline__ uint32_t mxfp4_reblock32(const uint32_t* nv /*[4]*/, uint32_t sf0,
                                                    uint32_t sf1, uint32_t* mx /*[4]*/) {
    float w[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) e2m1x8_to_f32(nv[j], w + 8 * j);
    const float s0 = e4m3_value(sf0), s1 = e4m3_value(sf1);
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        w[i] = __fmul_rn(w[i], i < 16 ? s0 : s1);
        ab = fmaxf(ab, fabsf(w[i]));
    }
    if (ab == 0.0f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mx[j] = nv[j] & 0x88888888u;  // sign bits only
        return 0;
    }
    const int X = floor_log2(ab) - 2;
    const float inv = u2f((uint32_t)(127 - X) << 23);  // 2^-X
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t o = 0;
        const float* u = w + 8 * j;
        o = e2m1_pair<0>(o, __fmul_rn(u[0], inv), __fmul_rn(u[1], inv));
        o = e2m1_pair<1>(o, __fmul_rn(u[2], inv), __fmul_rn(u[3], inv));
        o = e2m1_pair<2>(o, __fmul_rn(u[4], inv), __fmul_rn(u[5], inv));
        o = e2m1_pair<3>(o, __fmul_rn(u[6], inv), __fmul_rn(u[7], inv));
        mx[j] = o;
    }
    return (uint32_t)(X + 127);
}

// MXFP8 quantization of one 32-element block (OCP MX v1.0 scale rule):
// X = floor(log2(amax)) - 8 clamped to [-127, 127] (-127 for an all-zero
// block), elements E4M3(v * 2^-X). Returns the E8M0 code.
// MXFP8 block exponent X from the block's max |v| (E8M0 code X + 127), and the
// exact factor 2^-X that scales an element before its E4M3 rounding.
__device__ __forceinline__ int mxfp8_exponent(float ab) {
    const int X = ab == 0.0f ? -127 : floor_log2(ab) - 8;
    return X < -127 ? -127 : (X > 127 ? 127 : X);
}
__device__ __forceinline__ float mxfp8_inv_scale(int X) {
    return u2f((uint32_t)(127 - X) << 23);  // 2^-X, X <= 119 for finite input
}

__device__ __forceinline__ uint32_t mxfp8_block(const float* v, uint8_t* codes /*[32]*/) {
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ab = fmaxf(ab, fabsf(v[i]));
    const int X = mxfp8_exponent(ab);
    const float inv = mxfp8_inv_scale(X);
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        const uint32_t c = e4m3_code2(__fmul_rn(v[i], inv), __fmul_rn(v[i + 1], inv));
        codes[i] = (uint8_t)c;
        codes[i + 1] = (uint8_t)(c >> 8);
    }
    return (uint32_t)(X + 127);
}

}  // namespace moe
