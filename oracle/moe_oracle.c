/*
 * Reference CPU oracle for the block-scaled MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include, link or
 * call this file; only the tests, the smoke entry and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or constant generator
 * with the HIP path.
 *
 * Plain, slow, single-threaded C. Floating point is fp64 except where the method
 * fixes fp32 (the quantizer's scale arithmetic, which both sides must perform in
 * the same IEEE single-precision order). Build with -O2 -ffp-contract=off and no
 * fast-math so that every float expression below is one correctly rounded IEEE
 * operation.
 *
 * Sources for what is computed:
 *  - MegaMoE post (flashinfer.ai, "The problem" / "Our approach"): an MoE layer
 *    routes each token to a top-K subset of experts, quantizes activations, runs
 *    two grouped GEMMs and combines the results; NVFP4 uses block-16 scaling and
 *    MXFP8 block-32 scaling.
 *  - FlashInfer PR #4366 ("Description" / "Motivation"): for route r with
 *    a_r = activation(W1_r x), output-side placement computes sum_r p_r W2_r(a_r)
 *    and input-side placement computes sum_r W2_r(p_r a_r); the input-side scale
 *    is applied in FP32 after the activation and before the FC2-input
 *    quantization (W4A4) or BF16 store (W4A16), never to the FC1 pre-activation,
 *    and the finalize then uses neutral weights.
 *  - Newruntime summary of FlashInfer PR #5319 ("Retrieval answer"): W4A4 NVFP4
 *    with per-tensor or per-token activation scaling, W4A16 with BF16
 *    activations, fused and unfused (separate) finalize.
 *  - Element formats: OCP Microscaling Formats (MX) specification v1.0 (E2M1,
 *    E4M3 "FN", E8M0 and the MX block-scale rule). NVFP4 convention: E2M1
 *    values, an E4M3 scale per 16 elements and an FP32 global scale chosen as
 *    amax / (6 * 448), so that the largest block scale lands on E4M3's maximum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

/* ------------------------------------------------------------------------- */
/* Element codecs (OCP MX v1.0 element formats)                               */
/* ------------------------------------------------------------------------- */

/* E2M1 magnitudes for codes 0..7: exponent bias 1, one mantissa bit, code 1 is
 * the subnormal 0.5. Codes 8..15 are the negatives (code 8 is -0). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(int code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* Round to the nearest E2M1 magnitude, ties to the even code (mantissa bit 0),
 * saturating at 6. The sign bit always follows the sign of u, so -0 and small
 * negatives that round to zero give code 8. */
int orc_e2m1_encode(double u) {
    int sign = signbit(u) ? 8 : 0;
    double a = fabs(u);
    if (a >= 6.0) return sign | 7;
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - E2M1_MAG[c]);
        /* grid points are visited in increasing order, so a tie is always
           between best == c-1 and c: keep the even one */
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return sign | best;
}

/* E4M3 "FN": bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN,
 * exponent field 0 is subnormal (m/8 * 2^-6). Largest finite is 448. */
double orc_e4m3_decode(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to the nearest finite E4M3 value, ties to even code, saturating to
 * +-448. Magnitude codes 0..126 are strictly increasing in value, so the code
 * just below |u| is found by bisection and compared with its successor. */
int orc_e4m3_encode(double u) {
    int sign = signbit(u) ? 0x80 : 0;
    double a = fabs(u);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_decode(mid) <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    double below = a - orc_e4m3_decode(c);
    double above = orc_e4m3_decode(c + 1) - a;
    if (above < below || (above == below && ((c + 1) & 1) == 0)) c = c + 1;
    return sign | c;
}

/* E8M0: an unsigned power-of-two exponent with bias 127; 255 is NaN. */
double orc_e8m0_decode(int code) {
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite fp32 value to the nearest bf16 (8 significant bits, fp32's
 * exponent range), ties to even. The two bf16 neighbours of f are its
 * truncation toward zero and the next bf16 away from zero; the nearer one is
 * picked by comparing the exact differences in fp64. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x00010000u;
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double dl = fabs((double)f - (double)flo);
    double dh = fabs((double)fhi - (double)f);
    uint32_t pick;
    if (dl < dh) pick = lo;
    else if (dh < dl) pick = hi;
    else pick = ((lo >> 16) & 1) ? hi : lo;
    return (uint16_t)(pick >> 16);
}

/* ------------------------------------------------------------------------- */
/* S1: top-K routing with softmax renormalised over the chosen experts         */
/* (MegaMoE post, "The problem": tokens are routed to a top-K subset).         */
/* ------------------------------------------------------------------------- */

/* For each token the K largest logits in descending order, ties to the lower
 * expert index; p_k = exp(l_k - l_max) / sum_j exp(l_j - l_max) over the K
 * chosen. This equals a softmax over all E followed by renormalising the K
 * chosen probabilities. */
void orc_route(int T, int E, int K, const float* logits, int32_t* ids, double* p) {
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    double* ex = (double*)malloc((size_t)K * sizeof(double));
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: lower id wins ties */
            }
            ids[(size_t)t * K + k] = best;
            taken[best] = 1;
        }
        double m = (double)l[ids[(size_t)t * K]];
        double s = 0.0;
        for (int k = 0; k < K; ++k) {
            ex[k] = exp((double)l[ids[(size_t)t * K + k]] - m);
            s += ex[k];
        }
        for (int k = 0; k < K; ++k) p[(size_t)t * K + k] = ex[k] / s;
    }
    free(taken);
    free(ex);
}

/* ------------------------------------------------------------------------- */
/* S2: expert-contiguous permutation ("contiguous" grouped GEMM inputs and the  */
/* unpermutation of PR #4366's finalize).                                     */
/* ------------------------------------------------------------------------- */

/* Routes are numbered r = t*K + k. Rows of expert e occupy
 * [offsets[e], offsets[e+1]) in ascending route order (so ascending token). */
void orc_permute(int T, int K, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* row_to_route, int32_t* route_to_row) {
    int R = T * K;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int r = 0; r < R; ++r) counts[ids[r]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int r = 0; r < R; ++r) {
        int row = fill[ids[r]]++;
        row_to_route[row] = r;
        route_to_row[r] = row;
    }
    free(fill);
}

/* ------------------------------------------------------------------------- */
/* NVFP4 quantization (block 16, E4M3 block scale, FP32 global scale)         */
/* ------------------------------------------------------------------------- */

float orc_absmax(const float* v, size_t n) {
    float a = 0.0f;
    for (size_t i = 0; i < n; ++i) {
        float x = fabsf(v[i]);
        if (x > a) a = x;
    }
    return a;
}

/* Global decode scale: the tensor (or row) amax maps to 6 * 448 = 2688, the
 * largest representable E2M1 value times the largest E4M3 scale. */
float orc_nvfp4_global_scale(float amax) { return amax / 2688.0f; }

/* Quantize n values (n % 16 == 0) with global scale g. Binding fp32 order:
 *   s  = a_b / (6 * g)       block scale before encoding, a_b = block amax
 *   sf = E4M3(s)             RNE, saturating
 *   d  = float(sf) * g       per-element decode scale
 *   q  = E2M1(v / d)         RNE, saturating, sign kept
 * If g == 0 (all-zero input) or d == 0 the magnitude is zero and only the sign
 * bit is kept. Codes are written one per byte here (unpacked). */
void orc_nvfp4_quantize(int n, const float* v, float g, uint8_t* codes, uint8_t* sf) {
    for (int b = 0; b < n / 16; ++b) {
        const float* vb = v + (size_t)b * 16;
        uint8_t* cb = codes + (size_t)b * 16;
        if (g == 0.0f) {
            sf[b] = 0;
            for (int i = 0; i < 16; ++i) cb[i] = signbit(vb[i]) ? 8 : 0;
            continue;
        }
        float ab = orc_absmax(vb, 16);
        float six_g = 6.0f * g;
        float s = ab / six_g;
        int sfc = orc_e4m3_encode((double)s);
        sf[b] = (uint8_t)sfc;
        float d = (float)orc_e4m3_decode(sfc) * g;
        for (int i = 0; i < 16; ++i) {
            if (d == 0.0f) {
                cb[i] = signbit(vb[i]) ? 8 : 0;
            } else {
                float u = vb[i] / d;
                cb[i] = (uint8_t)orc_e2m1_encode((double)u);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* NVFP4 "4-over-6" block choice for per-token activations (FlashInfer PR     */
/* #4366, "Performance benchmark": the 4-over-6 per-token activation contract, */
/* named there by its environment switches only). Reading, step by step:      */
/*  - global scale g = amax / (6 * 256): the block scales of the usual         */
/*    max-to-6 mapping stay at or below 256, so the max-to-4 mapping (1.5x     */
/*    larger scales, up to 384) still fits E4M3's 448;                         */
/*  - per 16-block, two candidates: the usual one (block max mapped to the     */
/*    E2M1 maximum 6: s = a_b / (6 g)) and the max-to-4 one (s = a_b / (4 g)), */
/*    each with the same fp32 operation order as orc_nvfp4_quantize;          */
/*  - the candidate with the smaller sum of squared errors                    */
/*    sum_i (v_i - code_i * d)^2 over the block is kept, ties going to the     */
/*    usual one. The error is accumulated in fp64 in element order, each       */
/*    operation rounded once, so the decision is reproducible.                 */
/* ------------------------------------------------------------------------- */

float orc_nvfp4_global_scale_4o6(float amax) { return amax / 1536.0f; }

/* One 16-block with global scale g and the block max mapped to `top` (6 or
 * 4): writes the codes, returns the E4M3 scale code and the block's sum of
 * squared errors (fp64, element order). */
static int nvfp4_block_candidate(const float* vb, float g, float top, uint8_t* cb, double* err) {
    float ab = orc_absmax(vb, 16);
    float top_g = top * g;
    float s = ab / top_g;
    int sfc = orc_e4m3_encode((double)s);
    float d = (float)orc_e4m3_decode(sfc) * g;
    double e = 0.0;
    for (int i = 0; i < 16; ++i) {
        if (d == 0.0f) {
            cb[i] = signbit(vb[i]) ? 8 : 0;
        } else {
            float u = vb[i] / d;
            cb[i] = (uint8_t)orc_e2m1_encode((double)u);
        }
        double diff = (double)vb[i] - orc_e2m1_decode(cb[i]) * (double)d;
        e = e + diff * diff;
    }
    *err = e;
    return sfc;
}

void orc_nvfp4_quantize_4o6(int n, const float* v, float g, uint8_t* codes, uint8_t* sf) {
    for (int b = 0; b < n / 16; ++b) {
        const float* vb = v + (size_t)b * 16;
        uint8_t* cb = codes + (size_t)b * 16;
        if (g == 0.0f) {
            sf[b] = 0;
            for (int i = 0; i < 16; ++i) cb[i] = signbit(vb[i]) ? 8 : 0;
            continue;
        }
        uint8_t c6[16], c4[16];
        double e6, e4;
        int s6 = nvfp4_block_candidate(vb, g, 6.0f, c6, &e6);
        int s4 = nvfp4_block_candidate(vb, g, 4.0f, c4, &e4);
        int four = e4 < e6;
        sf[b] = (uint8_t)(four ? s4 : s6);
        memcpy(cb, four ? c4 : c6, 16);
    }
}

/* Dequantized value code * sf * g, exact in fp64 (at most 2 + 4 + 24 bits). */
void orc_nvfp4_dequant(int n, const uint8_t* codes, const uint8_t* sf, float g, double* out) {
    for (int i = 0; i < n; ++i)
        out[i] = orc_e2m1_decode(codes[i]) * orc_e4m3_decode(sf[i / 16]) * (double)g;
}

/* ------------------------------------------------------------------------- */
/* MXFP8 quantization (OCP MX v1.0: block 32, E8M0 shared scale, E4M3 elements) */
/* ------------------------------------------------------------------------- */

/* Shared exponent X = floor(log2(block amax)) - 8 (8 = exponent of E4M3's
 * largest normal), clamped to E8M0's [-127, 127]; elements are E4M3(v / 2^X),
 * RNE and saturating. An all-zero block gets X = -127 (code 0). */
void orc_mxfp8_quantize(int n, const float* v, uint8_t* codes, uint8_t* sc) {
    for (int b = 0; b < n / 32; ++b) {
        const float* vb = v + (size_t)b * 32;
        float ab = orc_absmax(vb, 32);
        int X;
        if (ab == 0.0f) {
            X = -127;
        } else {
            int ex;
            frexp((double)ab, &ex); /* ab = f * 2^ex, f in [0.5, 1) */
            X = (ex - 1) - 8;
            if (X < -127) X = -127;
            if (X > 127) X = 127;
        }
        sc[b] = (uint8_t)(X + 127);
        for (int i = 0; i < 32; ++i)
            codes[(size_t)b * 32 + i] = (uint8_t)orc_e4m3_encode(ldexp((double)vb[i], -X));
    }
}

void orc_mxfp8_dequant(int n, const uint8_t* codes, const uint8_t* sc, double* out) {
    for (int i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(codes[i]) * orc_e8m0_decode(sc[i / 32]);
}

/* ------------------------------------------------------------------------- */
/* Re-blocking NVFP4 to MXFP4 (the other NVFP4 GEMM option: block-scaled FP4   */
/* matrix units take E8M0 scales per 32 elements, NVFP4 has E4M3 per 16).      */
/* The block-local NVFP4 value w = E2M1(code) * E4M3(sf) (at most 6            */
/* significant bits, exact in fp64) of each 32-element block is re-quantized   */
/* by the OCP MX v1.0 rule for E2M1 elements: shared exponent                 */
/* X = floor(log2(block max)) - 2 (2 = exponent of E2M1's largest normal),     */
/* clamped to [-127, 127], elements E2M1_RNE(w / 2^X) (exact quotient,         */
/* saturating at 6, sign kept). An all-zero block gets X = -127 (code 0) and   */
/* sign-only codes. The FP32 global scale is not part of the block and stays   */
/* as it is. MXFP4 value: E2M1(code) * 2^X (* g).                              */
/* ------------------------------------------------------------------------- */
void orc_mxfp4_reblock(int n, const uint8_t* codes, const uint8_t* sf, uint8_t* mx_codes,
                       uint8_t* mx_scales) {
    for (int b = 0; b < n / 32; ++b) {
        double w[32];
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            int k = b * 32 + i;
            w[i] = orc_e2m1_decode(codes[k]) * orc_e4m3_decode(sf[k / 16]);
            if (fabs(w[i]) > amax) amax = fabs(w[i]);
        }
        int X;
        if (amax == 0.0) {
            X = -127;
        } else {
            int ex;
            frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
            X = (ex - 1) - 2;
            if (X < -127) X = -127;
            if (X > 127) X = 127;
        }
        mx_scales[b] = (uint8_t)(X + 127);
        for (int i = 0; i < 32; ++i) {
            if (amax == 0.0) {
                mx_codes[b * 32 + i] = (uint8_t)(codes[b * 32 + i] & 8);
            } else {
                /* w carries the NVFP4 code's sign, also for zeros (-0 -> 8) */
                mx_codes[b * 32 + i] = (uint8_t)orc_e2m1_encode(ldexp(w[i], -X));
            }
        }
    }
}

void orc_mxfp4_dequant(int n, const uint8_t* codes, const uint8_t* sc, double* out) {
    for (int i = 0; i < n; ++i)
        out[i] = orc_e2m1_decode(codes[i]) * orc_e8m0_decode(sc[i / 32]);
}

/* ------------------------------------------------------------------------- */
/* Weights: one NVFP4 global scale per expert per matrix                       */
/* ------------------------------------------------------------------------- */

/* w is one expert's [N][K] fp32 matrix (K contiguous, the checkpoint layout).
 * NVFP4: g = amax(w) / 2688, every row quantized along K with that g.
 * MXFP8: every row quantized along K in blocks of 32. */
void orc_quantize_weight(int fmt, int N, int K, const float* w, uint8_t* codes, uint8_t* scales,
                         float* g) {
    if (fmt == ORC_FMT_NVFP4) {
        float gg = orc_nvfp4_global_scale(orc_absmax(w, (size_t)N * K));
        *g = gg;
        for (int n = 0; n < N; ++n)
            orc_nvfp4_quantize(K, w + (size_t)n * K, gg, codes + (size_t)n * K,
                               scales + (size_t)n * (K / 16));
    } else {
        *g = 1.0f;
        for (int n = 0; n < N; ++n)
            orc_mxfp8_quantize(K, w + (size_t)n * K, codes + (size_t)n * K,
                               scales + (size_t)n * (K / 32));
    }
}

/* Dequantized weight element (n, k) of a quantized [N][K] matrix. */
static double weight_value(int fmt, int K, const uint8_t* codes, const uint8_t* scales, float g,
                           int n, int k) {
    uint8_t c = codes[(size_t)n * K + k];
    if (fmt == ORC_FMT_NVFP4)
        return orc_e2m1_decode(c) * orc_e4m3_decode(scales[(size_t)n * (K / 16) + k / 16]) *
               (double)g;
    if (fmt == ORC_FMT_MXFP4)
        return orc_e2m1_decode(c) * orc_e8m0_decode(scales[(size_t)n * (K / 32) + k / 32]) *
               (double)g;
    return orc_e4m3_decode(c) * orc_e8m0_decode(scales[(size_t)n * (K / 32) + k / 32]);
}

/* out[n] = sum_k a[k] * W[n][k], accumulated in fp64 in ascending k. */
void orc_expert_matvec(int fmt, int N, int K, const uint8_t* codes, const uint8_t* scales, float g,
                       const double* a, double* out) {
    for (int n = 0; n < N; ++n) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += a[k] * weight_value(fmt, K, codes, scales, g, n, k);
        out[n] = s;
    }
}

/* Same product for a subset of output rows (used to sample FC2 outputs). */
void orc_expert_matvec_rows(int fmt, int K, const uint8_t* codes, const uint8_t* scales, float g,
                            const double* a, int nrows, const int32_t* rows, double* out) {
    for (int i = 0; i < nrows; ++i) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += a[k] * weight_value(fmt, K, codes, scales, g, rows[i], k);
        out[i] = s;
    }
}

/* ------------------------------------------------------------------------- */
/* Activation and router-weight placement                                    */
/* ------------------------------------------------------------------------- */

/* h has N1 entries. SwiGLU: rows [0, I) are the gate, [I, 2I) the up
 * projection; a = silu(gate) * up with silu(z) = z / (1 + exp(-z)).
 * ReLU2: a = max(h, 0)^2, N1 == I.
 * Input-side placement multiplies the activation output by p (PR #4366: after
 * the activation, before the FC2-input store). pre_act_variant != 0 is a
 * deliberately wrong variant kept only for a negative test: it scales the FC1
 * output before the activation, which for ReLU2 gives p^2 * relu(z)^2 (the
 * problem PR #4366 "Existing SM120 status" describes). */
void orc_activation(int act, int I, const double* h, int on_input, double p, int pre_act_variant,
                    double* a) {
    for (int n = 0; n < I; ++n) {
        double v;
        if (act == ORC_ACT_SWIGLU) {
            double gt = h[n], up = h[I + n];
            if (on_input && pre_act_variant) { gt *= p; up *= p; }
            v = gt / (1.0 + exp(-gt)) * up;
        } else {
            double z = h[n];
            if (on_input && pre_act_variant) z *= p;
            v = z > 0.0 ? z * z : 0.0;
        }
        if (on_input && !pre_act_variant) v *= p;
        a[n] = v;
    }
}

/* ------------------------------------------------------------------------- */
/* S7: finalize (unpermute + top-K weighted reduction in fixed k order)       */
/* ------------------------------------------------------------------------- */

/* y[t][j] = sum_{k=0}^{K-1} w[t][k] * o[route_to_row[t*K+k]][j], sequential
 * in k, fp64. w == NULL means unit weights (input-side placement). */
void orc_finalize(int T, int K, int H, const double* o, const int32_t* route_to_row,
                  const double* w, double* y) {
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j) {
            double s = 0.0;
            for (int k = 0; k < K; ++k) {
                double wk = w ? w[(size_t)t * K + k] : 1.0;
                s += wk * o[(size_t)route_to_row[(size_t)t * K + k] * H + j];
            }
            y[(size_t)t * H + j] = s;
        }
    }
}
