/*
 * Reference CPU oracle for the block-scaled MoE layer forward: declarations.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.c). Not part of the product ABI.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#define ORC_FMT_NVFP4 0
#define ORC_FMT_MXFP8 1
#define ORC_FMT_MXFP4 2 /* NVFP4 weights re-blocked to MXFP4, with the NVFP4 global scale */
#define ORC_ACT_SWIGLU 0
#define ORC_ACT_RELU2 1

double orc_e2m1_decode(int code);
int orc_e2m1_encode(double u);
double orc_e4m3_decode(int code);
int orc_e4m3_encode(double u);
double orc_e8m0_decode(int code);
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);

void orc_route(int T, int E, int K, const float* logits, int32_t* ids, double* p);
void orc_permute(int T, int K, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* row_to_route, int32_t* route_to_row);

float orc_absmax(const float* v, size_t n);
float orc_nvfp4_global_scale(float amax);
void orc_nvfp4_quantize(int n, const float* v, float g, uint8_t* codes, uint8_t* sf);
float orc_nvfp4_global_scale_4o6(float amax);
void orc_nvfp4_quantize_4o6(int n, const float* v, float g, uint8_t* codes, uint8_t* sf);
void orc_nvfp4_dequant(int n, const uint8_t* codes, const uint8_t* sf, float g, double* out);
void orc_mxfp4_reblock(int n, const uint8_t* codes, const uint8_t* sf, uint8_t* mx_codes,
                       uint8_t* mx_scales);
void orc_mxfp4_dequant(int n, const uint8_t* codes, const uint8_t* sc, double* out);
void orc_mxfp8_quantize(int n, const float* v, uint8_t* codes, uint8_t* sc);
void orc_mxfp8_dequant(int n, const uint8_t* codes, const uint8_t* sc, double* out);

void orc_quantize_weight(int fmt, int N, int K, const float* w, uint8_t* codes, uint8_t* scales,
                         float* g);
void orc_expert_matvec(int fmt, int N, int K, const uint8_t* codes, const uint8_t* scales, float g,
                       const double* a, double* out);
void orc_expert_matvec_rows(int fmt, int K, const uint8_t* codes, const uint8_t* scales, float g,
                            const double* a, int nrows, const int32_t* rows, double* out);
void orc_activation(int act, int I, const double* h, int on_input, double p, int pre_act_variant,
                    double* a);
void orc_finalize(int T, int K, int H, const double* o, const int32_t* route_to_row,
                  const double* w, double* y);

#endif
