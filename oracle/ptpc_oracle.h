/*
 * CPU oracle for the PTPC-FP8 hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct definitions of what the GPU library
 * computes.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this; the product library never does, and the two
 * share no source, header, table or helper.
 *
 * Source of the method: vLLM blog, "PTPC-FP8: Boosting vLLM Performance on
 * AMD ROCm" (2025-02-24) -- hereafter [PTPC].  The FP8 format is the OCP
 * 8-bit floating point E4M3 encoding (OCP "OFP8 Formats for Deep Learning",
 * v1.0, E4M3 table), which [PTPC] does not spell out.
 *
 * Element types crossing this interface:
 *   bf16 values   : uint16_t bit patterns
 *   E4M3 codes    : uint8_t bit patterns
 *   scales        : float (fp32)
 *   exact sums    : double (exact, see orc_gemm_exact) or int64_t
 */
#ifndef PTPC_ORACLE_H
#define PTPC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* --- E4M3 codec ------------------------------------------------------- */
double  orc_e4m3_decode(uint8_t code);
uint8_t orc_e4m3_encode(float f);
void    orc_e4m3_encode_array(const float* f, int64_t n, uint8_t* out);

/* --- bf16 helpers ----------------------------------------------------- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_bf16_from_double(double v);
void     orc_bf16_from_double_array(const double* v, int64_t n, uint16_t* out);

/* --- quantizers ------------------------------------------------------- */
void orc_quant_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                   uint8_t* qx, int64_t ldq, float* dx);
void orc_quant_weight(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                      uint8_t* qw, int64_t ldqw, float* dw);
void orc_quant_tensor(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                      uint8_t* q, int64_t ldq, float* d);
/* Static per-tensor: codes for a given scalar scale s (> 0). */
void orc_quant_static(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float s,
                      uint8_t* q, int64_t ldq);

/* --- exact FP8 contraction ------------------------------------------- */
void orc_gemm_exact(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                    int64_t ldqw, int64_t T, int64_t Ci, int64_t Co,
                    double* acc);
void orc_gemm_exact_i64(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                        int64_t ldqw, int64_t T, int64_t Ci, int64_t Co,
                        int64_t* acc);
void orc_gemm_exact_sampled(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                            int64_t ldqw, int64_t Ci, const int64_t* rows,
                            const int64_t* cols, int64_t n, double* acc);

/* --- scale application ------------------------------------------------ */
void orc_apply_scales(const double* acc, int64_t T, int64_t Co,
                      const float* dx, const float* dw, double* ref);
void orc_apply_scales_sampled(const double* acc, const int64_t* rows,
                              const int64_t* cols, int64_t n, const float* dx,
                              const float* dw, double* ref);
void orc_gemm_dequant_first(const uint8_t* qx, int64_t ldq, const float* dx,
                            const uint8_t* qw, int64_t ldqw, const float* dw,
                            int64_t T, int64_t Ci, int64_t Co, double* out);

int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
