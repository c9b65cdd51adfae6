/*
 * CPU oracle for the PTPC-FP8 hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the checker, not the product: only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark load it.  It shares no code with
 * the GPU library.  Everything is written for a reader holding the source
 * page, [PTPC] = vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm"
 * (2025-02-24), and is deliberately plain: scalar loops, double precision
 * where the value is a reference, the library's fp32 only where the method
 * itself produces an fp32 number (the scales and the quotient that is cast).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math: every fp32
 * division below must be the IEEE correctly rounded one).  OpenMP only
 * spreads independent rows / columns / outputs over threads; no result
 * depends on the thread count (each output is produced by one thread, and
 * the exact sums below do not depend on summation order anyway).
 */
#include "ptpc_oracle.h"

#include <math.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------
 * E4M3 codec (OCP OFP8 v1.0, E4M3 encoding).  [PTPC] says only "FP8"
 * (§What is PTPC-FP8); the reading taken is OCP E4M3FN: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, no infinities, the all-ones
 * pattern S.1111.111 is NaN, largest finite magnitude 448.
 * ------------------------------------------------------------------- */

/* Value of an E4M3 bit pattern, straight from the format definition. */
double orc_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* subnormal: m * 2^-9   */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);       /* (1 + m/8) * 2^(e-7)   */
    return s ? -v : v;
}

/* Round-half-to-even of a non-negative double to an integer value. */
static double rne_int(double m) {
    double f = floor(m);
    double frac = m - f;                       /* exact: m < 2^52 here  */
    if (frac > 0.5) return f + 1.0;
    if (frac < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/*
 * Nearest E4M3 value to f, ties to the even mantissa, saturating at +-448,
 * sign kept (so -0 and negative values that round to zero give 0x80).
 * [PTPC] does not state the rounding or the overflow rule; round-to-nearest-
 * even with saturation is the reading taken.  NaN is outside the contract and
 * maps to 0x7F.
 */
uint8_t orc_e4m3_encode(float f) {
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a, m, r;
    int e2, E;
    if (isnan(f)) return 0x7F;
    a = fabs((double)f);
    if (a >= 448.0) return sign | 0x7E;                 /* saturate      */
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: representable values are r * 2^-9, r=0..8
           (r = 8 is the smallest normal 2^-6, whose code is also 8)   */
        r = rne_int(a * 512.0);                            /* exact scale */
        return sign | (uint8_t)r;
    }
    frexp(a, &e2);                  /* a in [2^(e2-1), 2^e2)              */
    E = e2 - 1;                     /* unbiased exponent, -6 .. 8        */
    m = ldexp(a, 3 - E);            /* in [8, 16), exact                 */
    r = rne_int(m);                 /* 8 .. 16                           */
    if (r == 16.0) { r = 8.0; E += 1; }
    /* a < 448 keeps the result at or below 448 = 1.75 * 2^8 */
    return sign | (uint8_t)(((E + 7) << 3) | ((int)r - 8));
}

void orc_e4m3_encode_array(const float* f, int64_t n, uint8_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode(f[i]);
}

/* ---------------------------------------------------------------------
 * bf16 helpers.  The inputs X and W are bf16 ([PTPC] §Benchmark 2.1 uses a
 * BF16 baseline model); bf16 is the top half of an fp32 word.
 * ------------------------------------------------------------------- */
float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bf16 (8 significant bits, fp32 exponent range), ties to even. */
uint16_t orc_bf16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), m, r;
    int e2, E, biased;
    if (isnan(v)) return 0x7FC0;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -126)) {                 /* subnormal: r * 2^-133 */
        r = rne_int(ldexp(a, 133));
        return sign | (uint16_t)r;              /* r = 128 -> min normal */
    }
    frexp(a, &e2);
    E = e2 - 1;
    m = ldexp(a, 7 - E);                        /* [128, 256) */
    r = rne_int(m);
    if (r == 256.0) { r = 128.0; E += 1; }
    biased = E + 127;
    if (biased >= 255) return sign | 0x7F80;    /* overflow -> inf */
    return sign | (uint16_t)((biased << 7) | ((int)r - 128));
}

void orc_bf16_from_double_array(const double* v, int64_t n, uint16_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_bf16_from_double(v[i]);
}

/* ---------------------------------------------------------------------
 * Quantizers.  [PTPC] §PTPC: a precision-targeted scheme -- every token
 * (row of X) gets its own scale, every weight column its own; §Understanding
 * the figure / Scaling factors -- Delta_X is [T x 1], Delta_W is [1 x Co].
 *
 * Readings taken where the page is silent:
 *   scale     Delta = amax / 448 computed in fp32 (a dequantization
 *             multiplier: the page's scales multiply the GEMM output);
 *             an all-zero vector gets Delta = 1.
 *   cast      code = E4M3(fp32(x) / Delta): one IEEE fp32 division, then
 *             the encoder above.
 * ------------------------------------------------------------------- */
static float scale_from_amax(float amax) {
    return (amax == 0.0f) ? 1.0f : amax / 448.0f;
}

/* Per-token activation quantization, X is [T x Ci] row-major (pitch ldx). */
void orc_quant_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                   uint8_t* qx, int64_t ldq, float* dx) {
    int64_t t;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        const uint16_t* row = x + t * ldx;
        float amax = 0.0f, d;
        int64_t k;
        for (k = 0; k < Ci; ++k) {
            float v = fabsf(orc_bf16_to_f32(row[k]));
            if (v > amax) amax = v;
        }
        d = scale_from_amax(amax);
        dx[t] = d;
        for (k = 0; k < Ci; ++k)
            qx[t * ldq + k] = orc_e4m3_encode(orc_bf16_to_f32(row[k]) / d);
    }
}

/* Per-output-channel weight quantization, W is [Ci x Co] row-major; the
 * codes come back in the same [Ci x Co] orientation (pitch ldqw).  The page
 * gives Delta_W the shape [1 x Co] and says each weight column gets its own
 * scale; its legend's "one per input channel" wording contradicts that shape
 * and is read as a slip -- the scale belongs to output column o.
 * Columns are handled in blocks of 64 so that a thread walks rows of W
 * contiguously; each column's result is still computed by exactly the
 * per-column definition. */
void orc_quant_weight(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                      uint8_t* qw, int64_t ldqw, float* dw) {
    int64_t ob;
#pragma omp parallel for schedule(dynamic, 1)
    for (ob = 0; ob < Co; ob += 64) {
        int64_t oe = (ob + 64 < Co) ? ob + 64 : Co, o, k;
        float amax[64], d[64];
        for (o = ob; o < oe; ++o) amax[o - ob] = 0.0f;
        for (k = 0; k < Ci; ++k)
            for (o = ob; o < oe; ++o) {
                float v = fabsf(orc_bf16_to_f32(w[k * ldw + o]));
                if (v > amax[o - ob]) amax[o - ob] = v;
            }
        for (o = ob; o < oe; ++o) {
            d[o - ob] = scale_from_amax(amax[o - ob]);
            dw[o] = d[o - ob];
        }
        for (k = 0; k < Ci; ++k)
            for (o = ob; o < oe; ++o)
                qw[k * ldqw + o] =
                    orc_e4m3_encode(orc_bf16_to_f32(w[k * ldw + o]) / d[o - ob]);
    }
}

/* Per-tensor FP8 ([PTPC] §Understanding the figure, top half: a single
 * scalar scale for the whole tensor). */
void orc_quant_tensor(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                      uint8_t* q, int64_t ldq, float* d) {
    float amax = 0.0f, s;
    int64_t i, j;
    for (i = 0; i < R; ++i)
        for (j = 0; j < C; ++j) {
            float v = fabsf(orc_bf16_to_f32(x[i * ldx + j]));
            if (v > amax) amax = v;
        }
    s = scale_from_amax(amax);
    *d = s;
#pragma omp parallel for schedule(static) private(j)
    for (i = 0; i < R; ++i)
        for (j = 0; j < C; ++j)
            q[i * ldq + j] = orc_e4m3_encode(orc_bf16_to_f32(x[i * ldx + j]) / s);
}

/* Static per-tensor FP8: one scale s fixed ahead of time (from calibration)
 * rather than measured on the tensor being quantized -- the "standard FP8"
 * comparator of [PTPC] (§PTPC: a precision-targeted scheme, the per-tensor
 * baseline; §Benchmark 1) with its scalar scale given.  code =
 * E4M3(fp32(x) / s), saturating at +-448 like every cast here. */
void orc_quant_static(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, float s,
                      uint8_t* q, int64_t ldq) {
    int64_t i, j;
#pragma omp parallel for schedule(static) private(j)
    for (i = 0; i < R; ++i)
        for (j = 0; j < C; ++j)
            q[i * ldq + j] = orc_e4m3_encode(orc_bf16_to_f32(x[i * ldx + j]) / s);
}

/* ---------------------------------------------------------------------
 * The FP8 x FP8 contraction ([PTPC] §The challenge: two-step vs fused,
 * step 1 of the naive code): acc[t,o] = sum_k dec(qx[t,k]) * dec(qw[k,o]).
 *
 * Exactness: every E4M3 value is an integer multiple of 2^-9, so every
 * product and every partial sum is an integer multiple of 2^-18.  Each
 * product is at most 448^2 < 2^17.62 in magnitude, so for Ci <= 2^17 every
 * partial sum is below 2^35 in magnitude, i.e. fewer than 2^53 units of
 * 2^-18: double holds every partial sum exactly and the order of summation
 * cannot change the result.  The int64 variant sums the integers dec*2^9
 * and must agree exactly.  Decoding goes through a 256-entry table filled
 * from orc_e4m3_decode (a cache of that function, nothing more).
 * ------------------------------------------------------------------- */
static double dec_tab[256];
static int64_t unit_tab[256];
static void fill_tables(void) {          /* idempotent; called serially */
    int c;
    for (c = 0; c < 256; ++c) {
        double v = orc_e4m3_decode((uint8_t)c);
        dec_tab[c] = v;
        unit_tab[c] = isnan(v) ? 0 : (int64_t)ldexp(v, 9);  /* dec * 2^9 */
    }
}

void orc_gemm_exact(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                    int64_t ldqw, int64_t T, int64_t Ci, int64_t Co,
                    double* acc) {
    int64_t t;
    fill_tables();
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        int64_t o, k;
        for (o = 0; o < Co; ++o) {
            double s = 0.0;
            for (k = 0; k < Ci; ++k)
                s += dec_tab[qx[t * ldq + k]] * dec_tab[qw[k * ldqw + o]];
            acc[t * Co + o] = s;
        }
    }
}

void orc_gemm_exact_i64(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                        int64_t ldqw, int64_t T, int64_t Ci, int64_t Co,
                        int64_t* acc) {
    int64_t t;
    fill_tables();
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        int64_t o, k;
        for (o = 0; o < Co; ++o) {
            int64_t s = 0;
            for (k = 0; k < Ci; ++k)
                s += unit_tab[qx[t * ldq + k]] * unit_tab[qw[k * ldqw + o]];
            acc[t * Co + o] = s;      /* in units of 2^-18 */
        }
    }
}

/* The same sum for an explicit list of (row, column) outputs. */
void orc_gemm_exact_sampled(const uint8_t* qx, int64_t ldq, const uint8_t* qw,
                            int64_t ldqw, int64_t Ci, const int64_t* rows,
                            const int64_t* cols, int64_t n, double* acc) {
    int64_t i;
    fill_tables();
#pragma omp parallel for schedule(dynamic, 4)
    for (i = 0; i < n; ++i) {
        int64_t t = rows[i], o = cols[i], k;
        double s = 0.0;
        for (k = 0; k < Ci; ++k)
            s += dec_tab[qx[t * ldq + k]] * dec_tab[qw[k * ldqw + o]];
        acc[i] = s;
    }
}

/* ---------------------------------------------------------------------
 * Scale application ([PTPC] §The challenge: two-step vs fused, step 2:
 * output * token_scales * channel_scales).  The reference value is the
 * exact sum times Delta_X[t] times Delta_W[o], in double.
 * ------------------------------------------------------------------- */
void orc_apply_scales(const double* acc, int64_t T, int64_t Co,
                      const float* dx, const float* dw, double* ref) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        int64_t o;
        for (o = 0; o < Co; ++o)
            ref[t * Co + o] = acc[t * Co + o] * (double)dx[t] * (double)dw[o];
    }
}

void orc_apply_scales_sampled(const double* acc, const int64_t* rows,
                              const int64_t* cols, int64_t n, const float* dx,
                              const float* dw, double* ref) {
    int64_t i;
    for (i = 0; i < n; ++i)
        ref[i] = acc[i] * (double)dx[rows[i]] * (double)dw[cols[i]];
}

/* Dequantize first, then contract: sum_k (dec(qx)*Delta_X[t]) *
 * (dec(qw)*Delta_W[o]).  Mathematically the same value as scaling after
 * the sum ([PTPC] §The solution: fusion -- the fused call returns what the
 * two-step code returns); used only to check that equality. */
void orc_gemm_dequant_first(const uint8_t* qx, int64_t ldq, const float* dx,
                            const uint8_t* qw, int64_t ldqw, const float* dw,
                            int64_t T, int64_t Ci, int64_t Co, double* out) {
    int64_t t;
    fill_tables();
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        int64_t o, k;
        for (o = 0; o < Co; ++o) {
            double s = 0.0;
            for (k = 0; k < Ci; ++k)
                s += (dec_tab[qx[t * ldq + k]] * (double)dx[t]) *
                     (dec_tab[qw[k * ldqw + o]] * (double)dw[o]);
            out[t * Co + o] = s;
        }
    }
}
