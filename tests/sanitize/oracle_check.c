/* The CPU oracle under AddressSanitizer / UBSan: every function on small
 * inputs of odd shapes (pitches wider than the extents, rows and columns
 * that are not multiples of anything), with the consistency checks that
 * need no reference: double == int64 sums, sampled == full, each row's and
 * column's amax element encodes to +-448.  Any sanitizer report aborts. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ptpc_oracle.h"

static int fails = 0;
#define REQUIRE(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {            /* xorshift64* */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return state * 0x2545F4914F6CDD1Dull;
}

/* a bf16 pattern of a finite value, never NaN/Inf */
static uint16_t rand_bf16(void) {
    uint16_t b = (uint16_t)next();
    if (((b >> 7) & 0xFF) == 0xFF) b &= 0xBFFF;
    return b;
}

int main(void) {
    const int64_t T = 7, Ci = 48, Co = 33, ldx = 53, ldw = 37;
    uint16_t* x = malloc(sizeof(uint16_t) * T * ldx);
    uint16_t* w = malloc(sizeof(uint16_t) * Ci * ldw);
    uint8_t* qx = malloc((size_t)T * Ci);
    uint8_t* qw = malloc((size_t)Ci * Co);
    uint8_t* qt = malloc((size_t)T * Ci);
    float* dx = malloc(sizeof(float) * T);
    float* dw = malloc(sizeof(float) * Co);
    double* acc = malloc(sizeof(double) * T * Co);
    int64_t* acc_i = malloc(sizeof(int64_t) * T * Co);
    double* ref = malloc(sizeof(double) * T * Co);
    double* dq = malloc(sizeof(double) * T * Co);
    int64_t rows[20], cols[20];
    double accs[20], refs[20];
    float dt;
    int64_t i, j;
    for (i = 0; i < T * ldx; ++i) x[i] = rand_bf16();
    for (i = 0; i < Ci * ldw; ++i) w[i] = rand_bf16();
    for (j = 0; j < Ci; ++j) x[3 * ldx + j] = 0;                 /* a zero row */

    orc_quant_act(x, T, Ci, ldx, qx, Ci, dx);
    orc_quant_weight(w, Ci, Co, ldw, qw, Co, dw);
    orc_quant_tensor(x, T, Ci, ldx, qt, Ci, &dt);
    orc_quant_static(x, T, Ci, ldx, dt, qt, Ci);
    REQUIRE(dx[3] == 1.0f);
    for (i = 0; i < T; ++i) {
        int hit = (i == 3);
        for (j = 0; j < Ci; ++j) hit |= (qx[i * Ci + j] & 0x7F) == 0x7E;
        REQUIRE(hit);
    }
    orc_gemm_exact(qx, Ci, qw, Co, T, Ci, Co, acc);
    orc_gemm_exact_i64(qx, Ci, qw, Co, T, Ci, Co, acc_i);
    for (i = 0; i < T * Co; ++i) REQUIRE(acc[i] == ldexp((double)acc_i[i], -18));
    for (i = 0; i < 20; ++i) { rows[i] = (int64_t)(next() % T); cols[i] = (int64_t)(next() % Co); }
    orc_gemm_exact_sampled(qx, Ci, qw, Co, Ci, rows, cols, 20, accs);
    orc_apply_scales(acc, T, Co, dx, dw, ref);
    orc_apply_scales_sampled(accs, rows, cols, 20, dx, dw, refs);
    for (i = 0; i < 20; ++i) {
        REQUIRE(accs[i] == acc[rows[i] * Co + cols[i]]);
        REQUIRE(refs[i] == ref[rows[i] * Co + cols[i]]);
    }
    orc_gemm_dequant_first(qx, Ci, dx, qw, Co, dw, T, Ci, Co, dq);
    for (i = 0; i < 256; ++i) {
        double v = orc_e4m3_decode((uint8_t)i);
        if (!isnan(v)) REQUIRE(orc_e4m3_encode((float)v) == (uint8_t)i || v == 0.0);
    }
    free(x); free(w); free(qx); free(qw); free(qt); free(dx); free(dw);
    free(acc); free(acc_i); free(ref); free(dq);
    printf("oracle_check: %d failures\n", fails);
    return fails == 0 ? 0 : 1;
}
