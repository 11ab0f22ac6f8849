/*
 * norm.c -- a row normalization followed by rowwise dynamic FP8 quantization,
 * the pair that quantization fused into the producer replaces ("FP8
 * Training: Quantization, Autograd, Torchao", section 8: a LayerNorm's output
 * write fused with the next layer's amax pass). Test infrastructure only (see
 * fp8_oracle.h).
 *
 * The steps, one row at a time, each a separate loop:
 *   1. s1 = sum x, s2 = sum x^2 over the row (x: bf16 widened; long double
 *      accumulation in column order), rounded to fp64;
 *   2. mean = s1 / n, ms = s2 / n; var = ms - mean^2 (LayerNorm) or ms (RMS);
 *      rstd = 1 / sqrt(var + norm_eps); all fp64 IEEE operations;
 *   3. y = ((x - mean32) * rstd32) * gamma + beta (LayerNorm) or
 *      (x * rstd32) * gamma (RMS), each operation an fp32 IEEE operation on
 *      mean32 = (float)mean and rstd32 = (float)rstd, then y rounded to bf16
 *      (nearest, ties to even) as the normalized activation is stored;
 *   4. the rowwise quantization of those bf16 values (orc_quant_row).
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* fp32 -> bf16 bits, round to nearest, ties to even (finite inputs). */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void orc_norm_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                  int64_t cols, int layer, double norm_eps, uint16_t* y) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        long double a1 = 0.0L, a2 = 0.0L;                               /* step 1 */
        for (int64_t c = 0; c < cols; ++c) {
            long double v = (long double)orc_bf16_to_f32(xr[c]);
            a1 += v;
            a2 += v * v;
        }
        double s1 = (double)a1, s2 = (double)a2;
        double n = (double)cols;                                         /* step 2 */
        double mean = s1 / n, ms = s2 / n;
        double var = layer ? ms - mean * mean : ms;
        double rstd = 1.0 / sqrt(var + norm_eps);
        float mean32 = (float)mean, rstd32 = (float)rstd;
        for (int64_t c = 0; c < cols; ++c) {                             /* step 3 */
            float v = orc_bf16_to_f32(xr[c]);
            float g = orc_bf16_to_f32(gamma[c]);
            float t;
            if (layer) {
                t = v - mean32;
                t = t * rstd32;
                t = t * g;
                t = t + (beta ? orc_bf16_to_f32(beta[c]) : 0.0f);
            } else {
                t = v * rstd32;
                t = t * g;
            }
            y[r * cols + c] = f32_to_bf16_rne(t);
        }
    }
}

void orc_norm_quant_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                        int64_t cols, int layer, double norm_eps, int fmt, double eps, uint16_t* y,
                        uint8_t* q, float* scale, float* inv) {
    orc_norm_row(x, gamma, beta, rows, cols, layer, norm_eps, y);
    orc_quant_row(y, 1, rows, cols, fmt, eps, q, scale, inv, 1);       /* step 4 */
}
