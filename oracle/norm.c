/*
 * norm.c -- a row normalization followed by rowwise dynamic FP8 quantization,
 * the pair that quantization fused into the producer replaces ("FP8
 * Training: Quantization, Autograd, Torchao", section 8: a LayerNorm's output
 * write fused with the next layer's amax pass). Test infrastructure only (see
 * fp8_oracle.h).
 *
 * The steps, one row at a time, each a separate loop:
 *   1. s1 = sum x, s2 = sum x^2 over the row (x: bf16), each the EXACT sum
 *      rounded once to fp64 (round to nearest, ties to even). The sums are
 *      kept exactly as fixed-point integers, so neither the order of the
 *      terms nor their range matters;
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

/* ---- exact sums ------------------------------------------------------------
 * A bf16 value is +-M * 2^q with an integer M < 256: q = E - 134 for a
 * biased exponent E >= 1 (M = 128 + mantissa), q = -133 for E = 0 (M =
 * mantissa). In units of 2^-133 the value is the integer M * 2^(max(E,1) - 1),
 * its square in units of 2^-266 the integer M^2 * 2^(2 (max(E,1) - 1)). Such
 * integers are added into a magnitude of base-2^32 digits, positive and
 * negative terms apart; the difference is rounded to fp64 at the end. */
#define SUM_DIGITS 24 /* 768 bits: above 2^553, the largest sum of squares of 2^31 terms */

typedef struct {
    uint32_t d[SUM_DIGITS];
} exact_sum;

/* acc += m * 2^shift, 0 <= m < 2^32. */
static void sum_add(exact_sum* acc, uint64_t m, int shift) {
    int i = shift / 32;
    uint64_t v = m << (shift % 32); /* < 2^63 */
    uint64_t carry = 0;
    for (int k = i; k < SUM_DIGITS && (v != 0 || carry != 0); ++k) {
        uint64_t t = (uint64_t)acc->d[k] + (v & 0xffffffffu) + carry;
        acc->d[k] = (uint32_t)t;
        carry = t >> 32;
        v >>= 32;
    }
}

/* a >= b as magnitudes. */
static int sum_ge(const exact_sum* a, const exact_sum* b) {
    for (int k = SUM_DIGITS - 1; k >= 0; --k)
        if (a->d[k] != b->d[k]) return a->d[k] > b->d[k];
    return 1;
}

/* r = a - b, a >= b. */
static void sum_sub(const exact_sum* a, const exact_sum* b, exact_sum* r) {
    int64_t borrow = 0;
    for (int k = 0; k < SUM_DIGITS; ++k) {
        int64_t t = (int64_t)a->d[k] - (int64_t)b->d[k] - borrow;
        borrow = t < 0;
        r->d[k] = (uint32_t)(t + (borrow ? ((int64_t)1 << 32) : 0));
    }
}

static int bit_of(const exact_sum* a, int p) { return (int)((a->d[p / 32] >> (p % 32)) & 1u); }

/* The value a * 2^unit_exp (sign: negative != 0) rounded to the nearest
 * fp64, ties to even. */
static double sum_to_double(const exact_sum* a, int negative, int unit_exp) {
    int lead = -1;
    for (int p = 32 * SUM_DIGITS - 1; p >= 0; --p)
        if (bit_of(a, p)) {
            lead = p;
            break;
        }
    if (lead < 0) return 0.0; /* an exact zero sum is +0 */
    uint64_t sig = 0;         /* the 53 bits from the leading one down */
    for (int p = lead; p > lead - 53; --p) sig = (sig << 1) | (uint64_t)(p >= 0 ? bit_of(a, p) : 0);
    const int round = lead - 53 >= 0 ? bit_of(a, lead - 53) : 0;
    int sticky = 0;
    for (int p = lead - 54; p >= 0 && !sticky; --p) sticky = bit_of(a, p);
    int e = lead - 52 + unit_exp; /* value = sig * 2^e before rounding */
    if (round && (sticky || (sig & 1u))) {
        sig += 1;
        if (sig == ((uint64_t)1 << 53)) {
            sig >>= 1;
            e += 1;
        }
    }
    const double v = ldexp((double)sig, e);
    return negative ? -v : v;
}

void orc_norm_stats(const uint16_t* x, int64_t rows, int64_t cols, double* s1, double* s2) {
    for (int64_t r = 0; r < rows; ++r) {
        exact_sum pos, neg, sq;
        memset(&pos, 0, sizeof pos);
        memset(&neg, 0, sizeof neg);
        memset(&sq, 0, sizeof sq);
        for (int64_t c = 0; c < cols; ++c) {
            const uint16_t b = x[r * cols + c];
            const int E = (b >> 7) & 0xff;
            const uint64_t M = E ? (uint64_t)(128 + (b & 0x7f)) : (uint64_t)(b & 0x7f);
            const int sh = (E ? E : 1) - 1;
            sum_add((b & 0x8000) ? &neg : &pos, M, sh);
            sum_add(&sq, M * M, 2 * sh);
        }
        exact_sum d;
        const int negative = !sum_ge(&pos, &neg);
        if (negative)
            sum_sub(&neg, &pos, &d);
        else
            sum_sub(&pos, &neg, &d);
        s1[r] = sum_to_double(&d, negative, -133);
        s2[r] = sum_to_double(&sq, 0, -266);
    }
}

void orc_norm_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                  int64_t cols, int layer, double norm_eps, uint16_t* y) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        double s1, s2;                                                   /* step 1 */
        orc_norm_stats(xr, 1, cols, &s1, &s2);
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
