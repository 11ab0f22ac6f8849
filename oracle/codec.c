/*
 * codec.c -- bit-level FP8 encode/decode, bf16 widening, and the per-group
 * scale derivation of the oracle. Test infrastructure only (see
 * fp8_oracle.h).
 *
 * Formats ("FP8 Training: Quantization, Autograd, Torchao", section 3
 * "Format choice: e4m3 vs e5m2", table; "FP8 training on AMD GPUs with
 * TorchTitan and TorchAO", section "AMD FP8 format in TorchAO", e4m3fnuz
 * table):
 *   e4m3   : 1 sign, 4 exponent, 3 mantissa bits; max 448 (OCP "fn": bias 7,
 *            NaN = S.1111.111, no infinity, has -0).
 *   e4m3fnuz: same bit split, max 240, finite, no negative zero (bias 8,
 *            the pattern 0x80 that would be -0 is the single NaN).
 *   e5m2   : 1/5/2 bits, max 57344 (IEEE-style: bias 15, exponent 31 holds
 *            inf/NaN, has -0).
 *   e5m2fnuz: 1/5/2 bits, bias 16, max 57344, finite, no negative zero.
 * The bias of each format follows from its bit split and its stated max.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stddef.h>

typedef struct {
    int ebits, mbits, bias;
    double maxval;   /* largest finite value */
    uint8_t maxcode; /* its positive code */
    int fnuz;        /* 1: no -0, 0x80 is NaN, no inf */
} fmt_info;

static const fmt_info FMT[4] = {
    /* ORC_E4M3FN   */ {4, 3, 7, 448.0, 0x7E, 0},
    /* ORC_E4M3FNUZ */ {4, 3, 8, 240.0, 0x7F, 1},
    /* ORC_E5M2     */ {5, 2, 15, 57344.0, 0x7B, 0},
    /* ORC_E5M2FNUZ */ {5, 2, 16, 57344.0, 0x7F, 1},
};

double orc_fp8_max(int fmt) { return FMT[fmt].maxval; }

float orc_bf16_to_f32(uint16_t b) {
    /* bf16 is the upper half of an fp32 word; widening is exact. */
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return v.f;
}

double orc_fp8_decode(int fmt, uint8_t c) {
    const fmt_info* f = &FMT[fmt];
    int s = c >> 7;
    int e = (c >> f->mbits) & ((1 << f->ebits) - 1);
    int m = c & ((1 << f->mbits) - 1);
    double mag;
    if (f->fnuz && c == 0x80) return NAN;
    if (fmt == ORC_E5M2 && e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (fmt == ORC_E4M3FN && e == 15 && m == 7) return NAN;
    if (e == 0) /* subnormal: fixed quantum 2^(1 - bias - mbits) */
        mag = ldexp((double)m, 1 - f->bias - f->mbits);
    else
        mag = ldexp((double)((1 << f->mbits) + m), e - f->bias - f->mbits);
    return s ? -mag : mag;
}

uint8_t orc_fp8_encode(int fmt, float y) {
    const fmt_info* f = &FMT[fmt];
    const int emin = 1 - f->bias; /* exponent of the smallest normal */
    uint8_t sign, code;
    double a, quantum, v;
    int ex, e;

    if (isnan(y)) return f->fnuz ? 0x80 : 0x7F;
    sign = signbit(y) ? 0x80 : 0x00;
    a = fabs((double)y);

    /* Saturation: anything at or beyond the largest finite value. */
    if (a >= f->maxval) return (uint8_t)(sign | f->maxcode);

    /* Round to nearest, ties to even, on the grid of the binade of a (or the
     * fixed subnormal grid below the smallest normal). a has at most 24
     * significant bits and the quantum is a power of two, so a / quantum is
     * exact and only the rounding to an integer is inexact. */
    if (a == 0.0) {
        e = emin;
    } else {
        frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
        e = ex - 1;
        if (e < emin) e = emin;
    }
    quantum = ldexp(1.0, e - f->mbits);
    v = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
    /* v <= maxval: maxval is itself on the grid and a < maxval. */

    if (v == 0.0) return f->fnuz ? 0x00 : sign;

    frexp(v, &ex);
    e = ex - 1; /* may have carried into the next binade */
    if (e < emin) {
        code = (uint8_t)(int)(v / ldexp(1.0, emin - f->mbits));
    } else {
        int mant = (int)(ldexp(v, -e) * (double)(1 << f->mbits)) - (1 << f->mbits);
        code = (uint8_t)(((e + f->bias) << f->mbits) | mant);
    }
    return (uint8_t)(sign | code);
}

void orc_decode_array(int fmt, const uint8_t* q, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(fmt, q[i]);
}

void orc_encode_array(int fmt, const float* y, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(fmt, y[i]);
}

/* scale = fp8_max / clamp(amax, min=EPS), divided in fp64; the quantize
 * multiplier is that quotient rounded to fp32, and inv_scale is the
 * reciprocal of the fp64 quotient rounded to fp32 ("FP8 Training:
 * Quantization, Autograd, Torchao", section 2 "The quantization math"). */
double orc_scale_from_amax(int fmt, float amax, double eps, float* scale, float* inv) {
    double d = (double)amax;
    double s64;
    if (d < eps) d = eps;
    s64 = FMT[fmt].maxval / d;
    if (scale) *scale = (float)s64;
    if (inv) *inv = (float)(1.0 / s64);
    return s64;
}

/* MXFP8 group scale ("FP8 training on AMD GPUs with TorchTitan and TorchAO",
 * section "AMD FP8 format in TorchAO": a scale per group stored with the
 * data). The pages give no rule; two readings are offered:
 *   mode 0: the page's scale formula rounded down to a power of two,
 *           k = floor(log2(fmax / max(amax, eps))), so amax * 2^k <= fmax
 *           and nothing clips.
 *   mode 1: the OCP MX rule, dequantization exponent
 *           floor(log2(max(amax, eps))) - floor(log2(fmax)), values above
 *           fmax saturate.
 * E8M0 holds the dequantization exponent plus 127. Callers keep eps >= 2^-100,
 * so that the exponent of an all-zero group fits E8M0. */
uint8_t orc_mx_scale_from_amax(int fmt, int mode, float amax, double eps, float* scale, float* inv) {
    int ex, kq; /* kq: quantize exponent, scale = 2^kq */
    if (mode == ORC_MX_POW2_FLOOR) {
        double s64 = orc_scale_from_amax(fmt, amax, eps, NULL, NULL);
        frexp(s64, &ex);
        kq = ex - 1; /* floor(log2 s64), exact */
    } else {
        double d = (double)amax;
        int emax_elem;
        if (d < eps) d = eps;
        frexp(d, &ex);
        frexp(FMT[fmt].maxval, &emax_elem);
        kq = -((ex - 1) - (emax_elem - 1));
    }
    if (scale) *scale = (float)ldexp(1.0, kq);
    if (inv) *inv = (float)ldexp(1.0, -kq);
    return (uint8_t)(127 - kq);
}

/* Apply the scale, clamp to +-fp8_max, cast ("FP8 Training: Quantization,
 * Autograd, Torchao", section 2): the multiply is one fp32 multiply. */
uint8_t orc_quant_elem(int fmt, uint16_t x_bf16, float scale) {
    float x = orc_bf16_to_f32(x_bf16);
    float fm = (float)FMT[fmt].maxval;
    volatile float y = x * scale; /* force one rounded fp32 product */
    float c = y;
    if (c > fm) c = fm;
    if (c < -fm) c = -fm;
    return orc_fp8_encode(fmt, c);
}

