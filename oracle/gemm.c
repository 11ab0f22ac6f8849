/*
 * gemm.c -- scaled FP8 GEMMs and the BF16 weight-gradient GEMM in fp64.
 * Test infrastructure only (see fp8_oracle.h).
 *
 * Contract ("FP8 Training: Quantization, Autograd, Torchao", section 4
 * "_scaled_mm layout requirements" and section 2): A is [M][K] row-major, B is
 * the column-major K x N operand stored as [N][K]; the product is dequantized
 * by multiplying by the two inverse scales. Grouped form ("FP8 training on
 * AMD GPUs with TorchTitan and TorchAO", section "Scaling FP8 to MoE
 * Architectures", Figure 3): an offset tensor assigns row ranges of A to
 * experts, each expert with its own B and per-column scales. Blockwise and MX
 * scales vary along K, so the sum is split at the scale boundaries and each
 * partial sum is multiplied by its own pair of scales. The weight gradient
 * stays in BF16 (same page, Figure 1 caption), here an fp64 sum of exact
 * bf16 x bf16 products.
 *
 * Every dot product is a plain sequential loop over k in fp64. For e4m3 x
 * e4m3 each product is a multiple of 2^-18 below 2^18 and the sum is exact in
 * any order for K up to 2^17, so the result is the exact value up to the
 * final rounding.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct { double v[256]; } dec_table;

static void build_table(int fmt, dec_table* t) {
    for (int c = 0; c < 256; ++c) t->v[c] = orc_fp8_decode(fmt, (uint8_t)c);
}

/* sum_k dec(a_k) * dec(b_k); with absolute != 0, sum_k |dec(a_k) * dec(b_k)|. */
static double dot(const dec_table* ta, const uint8_t* a, const dec_table* tb, const uint8_t* b, int64_t n,
                  int absolute) {
    double acc = 0.0;
    if (absolute) {
        for (int64_t k = 0; k < n; ++k) acc += fabs(ta->v[a[k]] * tb->v[b[k]]);
    } else {
        for (int64_t k = 0; k < n; ++k) acc += ta->v[a[k]] * tb->v[b[k]];
    }
    return acc;
}

static double e8m0_value(uint8_t e) { return ldexp(1.0, (int)e - 127); }

/* One output element of the grouped (or dense, E = 1) product. */
static double grouped_elem(const dec_table* ta, const dec_table* tb, const uint8_t* a, const uint8_t* b,
                           int scaling, const void* a_scale, const void* b_scale, int64_t e,
                           int64_t m, int64_t n, int64_t N, int64_t K, int ab) {
    const uint8_t* ar = a + m * K;
    const uint8_t* br = b + (e * N + n) * K;
    if (scaling == ORC_SCALE_TENSOR) {
        const float* sa = (const float*)a_scale;
        const float* sb = (const float*)b_scale;
        double sc = (double)sa[0] * (double)sb[0];
        return dot(ta, ar, tb, br, K, ab) * (ab ? fabs(sc) : sc);
    }
    if (scaling == ORC_SCALE_ROW) {
        const float* sa = (const float*)a_scale;
        const float* sb = (const float*)b_scale;
        double sc = (double)sa[m] * (double)sb[e * N + n];
        return dot(ta, ar, tb, br, K, ab) * (ab ? fabs(sc) : sc);
    }
    if (scaling == ORC_SCALE_BLOCK128) {
        const float* sa = (const float*)a_scale;
        const float* sb = (const float*)b_scale;
        int64_t nkb = K / 128, nnb = N / 128;
        double acc = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
            double part = dot(ta, ar + kb * 128, tb, br + kb * 128, 128, ab);
            double sc = (double)sa[m * nkb + kb] * (double)sb[(e * nnb + n / 128) * nkb + kb];
            acc += part * (ab ? fabs(sc) : sc);
        }
        return acc;
    }
    {   /* MX32 */
        const uint8_t* sa = (const uint8_t*)a_scale;
        const uint8_t* sb = (const uint8_t*)b_scale;
        int64_t ng = K / 32;
        double acc = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
            double part = dot(ta, ar + g * 32, tb, br + g * 32, 32, ab);
            acc += part * e8m0_value(sa[m * ng + g]) * e8m0_value(sb[(e * N + n) * ng + g]);
        }
        return acc;
    }
}

static void scaled_mm_impl(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                           const float* a_inv, const float* b_inv,
                           int64_t M, int64_t N, int64_t K, double* out, int threads, int ab) {
    dec_table ta, tb;
    int nt = orc_threads_used(threads);
    (void)nt;
    build_table(fa, &ta);
    build_table(fb, &tb);
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = grouped_elem(&ta, &tb, a, b, scaling, a_inv, b_inv, 0, m, n, N, K, ab);
}

void orc_scaled_mm(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                   const float* a_inv, const float* b_inv,
                   int64_t M, int64_t N, int64_t K, double* out, int threads) {
    scaled_mm_impl(a, fa, b, fb, scaling, a_inv, b_inv, M, N, K, out, threads, 0);
}

void orc_scaled_mm_abs(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                       const float* a_inv, const float* b_inv,
                       int64_t M, int64_t N, int64_t K, double* out, int threads) {
    scaled_mm_impl(a, fa, b, fb, scaling, a_inv, b_inv, M, N, K, out, threads, 1);
}

static void scaled_mm_sample_impl(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                                  const float* a_inv, const float* b_inv, int64_t N, int64_t K,
                                  const int64_t* rows, const int64_t* cols, int64_t ns, double* out, int ab) {
    dec_table ta, tb;
    build_table(fa, &ta);
    build_table(fb, &tb);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < ns; ++i)
        out[i] = grouped_elem(&ta, &tb, a, b, scaling, a_inv, b_inv, 0, rows[i], cols[i], N, K, ab);
}

void orc_scaled_mm_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                          const float* a_inv, const float* b_inv, int64_t M, int64_t N, int64_t K,
                          const int64_t* rows, const int64_t* cols, int64_t ns, double* out) {
    (void)M;
    scaled_mm_sample_impl(a, fa, b, fb, scaling, a_inv, b_inv, N, K, rows, cols, ns, out, 0);
}

void orc_scaled_mm_abs_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                              const float* a_inv, const float* b_inv, int64_t M, int64_t N, int64_t K,
                              const int64_t* rows, const int64_t* cols, int64_t ns, double* out) {
    (void)M;
    scaled_mm_sample_impl(a, fa, b, fb, scaling, a_inv, b_inv, N, K, rows, cols, ns, out, 1);
}

/* Expert owning row m: the e with off[e] <= m < off[e+1]. */
static int64_t expert_of(const int32_t* off, int32_t E, int64_t m) {
    for (int64_t e = 0; e < E; ++e)
        if (m >= off[e] && m < off[e + 1]) return e;
    return -1;
}

static void grouped_mm_impl(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                            const void* a_scale, const void* b_scale, const int32_t* offsets,
                            int32_t E, int64_t Mtot, int64_t N, int64_t K, double* out, int threads, int ab) {
    dec_table ta, tb;
    int nt = orc_threads_used(threads);
    (void)nt;
    build_table(fa, &ta);
    build_table(fb, &tb);
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t m = 0; m < Mtot; ++m) {
        int64_t e = expert_of(offsets, E, m);
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = e < 0 ? 0.0 : grouped_elem(&ta, &tb, a, b, scaling, a_scale, b_scale, e, m, n, N, K, ab);
    }
}

void orc_grouped_mm(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                    const void* a_scale, const void* b_scale, const int32_t* offsets,
                    int32_t E, int64_t Mtot, int64_t N, int64_t K, double* out, int threads) {
    grouped_mm_impl(a, fa, b, fb, scaling, a_scale, b_scale, offsets, E, Mtot, N, K, out, threads, 0);
}

void orc_grouped_mm_abs(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                        const void* a_scale, const void* b_scale, const int32_t* offsets,
                        int32_t E, int64_t Mtot, int64_t N, int64_t K, double* out, int threads) {
    grouped_mm_impl(a, fa, b, fb, scaling, a_scale, b_scale, offsets, E, Mtot, N, K, out, threads, 1);
}

static void grouped_sample_impl(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                                const void* a_scale, const void* b_scale, const int32_t* offsets,
                                int32_t E, int64_t N, int64_t K,
                                const int64_t* rows, const int64_t* cols, int64_t ns, double* out, int ab) {
    dec_table ta, tb;
    build_table(fa, &ta);
    build_table(fb, &tb);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < ns; ++i) {
        int64_t e = expert_of(offsets, E, rows[i]);
        out[i] = e < 0 ? 0.0
                       : grouped_elem(&ta, &tb, a, b, scaling, a_scale, b_scale, e, rows[i], cols[i], N, K, ab);
    }
}

void orc_grouped_mm_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                           const void* a_scale, const void* b_scale, const int32_t* offsets,
                           int32_t E, int64_t Mtot, int64_t N, int64_t K,
                           const int64_t* rows, const int64_t* cols, int64_t ns, double* out) {
    (void)Mtot;
    grouped_sample_impl(a, fa, b, fb, scaling, a_scale, b_scale, offsets, E, N, K, rows, cols, ns, out, 0);
}

void orc_grouped_mm_abs_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                               const void* a_scale, const void* b_scale, const int32_t* offsets,
                               int32_t E, int64_t Mtot, int64_t N, int64_t K,
                               const int64_t* rows, const int64_t* cols, int64_t ns, double* out) {
    (void)Mtot;
    grouped_sample_impl(a, fa, b, fb, scaling, a_scale, b_scale, offsets, E, N, K, rows, cols, ns, out, 1);
}

static double wgrad_elem(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                         int64_t n, int64_t k, int ab) {
    double acc = 0.0;
    for (int64_t m = 0; m < M; ++m) {
        double p = (double)orc_bf16_to_f32(g[m * N + n]) * (double)orc_bf16_to_f32(x[m * K + k]);
        acc += ab ? fabs(p) : p;
    }
    return acc;
}

void orc_wgrad_bf16(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                    double* dw, int threads) {
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) dw[n * K + k] = wgrad_elem(g, x, M, N, K, n, k, 0);
}

void orc_wgrad_bf16_abs(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                        double* dw, int threads) {
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) dw[n * K + k] = wgrad_elem(g, x, M, N, K, n, k, 1);
}

void orc_wgrad_bf16_sample(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                           const int64_t* ns_idx, const int64_t* ks_idx, int64_t ns, double* out) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < ns; ++i) out[i] = wgrad_elem(g, x, M, N, K, ns_idx[i], ks_idx[i], 0);
}

void orc_wgrad_bf16_abs_sample(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                               const int64_t* ns_idx, const int64_t* ks_idx, int64_t ns, double* out) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < ns; ++i) out[i] = wgrad_elem(g, x, M, N, K, ns_idx[i], ks_idx[i], 1);
}
