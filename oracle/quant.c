/*
 * quant.c -- dynamic FP8 quantization at every granularity, done as the
 * literal chain of steps ("FP8 training on AMD GPUs with TorchTitan and
 * TorchAO", section "Triton Kernel Optimization": absmax per group, then
 * derive and apply the scale, then clamp and cast), each step a separate
 * loop over the group. Test infrastructure only (see fp8_oracle.h).
 *
 * Granularities ("FP8 training on AMD GPUs with TorchTitan and TorchAO",
 * section "AMD FP8 format in TorchAO": one scale per tensor, per row, per
 * fixed-size tile, or per group packed with the data (MXFP8); section
 * "Scaling FP8 to MoE Architectures": per-row activation scales and
 * per-expert-column weight scales).
 *
 * The parallel-for only splits independent groups across threads; the
 * arithmetic inside a group is the same sequential loop at any thread count.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_threads_used(int threads) {
#ifdef _OPENMP
    return threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* Step 1: amax = max |fp32(x)| over a rows x cols window with row stride ld. */
static float window_amax(const uint16_t* x, int64_t nr, int64_t nc, int64_t ld) {
    float amax = 0.0f;
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t c = 0; c < nc; ++c) {
            float v = fabsf(orc_bf16_to_f32(x[r * ld + c]));
            if (v > amax) amax = v;
        }
    return amax;
}

void orc_quant_tensor(const uint16_t* x, int64_t n, int fmt, double eps,
                      uint8_t* q, float* scale, float* inv, float* amax_out) {
    float s, i;
    float amax = window_amax(x, 1, n, n);                 /* step 1 */
    orc_scale_from_amax(fmt, amax, eps, &s, &i);          /* step 2 */
    for (int64_t k = 0; k < n; ++k) q[k] = orc_quant_elem(fmt, x[k], s); /* step 3 */
    if (scale) scale[0] = s;
    if (inv) inv[0] = i;
    if (amax_out) amax_out[0] = amax;
}

void orc_quant_row(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                   int fmt, double eps, uint8_t* q, float* scale, float* inv, int threads) {
    int64_t R = batch * rows;
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t r = 0; r < R; ++r) {
        const uint16_t* xr = x + r * cols;
        float s, i;
        float amax = window_amax(xr, 1, cols, cols);
        orc_scale_from_amax(fmt, amax, eps, &s, &i);
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = orc_quant_elem(fmt, xr[c], s);
        scale[r] = s;
        if (inv) inv[r] = i;
    }
}

void orc_quant_col(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                   int fmt, double eps, uint8_t* qT, float* scale, float* inv, int threads) {
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t bc = 0; bc < batch * cols; ++bc) {
        int64_t b = bc / cols, c = bc % cols;
        const uint16_t* xb = x + b * rows * cols;
        float s, i;
        float amax = window_amax(xb + c, rows, 1, cols); /* column c */
        orc_scale_from_amax(fmt, amax, eps, &s, &i);
        for (int64_t r = 0; r < rows; ++r)
            qT[(b * cols + c) * rows + r] = orc_quant_elem(fmt, xb[r * cols + c], s);
        scale[b * cols + c] = s;
        if (inv) inv[b * cols + c] = i;
    }
}

void orc_quant_block(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                     int64_t br, int64_t bc, int fmt, double eps,
                     uint8_t* q, float* scale, float* inv, int threads) {
    int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
    int64_t nblk = batch * nbr * nbc;
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t blk = 0; blk < nblk; ++blk) {
        int64_t b = blk / (nbr * nbc), rb = (blk / nbc) % nbr, cb = blk % nbc;
        int64_t r0 = rb * br, c0 = cb * bc;
        int64_t nr = rows - r0 < br ? rows - r0 : br;
        int64_t nc = cols - c0 < bc ? cols - c0 : bc;
        const uint16_t* xw = x + (b * rows + r0) * cols + c0;
        uint8_t* qw = q + (b * rows + r0) * cols + c0;
        float s, i;
        float amax = window_amax(xw, nr, nc, cols);
        orc_scale_from_amax(fmt, amax, eps, &s, &i);
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t c = 0; c < nc; ++c) qw[r * cols + c] = orc_quant_elem(fmt, xw[r * cols + c], s);
        scale[blk] = s;
        if (inv) inv[blk] = i;
    }
}

void orc_quant_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                  int fmt, int mode, double eps, uint8_t* q, uint8_t* e8m0, int threads) {
    int64_t ng = cols / 32;
    int64_t R = batch * rows;
    int nt = orc_threads_used(threads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const uint16_t* xg = x + r * cols + g * 32;
            float s;
            float amax = window_amax(xg, 1, 32, 32);
            e8m0[r * ng + g] = orc_mx_scale_from_amax(fmt, mode, amax, eps, &s, NULL);
            for (int64_t c = 0; c < 32; ++c) q[r * cols + g * 32 + c] = orc_quant_elem(fmt, xg[c], s);
        }
    }
}
