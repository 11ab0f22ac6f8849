/*
 * fp8_oracle.h -- plain, slow CPU oracle for dynamic FP8 quantization and
 * scaled FP8 GEMMs.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library (the HIP kernels, the
 * C-ABI, the Python binding) may include, link, load or call this code. The
 * only users are the test suite, the smoke check and the benchmark's CPU
 * baseline leg. It shares no header, table, helper or constant with the GPU
 * path.
 *
 * What it follows (citations name the page and its section):
 *  [Q]  "FP8 Training: Quantization, Autograd, Torchao", section 2 "The
 *       quantization math": amax = max|x| in fp32, scale = fp8_max /
 *       clamp(amax in fp64, EPS), x*scale clamped to +-fp8_max then cast,
 *       inv_scale = reciprocal of the fp64 scale.
 *  [F]  same page, section 3 "Format choice: e4m3 vs e5m2" (table of max
 *       values 448 / 240 / 57344, 3 vs 2 mantissa bits) and
 *       "FP8 training on AMD GPUs with TorchTitan and TorchAO", section
 *       "AMD FP8 format in TorchAO" (e4m3fnuz table: max 240, no NaN/Inf,
 *       unsigned zero).
 *  [C]  "FP8 training on AMD GPUs with TorchTitan and TorchAO", section
 *       "Triton Kernel Optimization": the chain absmax -> derive and apply
 *       scale -> clamp and cast, which this oracle runs step by step.
 *  [G]  same page, sections "AMD FP8 format in TorchAO" (granularities:
 *       tensorwise, rowwise, blockwise, MXFP8) and "Scaling FP8 to MoE
 *       Architectures" (per-row activation scales, per-expert-column weight
 *       scales, offsets routing rows to experts; Figure 3).
 *  [S]  "FP8 Training: Quantization, Autograd, Torchao", section 4
 *       "_scaled_mm layout requirements": A row-major, B column-major,
 *       dequantize by multiplying by inv_a * inv_b.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - eps is an argument (1e-12 by convention).
 *  - the product x*scale is an fp32 multiply of fp32(x) by RN32(scale64).
 *  - the cast rounds to nearest, ties to even, and saturates at +-max.
 *  - fnuz formats have no negative zero: every value rounding to zero
 *    encodes as 0x00; e4m3fn / e5m2 keep the sign (0x80).
 *  - MX scales are powers of two: k = floor(log2(scale64)), stored as the
 *    E8M0 exponent 127 - k of the dequantization factor 2^-k (mode 0), or
 *    the OCP MX rule floor(log2 amax) - emax_elem with saturation (mode 1).
 *  - each GEMM operand is scaled along its non-contracted index.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Formats known to the oracle. */
enum { ORC_E4M3FN = 0, ORC_E4M3FNUZ = 1, ORC_E5M2 = 2, ORC_E5M2FNUZ = 3 };

/* MX scale rules. */
enum { ORC_MX_POW2_FLOOR = 0, ORC_MX_OCP = 1 };

/* GEMM scaling kinds. */
enum { ORC_SCALE_TENSOR = 0, ORC_SCALE_ROW = 1, ORC_SCALE_BLOCK128 = 2, ORC_SCALE_MX32 = 3 };

/* ---- codec ---------------------------------------------------------------- */
double  orc_fp8_max(int fmt);                 /* largest finite value */
double  orc_fp8_decode(int fmt, uint8_t code);/* NaN for NaN codes, +-inf for e5m2 inf */
uint8_t orc_fp8_encode(int fmt, float y);     /* RNE, saturating, format's zero sign rule */
float   orc_bf16_to_f32(uint16_t b);
void    orc_decode_array(int fmt, const uint8_t* q, int64_t n, double* out);
void    orc_encode_array(int fmt, const float* y, int64_t n, uint8_t* out);

/* ---- scale derivation ---------------------------------------------------- */
/* scale = RN32(fmax / max(amax, eps)) with the division in fp64;
 * inv = RN32(1 / that fp64 quotient). Returns the fp64 quotient. */
double  orc_scale_from_amax(int fmt, float amax, double eps, float* scale, float* inv);
/* MX: returns the E8M0 byte; *scale = 2^k (quantize multiplier),
 * *inv = 2^-k (dequantize multiplier). */
uint8_t orc_mx_scale_from_amax(int fmt, int mode, float amax, double eps, float* scale, float* inv);
/* One element: ENC(clamp(RN32(f32(x) * scale), -fmax, fmax)). */
uint8_t orc_quant_elem(int fmt, uint16_t x_bf16, float scale);

/* ---- quantization at each granularity -------------------------------------
 * x is bf16 bits, row-major [batch][rows][cols]. Threads: 0 = all available. */
void orc_quant_tensor(const uint16_t* x, int64_t n, int fmt, double eps,
                      uint8_t* q, float* scale, float* inv, float* amax_out);
void orc_quant_row(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                   int fmt, double eps, uint8_t* q, float* scale, float* inv, int threads);
/* Column groups: amax over rows; output transposed qT[batch][cols][rows]. */
void orc_quant_col(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                   int fmt, double eps, uint8_t* qT, float* scale, float* inv, int threads);
/* Blocks of br x bc (partial edge blocks take the valid elements);
 * scales [batch][ceil(rows/br)][ceil(cols/bc)]. */
void orc_quant_block(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                     int64_t br, int64_t bc, int fmt, double eps,
                     uint8_t* q, float* scale, float* inv, int threads);
/* 32-element groups along cols (cols % 32 == 0); e8m0 [batch][rows][cols/32]. */
void orc_quant_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                  int fmt, int mode, double eps, uint8_t* q, uint8_t* e8m0, int threads);

/* ---- normalization, then rowwise quantization (norm.c) ---------------------
 * x [rows][cols] bf16, gamma [cols] and beta [cols] (LayerNorm, may be NULL)
 * bf16; layer: 1 LayerNorm, 0 RMSNorm. y [rows][cols] bf16 (the normalized
 * activation); q/scale/inv as orc_quant_row of y. */
void orc_norm_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                  int64_t cols, int layer, double norm_eps, uint16_t* y);
/* The row sums the normalization starts from: s1[r] = sum x, s2[r] = sum x^2,
 * each the exact sum rounded once to fp64. */
void orc_norm_stats(const uint16_t* x, int64_t rows, int64_t cols, double* s1, double* s2);
void orc_norm_quant_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                        int64_t cols, int layer, double norm_eps, int fmt, double eps, uint16_t* y,
                        uint8_t* q, float* scale, float* inv);

/* ---- GEMMs in fp64 (results unrounded) -------------------------------------
 * a: [M][K] codes (row-major), b: [N][K] codes (the column-major K x N operand).
 * out[m][n] = inv_a * inv_b * sum_k dec(a[m][k]) * dec(b[n][k]).
 * TENSOR: a_inv[0], b_inv[0]; ROW: a_inv[M], b_inv[N]. */
void orc_scaled_mm(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                   const float* a_inv, const float* b_inv,
                   int64_t M, int64_t N, int64_t K, double* out, int threads);

/* Grouped: rows [off[e], off[e+1]) of a use b[e] ([E][N][K]).
 * ROW:      a_inv [Mtot], b_inv [E][N]                      (float)
 * BLOCK128: a_inv [Mtot][K/128], b_inv [E][N/128][K/128]     (float)
 * MX32:     a_sc [Mtot][K/32], b_sc [E][N][K/32]             (E8M0 bytes)
 * offsets are host int32 [E+1]. */
void orc_grouped_mm(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                    const void* a_scale, const void* b_scale, const int32_t* offsets,
                    int32_t E, int64_t Mtot, int64_t N, int64_t K, double* out, int threads);
/* Same, for a list of (row, col) output positions only. */
void orc_grouped_mm_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                           const void* a_scale, const void* b_scale, const int32_t* offsets,
                           int32_t E, int64_t Mtot, int64_t N, int64_t K,
                           const int64_t* rows, const int64_t* cols, int64_t ns, double* out);
void orc_scaled_mm_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                          const float* a_inv, const float* b_inv, int64_t M, int64_t N, int64_t K,
                          const int64_t* rows, const int64_t* cols, int64_t ns, double* out);

/* BF16 weight gradient: dw[n][k] = sum_m g[m][n] * x[m][k] in fp64.
 * g: [M][N] bf16, x: [M][K] bf16 (both contiguous along the kept index). */
void orc_wgrad_bf16(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                    double* dw, int threads);
void orc_wgrad_bf16_sample(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                           const int64_t* ns_idx, const int64_t* ks_idx, int64_t ns, double* out);

/* The same sums with every product taken in absolute value, times |scales|:
 * S = sum_k |dec(a) dec(b)| |inv_a inv_b| (per scale block). S bounds the
 * rounding error of any summation order of the product (componentwise error
 * analysis of dot products), so GEMM checks compare |y - ref| against it. */
void orc_scaled_mm_abs(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                       const float* a_inv, const float* b_inv,
                       int64_t M, int64_t N, int64_t K, double* out, int threads);
void orc_scaled_mm_abs_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                              const float* a_inv, const float* b_inv, int64_t M, int64_t N, int64_t K,
                              const int64_t* rows, const int64_t* cols, int64_t ns, double* out);
void orc_grouped_mm_abs(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                        const void* a_scale, const void* b_scale, const int32_t* offsets,
                        int32_t E, int64_t Mtot, int64_t N, int64_t K, double* out, int threads);
void orc_grouped_mm_abs_sample(const uint8_t* a, int fa, const uint8_t* b, int fb, int scaling,
                               const void* a_scale, const void* b_scale, const int32_t* offsets,
                               int32_t E, int64_t Mtot, int64_t N, int64_t K,
                               const int64_t* rows, const int64_t* cols, int64_t ns, double* out);
void orc_wgrad_bf16_abs(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                        double* dw, int threads);
void orc_wgrad_bf16_abs_sample(const uint16_t* g, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                               const int64_t* ns_idx, const int64_t* ks_idx, int64_t ns, double* out);

int orc_threads_used(int threads);

#ifdef __cplusplus
}
#endif
#endif
