/*
 * fp8dyn.h -- C ABI of the MI355X (gfx950) dynamic-FP8 library: fused
 * absmax -> scale -> clamp -> cast quantization at five granularities, and
 * the scaled FP8 GEMMs (dense and MoE grouped) that consume those scales.
 *
 * The operations are the ones described on these pages:
 *  [P-AMD]  "FP8 training on AMD GPUs with TorchTitan and TorchAO: upstreaming
 *           performance" (AMD blog): section "AMD FP8 format in TorchAO"
 *           (e4m3fnuz table; tensorwise / rowwise / blockwise / MXFP8
 *           granularities), section "Scaling FP8 to MoE Architectures"
 *           (Figure 3: per-row activation scales, per-expert-column weight
 *           scales, an offset tensor routing rows to experts, one launch),
 *           section "Triton Kernel Optimization" (the chain absmax -> scale ->
 *           clamp and cast, fused into one pass), Levels 1-3 (no transpose
 *           copy, coalesced transposed stores, relaxed atomics).
 *  [P-TAO]  "FP8 Training: Quantization, Autograd, Torchao": section 2 "The
 *           quantization math" (amax, fp64 scale with an eps clamp, clamp and
 *           cast, inverse scale), section 3 "Format choice" (e4m3 448 / fnuz
 *           240 / e5m2 57344; e4m3 for activations and weights, e5m2 for
 *           gradients), section 4 "_scaled_mm layout requirements" (A
 *           row-major, B column-major, the GEMM multiplies by the inverse
 *           scales), section 6 (three GEMMs per linear layer).
 *
 * Conventions shared by every call
 *  - Pointers named x, w, gy, a, b, q, scale, inv_scale, out, y, gx, gw, ws,
 *    offsets are DEVICE pointers owned by the caller. The library never
 *    allocates or frees memory in a call and keeps no pointer after it
 *    returns. Its only state is a per-device cache of fp8_probe's answer and,
 *    for fp8_quant_col_noalloc, one 64 KiB device buffer per GPU.
 *  - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *  - stream is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on it and returns; results are valid once the stream has
 *    been synchronized. No call reads device data back to the host, and no
 *    call synchronizes the device except the one-time probe (fp8_probe) that
 *    the first *_NATIVE format resolution on a device runs.
 *  - Every argument is validated on the host before anything is launched; on
 *    any error nothing is launched and the status says why. Launch failures return
 *    FP8_ERR_DEVICE; faults inside a kernel surface at the caller's next
 *    synchronization (fp8_last_device_error keeps the last HIP error seen).
 *  - Zero dimensions. Whatever holds no elements is neither read nor written
 *    (its pointer may be NULL). A quantization group with no elements (a row
 *    of 0 columns, a column of 0 rows, a tensor of 0 elements) still gets its
 *    scale: amax over an empty set is 0, so scale = fp8_max / eps. A GEMM
 *    with K = 0, and a weight gradient over M = 0 rows, write zeros (the
 *    empty sum) without reading any operand or scale. Anything else with a
 *    zero dimension does nothing.
 *  - eps must be finite and > 0; 1e-12 is the usual value.
 *  - Quantization writes `scale` (the quantize multiplier fp8_max/amax) and,
 *    when inv_scale is not NULL, its fp64 reciprocal rounded to fp32. GEMMs
 *    take only the inverse scales.
 *  - Device pointers to bf16/fp8 data must be 16-byte aligned, scale arrays
 *    4-byte aligned.
 */
#ifndef FP8DYN_H
#define FP8DYN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FP8DYN_API __attribute__((visibility("default")))
#else
#define FP8DYN_API
#endif

/* FP8 encodings [P-TAO section 3 table; P-AMD "AMD FP8 format in TorchAO"].
 * *_NATIVE resolve, per device, to the variant this GPU's converts and
 * matrix cores use, as measured by fp8_probe. */
typedef enum {
    FP8_E4M3FN = 0,      /* OCP e4m3: max 448, has -0, NaN = 0x7F/0xFF */
    FP8_E4M3FNUZ = 1,    /* max 240, no -0, 0x80 = NaN */
    FP8_E5M2 = 2,        /* OCP e5m2: max 57344, has -0, inf/NaN */
    FP8_E5M2FNUZ = 3,    /* max 57344, no -0, 0x80 = NaN */
    FP8_E4M3_NATIVE = 4,
    FP8_E5M2_NATIVE = 5
} fp8_format;

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum, eps <= 0 */
    FP8_ERR_ALIGNMENT = 2,        /* pointer or size alignment rule broken */
    FP8_ERR_UNSUPPORTED = 3,      /* format or shape this GPU/library cannot do */
    FP8_ERR_WORKSPACE = 4,        /* workspace missing or too small */
    FP8_ERR_DEVICE = 5            /* a HIP call failed */
} fp8_status;

typedef enum {
    FP8_SCALE_TENSOR = 0,   /* one inverse scale per operand: a_inv[1], b_inv[1] */
    FP8_SCALE_ROW = 1,      /* a_inv[M], b_inv[N] (grouped: b_inv[E][N]) */
    FP8_SCALE_BLOCK128 = 2, /* a_inv[M][K/128], b_inv[E][N/128][K/128] */
    FP8_SCALE_MX32 = 3      /* E8M0 bytes: a[M][K/32], b[E][N][K/32] */
} fp8_scaling;

typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_F32 = 1 } fp8_out;

typedef enum {
    FP8_MX_POW2_FLOOR = 0, /* scale = largest 2^k with amax*2^k <= fp8_max (never clips) */
    FP8_MX_OCP = 1         /* OCP MX rule: 2^(floor(log2 amax) - emax_elem), saturating */
} fp8_mx_mode;

typedef enum {
    FP8_NORM_RMS = 0,   /* y = x / sqrt(mean(x^2) + norm_eps) * gamma */
    FP8_NORM_LAYER = 1  /* y = (x - mean) / sqrt(var + norm_eps) * gamma + beta */
} fp8_norm;

typedef enum {
    FP8_RECIPE_TENSORWISE = 0,        /* one scale per tensor, all GEMMs FP8 */
    FP8_RECIPE_ROWWISE_BF16_WGRAD = 1 /* rowwise FP8 forward and grad-input; BF16 grad-weight */
} fp8_recipe;

/* ---- device facts -------------------------------------------------------- */

/* Measures, on `device`, which e4m3 and e5m2 variants the hardware FP8
 * converts and FP8 matrix-core instructions use (a wrong max silently
 * corrupts results [P-AMD "AMD FP8 format in TorchAO"]). Runs two tiny
 * kernels and synchronizes once; the answer is cached per device. The first
 * call on a device that resolves a *_NATIVE format (any quantization or GEMM
 * call) runs this probe and so synchronizes that device once; later calls
 * read the cache.
 * Returns FP8_ERR_UNSUPPORTED if the device is not gfx950 or the converts and
 * the matrix cores disagree. Output pointers are host pointers, may be NULL. */
FP8DYN_API fp8_status fp8_probe(int device, fp8_format* e4m3_native, fp8_format* e5m2_native);

FP8DYN_API const char* fp8_status_string(fp8_status s);
/* The last HIP error code (hipError_t value) the library saw, 0 if none. */
FP8DYN_API int fp8_last_device_error(void);
/* Largest finite value of a format (host helper; NATIVE formats need a probed device). */
FP8DYN_API double fp8_format_max(fp8_format f);

/* ---- quantization [P-TAO section 2; P-AMD "Triton Kernel Optimization"] ----
 * Per group g: amax = max |x| (fp32); s = fp8_max / max(amax, eps) in fp64;
 * scale[g] = (float)s; inv_scale[g] = (float)(1/s);
 * q = RNE-encode(clamp((float)x * scale[g], -fp8_max, fp8_max)).
 * Formats: the two NATIVE variants (after fp8_probe) are supported by every
 * call. fp8_quant_tensor and fp8_quant_row also write FP8_E4M3FNUZ and
 * FP8_E5M2FNUZ on an OCP device (gfx950) for MI300-generation interop [P-AMD
 * "AMD FP8 format in TorchAO": the fnuz variants, max 240 / 57344, no
 * negative zero]: a software encoder, not the hardware converts, so slower;
 * those bytes are for storage or export, no GEMM here reads them. Other
 * non-native requests return FP8_ERR_UNSUPPORTED. Each call is one pass over
 * x except where stated. */

/* One scale for all n elements. Needs a device workspace of
 * fp8_quant_tensor_ws_bytes() bytes (ws, 256-byte aligned); its content on
 * entry does not matter. Three stream-ordered launches: clear, amax with
 * relaxed atomics [P-AMD Level 3], cast. x: [n] bf16, q: [n]. */
FP8DYN_API fp8_status fp8_quant_tensor(const uint16_t* x, int64_t n, fp8_format fmt, double eps,
                                       uint8_t* q, float* scale, float* inv_scale,
                                       void* ws, size_t ws_bytes, void* stream);
FP8DYN_API size_t fp8_quant_tensor_ws_bytes(void);

/* Row groups: x [batch][rows][cols] -> q same layout, scale/inv [batch][rows]. */
FP8DYN_API fp8_status fp8_quant_row(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                    fp8_format fmt, double eps, uint8_t* q, float* scale,
                                    float* inv_scale, void* stream);

/* Row groups as fp8_quant_row (same scales, same codes), with the codes
 * written "k-packed" for fp8_grouped_mm_kpacked's B operand: within each
 * batch slice, code (r, c) goes to byte ((r / 16) * (cols / 64) + c / 64)
 * * 1024 + (r % 16) * 64 + c % 64, i.e. 1 KB chunks of 16 rows x 64 columns,
 * chunks ordered by column block within a 16-row group. rows % 16 == 0 and
 * cols % 64 == 0 (else FP8_ERR_ALIGNMENT), cols <= 16384 (else
 * FP8_ERR_UNSUPPORTED); native formats only. q holds batch * rows * cols
 * bytes. */
FP8DYN_API fp8_status fp8_quant_row_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                            fp8_format fmt, double eps, uint8_t* q, float* scale,
                                            float* inv_scale, void* stream);

/* Row groups as fp8_quant_row (same scales, same codes), with the codes
 * pair-interleaved for fp8_grouped_mm_kpacked's A operand: within each batch
 * slice, code (r, c) goes to byte ((r / 2) * (cols / 64) + c / 64) * 128 +
 * (r % 2) * 64 + c % 64, so rows 2i and 2i + 1 share each 128-byte line of a
 * 64-column block. rows % 2 == 0 and cols % 64 == 0 (else
 * FP8_ERR_ALIGNMENT), cols <= 16384 (else FP8_ERR_UNSUPPORTED); native
 * formats only. */
FP8DYN_API fp8_status fp8_quant_row_kpaired(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                            fp8_format fmt, double eps, uint8_t* q, float* scale,
                                            float* inv_scale, void* stream);

/* Column groups with the transposed output the GEMM's column-major operand
 * needs [P-TAO section 4; P-AMD Level 1 and Level 2]: x [batch][rows][cols] ->
 * qT [batch][cols][rows], scale/inv [batch][cols]. One launch when rows <=
 * 2048 or the tensor has at least 1024 strips of 64 columns (batch *
 * ceil(cols / 64)); otherwise a column-amax launch over row chunks with
 * relaxed atomics and a cast launch, which need ws of
 * fp8_quant_col_ws_bytes(batch, rows, cols) bytes (0 when one launch does). */
FP8DYN_API fp8_status fp8_quant_col(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                    fp8_format fmt, double eps, uint8_t* qT, float* scale,
                                    float* inv_scale, void* ws, size_t ws_bytes, void* stream);

/* Column groups as fp8_quant_col (same scales, same codes), with qT written
 * k-packed as the [cols][rows] B operand of fp8_scaled_mm_kpacked: within each
 * batch slice, code (n = column, k = row) at byte ((n / 16) * (rows / 64) +
 * k / 64) * 1024 + (n % 16) * 64 + k % 64. rows % 64 == 0, cols % 16 == 0
 * (else FP8_ERR_ALIGNMENT), rows * cols < 2^30 (else FP8_ERR_UNSUPPORTED);
 * native formats only; the same workspace as fp8_quant_col. */
FP8DYN_API fp8_status fp8_quant_col_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                            fp8_format fmt, double eps, uint8_t* qT, float* scale,
                                            float* inv_scale, void* ws, size_t ws_bytes, void* stream);
FP8DYN_API size_t fp8_quant_col_ws_bytes(int64_t batch, int64_t rows, int64_t cols);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fp8_quant_col with no workspace argument -- the same kernels, codes and
 * scales. The split form's column-amax words live in a 64 KiB buffer the
 * library keeps in device memory, one per GPU, held until the process ends;
 * its device address is looked up once per device on the first call there.
 * Limit: fp8_quant_col_ws_bytes(batch, rows, cols) <= 65536, i.e. at most
 * 16384 columns (batch * cols) when the split form is used; larger problems
 * return FP8_ERR_UNSUPPORTED before anything is launched. Nothing is
 * allocated or freed. Every call on one GPU shares that GPU's buffer and
 * clears the words it uses with a fill kernel on its stream: calls on
 * streams of one GPU that are not ordered with each other race on it. */
FP8DYN_API fp8_status fp8_quant_col_noalloc(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                            fp8_format fmt, double eps, uint8_t* qT, float* scale,
                                            float* inv_scale, void* stream);

/* Normalization fused with the rowwise quantization of its output ["FP8
 * Training: Quantization, Autograd, Torchao" section 8: the norm's output
 * write and the next layer's amax pass as one memory pass]. Per row of x
 * [rows][cols] bf16: the row statistics in fp64 (sums of x and x^2; mean,
 * var = E[x^2] - mean^2 for LAYER, rstd = 1/sqrt(var + norm_eps)), then
 *   y = ((x - mean32) * rstd32) * gamma + beta   (LAYER; beta may be NULL = 0)
 *   y = (x * rstd32) * gamma                     (RMS; beta must be NULL)
 * in fp32 IEEE operations on mean32 = (float)mean, rstd32 = (float)rstd,
 * stored as bf16 (RNE): the activation an unfused norm would write. q, scale,
 * inv_scale are then exactly fp8_quant_row of that bf16 row. x is read once;
 * y [rows][cols] is written only if non-NULL (the backward's copy); q may be
 * NULL (normalization only). gamma, beta [cols] bf16. cols % 8 == 0 (else
 * FP8_ERR_ALIGNMENT), cols <= 16384 (else FP8_ERR_UNSUPPORTED); x, gamma,
 * beta, y 16-byte aligned, q 8-byte aligned. NATIVE formats only. */
FP8DYN_API fp8_status fp8_norm_quant_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                                         int64_t rows, int64_t cols, fp8_norm kind, double norm_eps,
                                         fp8_format fmt, double eps, uint16_t* y, uint8_t* q, float* scale,
                                         float* inv_scale, void* stream);

/* Dual tensorwise quantization for the all-FP8 Linear backward ["FP8
 * Training: Quantization, Autograd, Torchao" section 4: grad_weight =
 * grad_output^T @ input takes grad_output transposed (row-major [N][M]) and
 * the input column-major; "FP8 training on AMD GPUs with TorchTitan and
 * TorchAO" Figure 4 caption: a companion kernel quantizes grad_output and the
 * activation together]. One scale per tensor (amax over the whole tensor,
 * then the scale rule of fp8_quant_tensor); one amax launch over gy and x,
 * then ONE cast launch that reads each input once and writes
 *   gq  [M][N] = ENC(gy * g_scale), row-major (grad-input GEMM's A); may be NULL
 *   gqT [N][M] = the same bytes transposed (grad-weight GEMM's A)
 *   xqT [K][M] = ENC(x * x_scale) transposed (grad-weight GEMM's B).
 * gy [M][N], x [M][K] bf16 row-major; g_scale, x_scale [1] (inv: [1] or
 * NULL). All pointers device memory owned by the caller. M % 16 == 0,
 * N % 8 == 0, K % 8 == 0 (else FP8_ERR_ALIGNMENT); M*N and M*K < 2^30 (else
 * FP8_ERR_UNSUPPORTED); gy, x, gqT, xqT 16-byte aligned, gq 8-byte aligned.
 * ws: fp8_quant_dual_ws_bytes() bytes, 256-byte aligned (two amax words). */
FP8DYN_API fp8_status fp8_quant_dual(const uint16_t* gy, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                                     fp8_format g_fmt, fp8_format x_fmt, double eps, uint8_t* gq, uint8_t* gqT,
                                     float* g_scale, float* g_inv, uint8_t* xqT, float* x_scale, float* x_inv,
                                     void* ws, size_t ws_bytes, void* stream);
FP8DYN_API size_t fp8_quant_dual_ws_bytes(void);

/* Blocks of block_rows x block_cols (1x128 for activations, 128x128 for
 * weights [P-AMD "AMD FP8 format in TorchAO", blockwise]): x
 * [batch][rows][cols] -> q same layout, scale/inv
 * [batch][ceil(rows/block_rows)][ceil(cols/block_cols)]. Partial edge blocks
 * use their valid elements. block_rows in {1, 128}, block_cols == 128. */
FP8DYN_API fp8_status fp8_quant_block(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                      int block_rows, int block_cols, fp8_format fmt, double eps,
                                      uint8_t* q, float* scale, float* inv_scale, void* stream);

/* MXFP8: 32 consecutive elements along cols share one E8M0 power-of-two
 * scale [P-AMD "AMD FP8 format in TorchAO", MXFP8; "Summary and Next Steps"].
 * e8m0[g] = 127 + log2(dequantize factor); q = encode(clamp(x * 2^k)).
 * cols % 32 == 0. x [batch][rows][cols] -> q same, e8m0 [batch][rows][cols/32].
 * eps >= 2^-100 (else FP8_ERR_INVALID_ARGUMENT): then every group's exponent,
 * an all-zero group's included, fits E8M0 (bytes 12 .. 247). */
FP8DYN_API fp8_status fp8_quant_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                   fp8_format fmt, fp8_mx_mode mode, double eps, uint8_t* q,
                                   uint8_t* e8m0, void* stream);

/* MXFP8 as fp8_quant_mx (same codes, same E8M0 bytes, e8m0 row-major), with
 * the codes written in the packed layouts of fp8_grouped_mm_kpacked's
 * operands: _kpacked, its B, code (r, c) of each batch slice at byte
 * ((r / 16) * (cols / 64) + c / 64) * 1024 + (r % 16) * 64 + c % 64 (as
 * fp8_quant_row_kpacked), rows % 16 == 0; _kpaired, its A, at
 * ((r / 2) * (cols / 64) + c / 64) * 128 + (r % 2) * 64 + c % 64 (as
 * fp8_quant_row_kpaired), rows % 2 == 0. Both need cols % 64 == 0 and
 * 16-byte aligned x and q (else FP8_ERR_ALIGNMENT); native formats only.
 * q holds batch * rows * cols bytes. */
FP8DYN_API fp8_status fp8_quant_mx_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                           fp8_format fmt, fp8_mx_mode mode, double eps, uint8_t* q,
                                           uint8_t* e8m0, void* stream);
FP8DYN_API fp8_status fp8_quant_mx_kpaired(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                           fp8_format fmt, fp8_mx_mode mode, double eps, uint8_t* q,
                                           uint8_t* e8m0, void* stream);

/* ---- GEMMs [P-TAO section 4; P-AMD "Scaling FP8 to MoE Architectures"] ----
 * out[m][n] = a_inv * b_inv * sum_k dec(a[m][k]) * dec(b[n][k]) on the matrix
 * cores, scales applied in fp32, stored as bf16 (round to nearest even) or
 * fp32.
 * a: [M][K] row-major codes; b: [N][K] row-major codes, i.e. the column-major
 * K x N operand (a Linear weight as stored). fa in {e4m3, e5m2} native
 * variants; fb must be the e4m3 native variant (an e5m2 B returns
 * FP8_ERR_UNSUPPORTED). K % 16 == 0 (K % 128 == 0 for BLOCK128, K % 32 == 0
 * for MX32).
 * use_fast_accum [P-TAO section 5: fast accumulation in the forward, full
 * precision in both backward GEMMs]:
 *  - nonzero: the FP8 matrix-core instructions. Measured on MI355X, each
 *    one aligns its products to the largest of them and keeps about 12 bits
 *    below it (error up to ~2^-12 of the instruction's largest product,
 *    independent of the accumulator); full FP8 rate.
 *  - 0: full precision. The codes are decoded to bf16 (every e4m3 and e5m2
 *    value is a bf16 value) and summed by the BF16 matrix-core instructions,
 *    which accumulate at fp32 precision; the BF16 rate, half the FP8 one.
 * fp8_scaled_mm scaling: TENSOR or ROW. */
FP8DYN_API fp8_status fp8_scaled_mm(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                    fp8_scaling scaling, const float* a_inv, const float* b_inv,
                                    int64_t M, int64_t N, int64_t K, fp8_out out_type, void* out,
                                    int use_fast_accum, void* stream);

/* fp8_scaled_mm with b k-packed ([N][K] codes in 1 KB chunks of 16 rows x
 * 64 K, as fp8_quant_row_kpacked writes a weight and fp8_quant_col_kpacked a
 * transposed one): the same result. Scaling TENSOR or ROW. N % 16 == 0 and
 * K % 128 == 0 (else FP8_ERR_ALIGNMENT); N * K < 2^31 and 16-byte aligned a,
 * b (else FP8_ERR_UNSUPPORTED). use_fast_accum as for fp8_scaled_mm. */
FP8DYN_API fp8_status fp8_scaled_mm_kpacked(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                            fp8_scaling scaling, const float* a_inv, const float* b_inv,
                                            int64_t M, int64_t N, int64_t K, fp8_out out_type, void* out,
                                            int use_fast_accum, void* stream);

/* MoE grouped GEMM in one launch: rows [offsets[e], offsets[e+1]) of a use
 * expert e's b[e] ([E][N][K]) and scales. offsets: DEVICE int32 [E+1] with
 * offsets[0] = 0, non-decreasing, offsets[E] = Mtot (not read back; use
 * fp8_validate_offsets on a host copy to check). Empty experts are skipped.
 * Scaling: ROW (a_inv [Mtot] float, b_inv [E][N] float), BLOCK128
 * (a_inv [Mtot][K/128], b_inv [E][N/128][K/128] float; N % 128 == 0) or MX32
 * (E8M0 bytes a [Mtot][K/32], b [E][N][K/32]). use_fast_accum as for
 * fp8_scaled_mm; with MX32 and use_fast_accum == 0 the E8M0 scales are
 * folded into the bf16 decode (exact while the scaled codes stay in bf16's
 * range). */
FP8DYN_API fp8_status fp8_grouped_mm(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                     fp8_scaling scaling, const void* a_scale, const void* b_scale,
                                     const int32_t* offsets, int32_t E, int64_t Mtot, int64_t N,
                                     int64_t K, fp8_out out_type, void* out, int use_fast_accum,
                                     void* stream);

/* fp8_grouped_mm with a pair-interleaved as fp8_quant_row_kpaired writes it
 * and b k-packed as fp8_quant_row_kpacked writes it (each expert's [N][K]
 * codes as 1 KB chunks of 16 rows x 64 K): the same result. The
 * matrix-core kernel loads a 64-deep stage of 16 rows of each operand from
 * HBM into LDS; row-major, that is 16 half cache lines, here 8 or 9 whole
 * lines of A (an expert may start at an odd row) and one contiguous KB of B.
 * Scaling ROW or MX32 (scales as for fp8_grouped_mm, row-major); BLOCK128
 * and TENSOR return FP8_ERR_UNSUPPORTED. N % 16 == 0, K % 128 == 0 and
 * Mtot % 2 == 0 (else FP8_ERR_ALIGNMENT); N * K < 2^31, K < 2^22 and
 * 16-byte aligned a, b (else FP8_ERR_UNSUPPORTED). use_fast_accum as for
 * fp8_scaled_mm; full precision (0) with ROW scaling only, else
 * FP8_ERR_UNSUPPORTED. */
FP8DYN_API fp8_status fp8_grouped_mm_kpacked(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                             fp8_scaling scaling, const void* a_scale, const void* b_scale,
                                             const int32_t* offsets, int32_t E, int64_t Mtot, int64_t N,
                                             int64_t K, fp8_out out_type, void* out, int use_fast_accum,
                                             void* stream);

/* BF16 weight-gradient GEMM [P-AMD Figure 1 caption: the weight-update GEMM
 * stays in BF16]: gw[n][k] = sum_m gy[m][n] * x[m][k], fp32 accumulation,
 * bf16 out. gy [M][N], x [M][K], gw [N][K], all bf16 row-major; no
 * transposed copies are made. N % 8 == 0 and K % 8 == 0 (else
 * FP8_ERR_ALIGNMENT); any M >= 0 (M = 0 writes zeros); gy and x 16-byte
 * aligned, gw 4-byte aligned. */
FP8DYN_API fp8_status fp8_wgrad_bf16(const uint16_t* gy, const uint16_t* x, int64_t M, int64_t N,
                                     int64_t K, uint16_t* gw, void* stream);

/* Grouped BF16 weight gradient of an MoE layer over device offsets, the
 * weight side of the grouped GEMM's backward ["FP8 training on AMD GPUs with
 * TorchTitan and TorchAO" Figure 1 caption: the weight-update GEMM stays in
 * BF16; section
 * "Scaling FP8 to MoE Architectures": expert e owns rows [off[e], off[e+1])]:
 *   gw[e][n][k] = sum over m in [off[e], off[e+1]) of gy[m][n] * x[m][k],
 * fp32 accumulation, bf16 out (RNE); an expert with no rows gets zeros.
 * gy [Mtot][N], x [Mtot][K] bf16 row-major (the grouped forward's output
 * gradient and input, as stored: no transposed copies), gw [E][N][K] bf16.
 * offsets: device int32[E+1] with offsets[0] == 0, non-decreasing,
 * offsets[E] == Mtot (check a host copy with fp8_validate_offsets; the
 * kernel trusts them and never reads them back to the host). N % 8 == 0,
 * K % 8 == 0, gy and x 16-byte aligned (else FP8_ERR_ALIGNMENT);
 * 64 * max(N, K) < 2^31 and E <= 1024 (else FP8_ERR_UNSUPPORTED). */
FP8DYN_API fp8_status fp8_grouped_wgrad_bf16(const uint16_t* gy, const uint16_t* x, const int32_t* offsets,
                                             int32_t E, int64_t Mtot, int64_t N, int64_t K, uint16_t* gw,
                                             void* stream);

/* ---- one Linear layer [P-TAO section 6; P-AMD "AMD FP8 format in TorchAO"] ---
 * Forward y = x w^T: x [M][K], w [N][K] bf16; quantize both (TENSORWISE: one
 * scale each; ROWWISE: per row of x and of w, e4m3), then the scaled GEMM
 * with the accumulation use_fast_accum selects (as for fp8_scaled_mm; the
 * pages' recipe runs the forward with fast accumulation [P-TAO section 5]);
 * y [M][N] bf16 or fp32. TENSORWISE quantizes x and w together, one amax
 * launch and one cast launch for both (same codes and scales as two
 * fp8_quant_tensor calls); x and w 16-byte aligned (else FP8_ERR_ALIGNMENT).
 * ROWWISE with N % 16 == 0, K % 128 == 0 and K <= 16384 writes w k-packed
 * (fp8_quant_row_kpacked, fp8_scaled_mm_kpacked), except for outputs of at
 * most one 64 x 64 tile per compute unit, which the GEMM's small-output form
 * takes row-major. eps as for the quantizers (else FP8_ERR_INVALID_ARGUMENT).
 * ws: fp8_linear_ws_bytes(M, N, K, recipe) bytes. */
FP8DYN_API fp8_status fp8_linear_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                     int64_t K, fp8_recipe recipe, double eps, fp8_out out_type,
                                     int use_fast_accum, void* y, void* ws, size_t ws_bytes, void* stream);
/* Backward ["FP8 Training: Quantization, Autograd, Torchao" section 4: the
 * grad-input and grad-weight GEMMs]: gy [M][N], x [M][K], w [N][K] bf16.
 * gx [M][K] bf16 = FP8 GEMM of gy (e5m2) and w (e4m3, written transposed
 * [K][N]; per column of w for ROWWISE). gw [N][K] bf16:
 *  - TENSORWISE: all-FP8, gw = (gy^T in e5m2) x (x in e4m3) over m, with the
 *    operands gy^T [N][M] and x^T [K][M] written by the same single cast
 *    launch that writes gy [M][N] and w^T (fp8_quant_dual's kernels, one
 *    scale per tensor); needs M % 16 == 0 (else FP8_ERR_ALIGNMENT) and
 *    M*N, M*K, N*K < 2^30 (else FP8_ERR_UNSUPPORTED);
 *  - ROWWISE_BF16_WGRAD: the BF16 GEMM gy^T x ["FP8 training on AMD GPUs
 *    with TorchTitan and TorchAO" Figure 1 caption]; with N % 128 == 0 and
 *    K % 16 == 0 w^T is written k-packed (fp8_quant_col_kpacked) for the
 *    grad-input GEMM, unless gx has at most one 64 x 64 tile per compute
 *    unit (then row-major, as in the forward).
 * eps as for the quantizers (else FP8_ERR_INVALID_ARGUMENT).
 * Both FP8 GEMMs of the backward use full-precision accumulation [P-TAO
 * section 5]. */
FP8DYN_API fp8_status fp8_linear_bwd(const uint16_t* gy, const uint16_t* x, const uint16_t* w,
                                     int64_t M, int64_t N, int64_t K, fp8_recipe recipe, double eps,
                                     uint16_t* gx, uint16_t* gw, void* ws, size_t ws_bytes,
                                     void* stream);
FP8DYN_API size_t fp8_linear_ws_bytes(int64_t M, int64_t N, int64_t K, fp8_recipe recipe);

/* Host helper: checks a HOST copy of an offsets array (offsets[0] == 0,
 * non-decreasing, offsets[E] == Mtot). */
FP8DYN_API fp8_status fp8_validate_offsets(const int32_t* host_offsets, int32_t E, int64_t Mtot);

#ifdef __cplusplus
}
#endif
#endif
