/*
 * synth.c -- seeded synthetic inputs shared by the tests, the benchmark and
 * the oracle checks. It holds none of the quantization or GEMM arithmetic:
 * only a counter-based random stream and the rounding of the generated fp32
 * values to bf16 storage.
 *
 * Stream: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014): output i is mix64(key + (i + 1) * gamma)
 * with key = mix64(seed). Normals: Box-Muller in fp64 from outputs 2j and
 * 2j + 1. Storage: fp32(sigma * z * row_multiplier) rounded to bf16, nearest
 * even.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t stream_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static double normal_at(uint64_t key, uint64_t j) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t h1 = stream_at(key, 2 * j), h2 = stream_at(key, 2 * j + 1);
    double u1 = ((double)(h1 >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(h2 >> 11) * 0x1.0p-53;         /* [0, 1) */
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static uint16_t f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v;
    v.f = f;
    v.u += 0x7FFFu + ((v.u >> 16) & 1u);
    return (uint16_t)(v.u >> 16);
}

static float bf16_to_f32(uint16_t b) {
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return v.f;
}

/* out[r][c] = bf16(fp32(sigma * z[r*cols + c] * row_mult[r])); row_mult may be NULL. */
void synth_normal_bf16(uint16_t* out, int64_t rows, int64_t cols, uint64_t seed, double sigma,
                       const double* row_mult) {
    uint64_t key = mix64(seed);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double m = row_mult ? row_mult[r] : 1.0;
        for (int64_t c = 0; c < cols; ++c) {
            uint64_t j = (uint64_t)(r * cols + c);
            out[r * cols + c] = f32_to_bf16_rne((float)(sigma * normal_at(key, j) * m));
        }
    }
}

/* Element i becomes an outlier when its stream value falls below p * 2^64:
 * x[i] = bf16(fp32(x[i]) * mult). Returns the number of outliers. */
int64_t synth_outliers_bf16(uint16_t* x, int64_t n, uint64_t seed, double p, float mult) {
    uint64_t key = mix64(seed);
    uint64_t thr = (uint64_t)(p * 18446744073709551616.0);
    int64_t count = 0;
#pragma omp parallel for schedule(static) reduction(+ : count)
    for (int64_t i = 0; i < n; ++i) {
        if (stream_at(key, (uint64_t)i) < thr) {
            x[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) * mult);
            ++count;
        }
    }
    return count;
}

/* Uniform doubles in [0, 1) from the same stream (for small host-side choices). */
void synth_uniform(double* out, int64_t n, uint64_t seed) {
    uint64_t key = mix64(seed);
    for (int64_t i = 0; i < n; ++i) out[i] = (double)(stream_at(key, (uint64_t)i) >> 11) * 0x1.0p-53;
}
