// common.hpp -- device helpers shared by the gfx950 kernels of the library.
//
// The quantization step follows "FP8 Training: Quantization, Autograd,
// Torchao", section 2 "The quantization math": amax = max|x| in fp32, the scale
// fp8_max / max(amax, eps) divided in fp64, the product x * scale in fp32,
// clamped to +-fp8_max and cast with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8dyn {

// Format ids, numbered as fp8_format in include/fp8dyn.h.
enum Fmt : int { kE4M3FN = 0, kE4M3FNUZ = 1, kE5M2 = 2, kE5M2FNUZ = 3 };

__host__ __device__ constexpr double fmt_max(int f) {
  return f == kE4M3FN ? 448.0 : (f == kE4M3FNUZ ? 240.0 : 57344.0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte load and 8/16-byte stores: data touched
// once should not displace reused lines in the caches.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt8(void* p, const uint2& v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// bf16 halves of a 32-bit word -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float amax8(const uint4& v, float m) {
  m = fmaxf(m, fabsf(bf16_lo(v.x)));
  m = fmaxf(m, fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fabsf(bf16_lo(v.y)));
  m = fmaxf(m, fabsf(bf16_hi(v.y)));
  m = fmaxf(m, fabsf(bf16_lo(v.z)));
  m = fmaxf(m, fabsf(bf16_hi(v.z)));
  m = fmaxf(m, fabsf(bf16_lo(v.w)));
  m = fmaxf(m, fabsf(bf16_hi(v.w)));
  return m;
}

// scale = RN32(fmax / max(amax, eps)) with an IEEE fp64 division;
// inv = RN32(1 / that fp64 quotient).
__device__ __forceinline__ void scale_from_amax(float amax, double fmax, double eps, float& scale,
                                                float& inv) {
  double d = (double)amax;
  d = d < eps ? eps : d;
  const double s = fmax / d;
  scale = (float)s;
  inv = (float)(1.0 / s);
}

// Power-of-two (MX) scale. Returns the quantize exponent k (scale = 2^k).
// mode 0: k = floor(log2(fmax / max(amax, eps))), the fp64 quotient's exponent.
// mode 1: k = floor(log2 fmax) - floor(log2 max(amax, eps)).
__device__ __forceinline__ int mx_exponent(float amax, double fmax, double eps, int mode) {
  double d = (double)amax;
  d = d < eps ? eps : d;
  if (mode == 0) {
    const double s = fmax / d;  // normal fp64 for any finite bf16 amax and eps >= 1e-300
    return (int)((__double_as_longlong(s) >> 52) & 0x7ff) - 1023;
  }
  const int ed = (int)((__double_as_longlong(d) >> 52) & 0x7ff) - 1023;
  const int em = (int)((__double_as_longlong(fmax) >> 52) & 0x7ff) - 1023;
  return em - ed;
}

__device__ __forceinline__ float exp2i(int k) {  // 2^k for k in [-126, 127]
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float clampf(float y, float fm) { return fminf(fmaxf(y, -fm), fm); }

// Hardware convert of four fp32 values to four fp8 bytes (round to nearest
// even; the OCP encodings on gfx950). E5 selects e5m2, else e4m3.
template <bool E5>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (E5) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

template <bool E5>
__device__ __forceinline__ uint8_t cvt1(float a) {
  int w;
  if constexpr (E5) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, 0.0f, 0, false);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false);
  }
  return (uint8_t)(w & 0xff);
}

// Software encoder for the fnuz variants ("FP8 training on AMD GPUs with
// TorchTitan and TorchAO", section "AMD FP8 format in TorchAO": finite, no
// negative zero; e4m3fnuz: exponent bias 8, 3 mantissa bits, max 240; e5m2fnuz:
// bias 16, 2 mantissa bits, max 57344). gfx950's converts write the OCP
// encodings, so MI300-readable bytes are produced here from the bits of the
// clamped fp32 value: round to nearest, ties to even mantissa, including the
// subnormal band (quantum 2^(1 - bias - mbits)); a value that rounds to zero
// is 0x00 whatever its sign; 0x80 (NaN) is never written. |y| <= max.
template <bool E5>
__device__ __forceinline__ uint32_t enc_fnuz(float y) {
  constexpr int MB = E5 ? 2 : 3, BIAS = E5 ? 16 : 8;
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t ab = bits & 0x7fffffffu;
  const int e = (int)(ab >> 23) - 127;  // exponent of |y| (fp32 denormals: far below the fnuz range)
  uint32_t code;
  if (e < 1 - BIAS) {
    // below the smallest normal: q = |y| / 2^(1 - BIAS - MB), rounded to even
    // (scaling by a power of two is exact; rintf rounds to nearest even)
    const float q = rintf(__uint_as_float(ab) * __uint_as_float((uint32_t)(127 + BIAS + MB - 1) << 23));
    code = (uint32_t)q;  // 2^MB here is the smallest normal: the same bits
  } else {
    // normal: keep MB of the 23 mantissa bits, round to nearest even
    constexpr int SH = 23 - MB;
    const uint32_t mant = ab & 0x7fffffu;
    uint32_t qm = mant >> SH;
    const uint32_t rem = mant & ((1u << SH) - 1), half = 1u << (SH - 1);
    qm += (rem > half || (rem == half && (qm & 1u))) ? 1u : 0u;
    code = ((uint32_t)(e + BIAS) << MB) + qm;  // a mantissa carry bumps the exponent
  }
  return code == 0 ? 0u : (sign | code);
}

// Four values -> four packed bytes (a in the low byte); NZ: the fnuz bytes.
template <bool E5, bool NZ>
__device__ __forceinline__ uint32_t cvt4x(float a, float b, float c, float d) {
  if constexpr (NZ)
    return enc_fnuz<E5>(a) | (enc_fnuz<E5>(b) << 8) | (enc_fnuz<E5>(c) << 16) | (enc_fnuz<E5>(d) << 24);
  else
    return cvt4<E5>(a, b, c, d);
}

template <bool E5, bool NZ>
__device__ __forceinline__ uint8_t cvt1x(float a) {
  if constexpr (NZ)
    return (uint8_t)enc_fnuz<E5>(a);
  else
    return cvt1<E5>(a);
}

// Eight bf16 (one 16-byte load) -> eight fp8 bytes.
template <bool E5, bool NZ = false>
__device__ __forceinline__ uint2 quant8(const uint4& v, float s, float fm) {
  uint2 r;
  r.x = cvt4x<E5, NZ>(clampf(bf16_lo(v.x) * s, fm), clampf(bf16_hi(v.x) * s, fm),
                      clampf(bf16_lo(v.y) * s, fm), clampf(bf16_hi(v.y) * s, fm));
  r.y = cvt4x<E5, NZ>(clampf(bf16_lo(v.z) * s, fm), clampf(bf16_hi(v.z) * s, fm),
                      clampf(bf16_lo(v.w) * s, fm), clampf(bf16_hi(v.w) * s, fm));
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max over a whole workgroup of NT threads; every thread gets the result.
// red must hold NT/64 floats of shared memory.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if constexpr (NT > 64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) v = fmaxf(v, red[i]);
  }
  return v;
}

// Keeps a value's registers live after the instruction that reads it. Used
// after each matrix-core instruction so the register allocator can never give
// the instruction's destination the registers of its A/B sources: the
// multi-pass f8f6f4 MFMAs produce wrong results when they overlap.
template <class T>
__host__ __device__ __forceinline__ void keep_live(const T& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(v));
#else
  (void)v;
#endif
}

__device__ __forceinline__ void atomic_max_relaxed(uint32_t* p, float v) {
  // v >= 0, so its bit pattern orders like the value.
  __hip_atomic_fetch_max(p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compute units of the current device (host side; 256 on MI355X).
inline int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return cus;
}

}  // namespace fp8dyn
