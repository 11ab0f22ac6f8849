// gemm_common.hpp -- pieces shared by the FP8 GEMM kernels: parameters, the
// per-expert tile walk over device offsets, bf16 rounding.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace fp8dyn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Full-precision accumulation ("FP8 Training: Quantization, Autograd,
// Torchao", section 5: use_fast_accum off). Measured on MI355X, an FP8
// matrix-core instruction aligns its products to the largest one and keeps
// about 12 bits below it, whatever the accumulator holds; the BF16
// instruction sums at fp32 precision. Every e4m3 and e5m2 value is exactly a
// bf16 value, so decoding the codes to bf16 and running the BF16 instruction
// gives the same products with fp32 accumulation. bf16x8: the 8 codes of
// bytes [8 q, 8 q + 8) of a 32-byte fragment, decoded by gfx950's converts
// (scale 1). Both operands of a product go through the same byte positions,
// so each 8-byte piece pairs A and B codes of the same K.
template <bool E5>
__device__ __forceinline__ v8bf bf16x8(const v8i& f, int q) {
  const uint32_t d0 = (uint32_t)f[2 * q], d1 = (uint32_t)f[2 * q + 1];
  v2bf p0, p1, p2, p3;
  if constexpr (E5) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  }
  return (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The value 2^(e - 127) of an E8M0 byte as fp32 (e = 0: 2^-127, a subnormal;
// e = 255: NaN).
__device__ __forceinline__ float e8m0_to_f32(int e) {
  const uint32_t bits = e == 0 ? 0x00400000u : e == 255 ? 0x7fc00000u : (uint32_t)e << 23;
  return __builtin_bit_cast(float, bits);
}

// bf16x8 with every decoded code multiplied by `scale`, a power of two (an
// E8M0 group scale; exact while the products stay inside bf16's range).
template <bool E5>
__device__ __forceinline__ v8bf bf16x8_scaled(const v8i& f, int q, float scale) {
  const uint32_t d0 = (uint32_t)f[2 * q], d1 = (uint32_t)f[2 * q + 1];
  v2bf p0, p1, p2, p3;
  if constexpr (E5) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
  }
  return (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

constexpr int kMaxExperts = 1024;
constexpr int kGroupM = 4;
constexpr int kNumXcd = 8;

struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  const int32_t* offsets;
  int32_t E;
  int64_t M, N, K;
  void* out;
};

// Tile bookkeeping shared by the workgroup.
struct TileInfo {
  int64_t m0, m_end, n0;
  int32_t e;
};

template <int BM, int BN>
__device__ __forceinline__ void tile_of(int64_t t, const int32_t* s_off, const int64_t* s_pref, int E, int64_t nt,
                                        TileInfo& ti) {
  // expert: largest e with s_pref[e] <= t (s_pref[E] = total)
  int lo = 0, hi = E;  // invariant: s_pref[lo] <= t < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= t) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int64_t u = t - s_pref[e];
  const int64_t mrows = (int64_t)s_off[e + 1] - s_off[e];
  const int64_t mt = (mrows + BM - 1) / BM;
  const int64_t g = u / (kGroupM * nt);
  const int64_t rem = u % (kGroupM * nt);
  const int64_t gm = (mt - g * kGroupM) < kGroupM ? (mt - g * kGroupM) : kGroupM;
  const int64_t ntile = rem / gm, mtile = g * kGroupM + rem % gm;
  ti.e = e;
  ti.m0 = s_off[e] + mtile * BM;
  ti.m_end = s_off[e + 1];
  ti.n0 = ntile * BN;
}


__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Thread 0 makes the offsets in LDS usable as given or not: each is clamped
// into [0, Mtot] and to at least its predecessor (a running max), so offsets
// that break the contract (offsets[0] = 0, non-decreasing, offsets[E] = Mtot)
// can route rows to the wrong expert or leave rows unwritten, but never
// address outside the operands or the output. Valid offsets pass unchanged.
__device__ __forceinline__ void clamp_offsets_serial(int32_t* s_off, int E, int64_t Mtot) {
  int64_t prev = 0;
  for (int i = 0; i <= E; ++i) {
    int64_t v = s_off[i];
    v = v < prev ? prev : v;
    v = v > Mtot ? Mtot : v;
    s_off[i] = (int32_t)v;
    prev = v;
  }
}

// Reads offsets[0..E] into LDS (clamped as above) and builds the prefix of
// tiles per expert. Dense problems pass offsets == nullptr: one expert
// covering rows [0, M). Returns the total number of tiles.
template <int BM, int NT>
__device__ __forceinline__ int64_t build_tile_prefix(const GemmParams& p, int64_t nt, int32_t* s_off,
                                                     int64_t* s_pref) {
  const int tid = threadIdx.x;
  const int E = p.E;
  if (p.offsets) {
    for (int i = tid; i <= E; i += NT) s_off[i] = p.offsets[i];
  } else if (tid == 0) {
    s_off[0] = 0;
    s_off[1] = (int32_t)p.M;
  }
  __syncthreads();
  if (tid == 0) {
    if (p.offsets) clamp_offsets_serial(s_off, E, p.M);
    int64_t acc = 0;
    for (int e = 0; e < E; ++e) {
      s_pref[e] = acc;
      const int64_t mrows = (int64_t)s_off[e + 1] - s_off[e];
      acc += (mrows > 0 ? (mrows + BM - 1) / BM : 0) * nt;
    }
    s_pref[E] = acc;
  }
  __syncthreads();
  return s_pref[E];
}

// XCD-aware split of the tile list: with the grid a multiple of the 8 XCDs,
// XCD x (workgroups dealt round robin) owns tiles [x*T/8, (x+1)*T/8) and its
// workgroups walk them in order, so concurrently running workgroups of one
// XCD share operands in that XCD's L2.
__device__ __forceinline__ void xcd_range(int64_t total, int64_t& t_begin, int64_t& t_end, int64_t& t_step) {
  const int64_t G = gridDim.x;
  const int64_t per_xcd_blocks = G / kNumXcd;
  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  if (per_xcd_blocks > 0 && G % kNumXcd == 0) {
    t_begin = xcd * total / kNumXcd + slot;
    t_end = (xcd + 1) * total / kNumXcd;
    t_step = per_xcd_blocks;
  } else {
    t_begin = blockIdx.x;
    t_end = total;
    t_step = G;
  }
}

// ---- LDS DMA pipeline helpers (gfx950) ----

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide 16-byte-per-lane load from global (uniform base + per-lane
// 32-bit offset) into LDS at lds (uniform; lane i lands at lds + 16 i).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm_and_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace fp8dyn
