// quant.hip -- fused dynamic FP8 quantization kernels for gfx950.
//
// Each kernel does the whole chain of "FP8 training on AMD GPUs with
// TorchTitan and TorchAO", section "Triton Kernel Optimization" (absmax per
// group, derive and apply the scale, clamp and cast) in one pass over HBM,
// with the group's data held in registers between the reduction and the
// cast, so nothing intermediate is written (Level 1 of that page). The math is
// that of "FP8 Training: Quantization, Autograd, Torchao", section 2.
//
// Memory design for MI355X: 16-byte loads per lane, 8-byte (or 16-byte)
// stores, amax reduced with wavefront shuffles and a few words of LDS,
// fp64 scale derived redundantly per lane (cheaper than a broadcast), and
// the hardware packed converts (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32).
#include "common.hpp"
#include "internal.hpp"

namespace fp8dyn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Row groups. One workgroup of 256 threads per row; the row (up to
// 2048 * J elements) stays in registers between amax and cast.
template <int J, bool E5>
__global__ __launch_bounds__(256) void k_quant_row(const uint16_t* __restrict__ x, int64_t cols,
                                                   uint8_t* __restrict__ q, float* __restrict__ scale,
                                                   float* __restrict__ inv, double fmax, double eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * cols;
  uint8_t* qr = q + row * cols;
  const int tid = threadIdx.x;
  uint4 v[J];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(tid + 256 * j) * 8;
    if (c < cols) {
      v[j] = ld_nt16(xr + c);
      m = amax8(v[j], m);
    }
  }
  m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (tid == 0) {
    scale[row] = s;
    if (inv) inv[row] = iv;
  }
  const float fm = (float)fmax;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(tid + 256 * j) * 8;
    if (c < cols) {
      uint2 r = quant8<E5>(v[j], s, fm);
      st_nt8(qr + c, r);
    }
  }
}

// Rowwise groups with the codes written k-packed: row r, column c of a batch
// slice's [rows][cols] codes lands at ((r / 16) * (cols / 64) + c / 64) * 1024
// + (r % 16) * 64 + c % 64, i.e. 1 KB chunks of 16 rows x 64 columns (the
// layout the grouped GEMM loads a stage of B from in whole cache lines). One
// 256-thread workgroup per row as in k_quant_row; a row's 64-byte pieces are
// half lines whose other halves belong to the neighbouring row, so rows are
// dealt to XCDs in contiguous ranges (workgroup i runs on XCD i % 8) and the
// two halves meet in one L2; plain stores let it merge them.
// G = 2: the pair-interleaved rows of a grouped GEMM's A (chunks of 2 rows x
// 64 columns, 128 bytes), otherwise G = 16.
template <int J, bool E5, int G>
__global__ __launch_bounds__(256) void k_quant_row_kpacked(const uint16_t* __restrict__ x, int64_t nrows,
                                                           int64_t cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale, float* __restrict__ inv,
                                                           double fmax, double eps) {
  __shared__ float red[4];
  // (tensors below 2^26 elements keep the plain order, which measured faster
  // there: the k-packed [14336][4096] weight 36.0 against 36.6 us, a
  // pair-interleaved [8192][4096] activation 22.8 against 24.9 us, cold input)
  const int64_t nwg = gridDim.x;
  int64_t row = blockIdx.x;
  if (nwg % 8 == 0 && nrows * cols >= ((int64_t)1 << 26)) row = (row % 8) * (nwg / 8) + row / 8;
  const uint16_t* xr = x + row * cols;
  // chunk row (row / G, 0) of the packed codes, then this row's 64 bytes in it
  uint8_t* qg = q + (row / G) * G * cols + (row % G) * 64;
  const int tid = threadIdx.x;
  uint4 v[J];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(tid + 256 * j) * 8;
    if (c < cols) {
      v[j] = ld_nt16(xr + c);
      m = amax8(v[j], m);
    }
  }
  m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (tid == 0) {
    scale[row] = s;
    if (inv) inv[row] = iv;
  }
  const float fm = (float)fmax;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(tid + 256 * j) * 8;
    if (c < cols) *reinterpret_cast<uint2*>(qg + (c / 64) * (64 * G) + c % 64) = quant8<E5>(v[j], s, fm);
  }
}

// Row groups, one wavefront per row (4 rows per 256-thread workgroup): the
// row (up to 512 * J elements) stays in registers, the amax is reduced with
// wavefront shuffles only (no LDS, no workgroup barrier), so each wave
// streams independently and keeps J 16-byte loads in flight.
// PAIRED: codes pair-interleaved as k_quant_row_kpacked<.., 2> writes them
// (rows 2i, 2i + 1 share each 128-byte line of a 64-column block); the two
// rows of a pair are waves of one workgroup, so both halves of a line are
// stored from one CU.
template <int J, bool E5, bool PAIRED = false>
__global__ __launch_bounds__(256) void k_quant_row_wave(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale,
                                                        float* __restrict__ inv, double fmax, double eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* xr = x + row * cols;
  // paired: row r's 64-column block b at ((r / 2) * (cols / 64) + b) * 128 +
  // (r % 2) * 64
  uint8_t* qr = PAIRED ? q + (row >> 1) * 2 * cols + (row & 1) * 64 : q + row * cols;
  uint4 v[J];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(lane + 64 * j) * 8;
    if (c < cols) {
      v[j] = ld_nt16(xr + c);
      m = amax8(v[j], m);
    }
  }
  m = wave_max(m);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (lane == 0) {
    scale[row] = s;
    if (inv) inv[row] = iv;
  }
  const float fm = (float)fmax;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = (int64_t)(lane + 64 * j) * 8;
    if (c < cols) {
      if constexpr (PAIRED)
        *reinterpret_cast<uint2*>(qr + (c / 64) * 128 + c % 64) = quant8<E5>(v[j], s, fm);
      else
        st_nt8(qr + c, quant8<E5>(v[j], s, fm));
    }
  }
}

// Any row length / alignment: two passes over the row (the second hits cache).
// NZ: fnuz output bytes (interop with MI300-generation GPUs).
template <bool E5, bool NZ = false>
__global__ __launch_bounds__(256) void k_quant_row_generic(const uint16_t* __restrict__ x, int64_t cols,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale,
                                                           float* __restrict__ inv, double fmax, double eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * cols;
  float m = 0.0f;
  for (int64_t c = threadIdx.x; c < cols; c += 256)
    m = fmaxf(m, fabsf(__uint_as_float((uint32_t)xr[c] << 16)));
  m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (threadIdx.x == 0) {
    scale[row] = s;
    if (inv) inv[row] = iv;
  }
  const float fm = (float)fmax;
  for (int64_t c = threadIdx.x; c < cols; c += 256)
    q[row * cols + c] = cvt1x<E5, NZ>(clampf(__uint_as_float((uint32_t)xr[c] << 16) * s, fm));
}

// ---------------------------------------------------------------------------
// Column groups with transposed output qT[b][c][r]. A 256-thread workgroup
// owns a strip of 64 columns over a range of rows. Lane layout: l8 = tid % 8
// picks 8 adjacent columns (one 16-byte load per row), rg = tid / 8 picks a
// row group.
//
// Pass 1 streams the strip (rows rg, rg + 32, ...) and reduces the 64 column
// maxima (wavefront shuffles, then 4 words per column in LDS). Pass 2 reads
// the strip again, 16 consecutive rows x 8 columns per thread, and packs the
// 16 rows of each column into 16 bytes with the packed converts (each
// convert's pair of inputs is two consecutive rows of one column), so every
// store instruction writes 8 columns x 128 contiguous bytes of qT: the
// coalesced transposed store of "FP8 training on AMD GPUs with TorchTitan and
// TorchAO", Level 2, formed in registers instead of an LDS transpose.
// Pass 2 walks the strip backwards, so the rows pass 1 read last (still in
// L2) are read first; HBM sees the strip once per pass at most and in the
// common case the second read is served by L2 / the Infinity Cache.
//
// MODE 0: both passes, the workgroup covers all rows of its strip.
// MODE 1: pass 2 only; column amax from colmax[] (cm_stride 1: per column,
//         0: one word for the whole tensor).
// MODE 2: pass 1 only over a row chunk: relaxed atomic max into colmax[]
//         ("FP8 training on AMD GPUs with TorchTitan and TorchAO", Level 3).
constexpr int kColRPT = 16;     // rows per thread in pass 2
// rows per workgroup in the split form (measured on the Llama3-8B weight,
// 14336 x 4096: 512 rows 56 us, 256 or 768 rows 58 us, 1024 rows 59 us)
constexpr int kColChunk = 512;
constexpr int kDualChunk = 1024;  // rows per block of the dual cast below

// The 16 codes of column n, rows k0 .. k0 + 15 (k0 % 16 == 0) of a transposed
// [N][K] operand: k-packed (1 KB chunks of 16 n x 64 k, see k_quant_row_kpacked)
// with a plain store, so the L2 merges the half lines of neighbouring n; else
// row-major with a non-temporal store.
template <bool PK>
__device__ __forceinline__ void store_col16(uint8_t* qs, uint32_t n, uint32_t k0, uint32_t K, const uint4& v) {
  if constexpr (PK) {
    *reinterpret_cast<uint4*>(qs + ((n >> 4) * (K >> 6) + (k0 >> 6)) * 1024u + (n & 15u) * 64u + (k0 & 63u)) = v;
  } else {
    st_nt16(qs + n * K + k0, v);
  }
}

template <bool E5, int MODE, bool PK = false>
__global__ __launch_bounds__(256, 4) void k_quant_col(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                   int64_t strips, int64_t rchunks, int64_t rows_per_blk,
                                                   uint8_t* __restrict__ qT, float* __restrict__ scale,
                                                   float* __restrict__ inv, uint32_t* __restrict__ colmax,
                                                   int64_t cm_stride, double fmax, double eps) {
  __shared__ float red[4][64];
  __shared__ float s_scale[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l8 = tid & 7, rg = tid >> 3;
  // strip fastest: the workgroups of one row chunk run side by side and
  // together read whole rows, rather than 128-byte pieces of rows far apart
  int64_t blk = blockIdx.x;
  const int64_t strip = blk % strips;
  blk /= strips;
  const int64_t rc = blk % rchunks;
  const int64_t b = blk / rchunks;
  const int64_t c0 = strip * 64 + l8 * 8;
  const bool cok = c0 < C;
  const int64_t r_beg = rc * rows_per_blk;
  const int64_t r_end = r_beg + rows_per_blk < R ? r_beg + rows_per_blk : R;
  const uint16_t* xb = x + b * R * C + c0;

  if constexpr (MODE != 1) {
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0.0f;
    if (cok) {
      for (int64_t base = r_beg; base < r_end; base += 8 * 32) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t r = base + rg + 32 * u;
          // plain loads: pass 2 reads these lines again
          v[u] = r < r_end ? *reinterpret_cast<const uint4*>(xb + r * C) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          m[0] = fmaxf(m[0], fabsf(bf16_lo(v[u].x)));
          m[1] = fmaxf(m[1], fabsf(bf16_hi(v[u].x)));
          m[2] = fmaxf(m[2], fabsf(bf16_lo(v[u].y)));
          m[3] = fmaxf(m[3], fabsf(bf16_hi(v[u].y)));
          m[4] = fmaxf(m[4], fabsf(bf16_lo(v[u].z)));
          m[5] = fmaxf(m[5], fabsf(bf16_hi(v[u].z)));
          m[6] = fmaxf(m[6], fabsf(bf16_lo(v[u].w)));
          m[7] = fmaxf(m[7], fabsf(bf16_hi(v[u].w)));
        }
      }
    }
    // reduce over the 8 row groups of the wave (lanes with equal l8)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m[i] = fmaxf(m[i], __shfl_xor(m[i], 8, 64));
      m[i] = fmaxf(m[i], __shfl_xor(m[i], 16, 64));
      m[i] = fmaxf(m[i], __shfl_xor(m[i], 32, 64));
    }
    if (lane < 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    }
    __syncthreads();
    if (tid < 64) {
      const float cm = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
      const int64_t c = strip * 64 + tid;
      if constexpr (MODE == 2) {
        if (c < C) atomic_max_relaxed(colmax + b * C + c, cm);
      } else {
        float s, iv;
        scale_from_amax(cm, fmax, eps, s, iv);
        s_scale[tid] = s;
        if (c < C) {
          scale[b * C + c] = s;
          if (inv) inv[b * C + c] = iv;
        }
      }
    }
    if constexpr (MODE == 2) return;
  } else {
    if (tid < 64) {
      const int64_t c = strip * 64 + tid;
      const int64_t si = (b * C + c) * cm_stride;
      const float cm = c < C ? __uint_as_float(colmax[si]) : 0.0f;
      float s, iv;
      scale_from_amax(cm, fmax, eps, s, iv);
      s_scale[tid] = s;
      if (rc == 0 && c < C && (cm_stride != 0 || (b == 0 && c == 0))) {
        scale[si] = s;
        if (inv) inv[si] = iv;
      }
    }
  }
  __syncthreads();
  if (!cok) return;

  const float fm = (float)fmax;
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = s_scale[l8 * 8 + i];
  // Uniform bases of this strip plus 32-bit per-lane byte offsets (one batch
  // slice is below 2^31 bytes; the launcher checks).
  const uint8_t* xs = reinterpret_cast<const uint8_t*>(x + b * R * C + strip * 64);
  uint8_t* qs = qT + (b * C + strip * 64) * R;
  const uint32_t row_b = (uint32_t)(C * 2);
  const uint32_t R32 = (uint32_t)R;
  // 16-row groups of this thread: g = rg, rg + 32, ... (walked backwards)
  const int64_t ngroups = (r_end - r_beg) / kColRPT;  // rows are a multiple of 16
  const int64_t last = rg + ((ngroups - 1 - rg) >= 0 ? ((ngroups - 1 - rg) / 32) * 32 : -32);
  for (int64_t g = last; g >= rg; g -= 32) {
    const uint32_t r0 = (uint32_t)(r_beg + g * kColRPT);
    const uint32_t xo = r0 * row_b + (uint32_t)(l8 * 16);
    // pk[i][d]: column i, rows r0 + 4d .. r0 + 4d + 3 as four fp8 bytes
    uint32_t pk[8][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ld_nt16(xs + xo + (uint32_t)(8 * h + j) * row_b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = (i < 2) ? v[j].x : (i < 4) ? v[j].y : (i < 6) ? v[j].z : v[j].w;
          f[j] = clampf(((i & 1) ? bf16_hi(w) : bf16_lo(w)) * sc[i], fm);
        }
        pk[i][2 * h] = cvt4<E5>(f[0], f[1], f[2], f[3]);
        pk[i][2 * h + 1] = cvt4<E5>(f[4], f[5], f[6], f[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      store_col16<PK>(qs, (uint32_t)(l8 * 8 + i), r0, R32, make_uint4(pk[i][0], pk[i][1], pk[i][2], pk[i][3]));
  }
}

// Single pass for up to 2048 rows. A workgroup holds a strip of CW columns x
// all rows in registers: 16 rows x 8 columns = 64 VGPRs per thread; lanes:
// lc = tid % (CW / 8) picks 8 adjacent columns, rg = tid / (CW / 8) picks 16
// consecutive rows. It reduces the CW column maxima, then casts and stores
// from the same registers with the transposed 16-byte packing described above
// (each store instruction writes CW / 8 columns x 16 * 64 / (CW / 8)
// contiguous bytes). With fewer rows several workgroups share a CU, so some
// load while others cast and store; at 2048 rows (1024 threads of about 90
// VGPRs) one fits. Consecutive strips go to the same XCD (strips narrower
// than 64 columns share 128-byte lines of x).
#ifndef FP8DYN_COL_CW
#define FP8DYN_COL_CW 64
#endif
constexpr int kColCW = FP8DYN_COL_CW;

template <bool E5, int CW, bool PK = false>
__global__ __launch_bounds__(2048 / 16 * (CW / 8)) void k_quant_col_reg(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t strips, uint8_t* __restrict__ qT,
    float* __restrict__ scale, float* __restrict__ inv, double fmax, double eps) {
  constexpr int LPR = CW / 8;                 // lanes per row
  constexpr int MAXW = 2048 / 16 * LPR / 64;  // waves at 2048 rows
  __shared__ float red[MAXW][CW];
  __shared__ float s_scale[CW];
  const int tid = threadIdx.x;
  const int nwaves = blockDim.x >> 6;
  const int lane = tid & 63, wave = tid >> 6;
  const int lc = tid % LPR, rg = tid / LPR;
  int64_t blk = blockIdx.x;
  const int64_t G = gridDim.x;
  if (G % 8 == 0) blk = (blk % 8) * (G / 8) + blk / 8;
  const int64_t strip = blk % strips;
  const int64_t b = blk / strips;
  const int64_t c0 = strip * CW + lc * 8;
  const bool cok = c0 < C;
  const int64_t r0 = (int64_t)rg * kColRPT;
  const bool rok = cok && r0 < R;  // R % 16 == 0: a row group is all in or all out
  const uint8_t* xs = reinterpret_cast<const uint8_t*>(x + b * R * C + strip * CW);
  const uint32_t row_b = (uint32_t)(C * 2);
  const uint32_t xo = (uint32_t)r0 * row_b + (uint32_t)(lc * 16);

  uint4 v[kColRPT];
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  if (rok) {
#pragma unroll
    for (int j = 0; j < kColRPT; ++j) v[j] = ld_nt16(xs + xo + (uint32_t)j * row_b);
#pragma unroll
    for (int j = 0; j < kColRPT; ++j) {
      m[0] = fmaxf(m[0], fabsf(bf16_lo(v[j].x)));
      m[1] = fmaxf(m[1], fabsf(bf16_hi(v[j].x)));
      m[2] = fmaxf(m[2], fabsf(bf16_lo(v[j].y)));
      m[3] = fmaxf(m[3], fabsf(bf16_hi(v[j].y)));
      m[4] = fmaxf(m[4], fabsf(bf16_lo(v[j].z)));
      m[5] = fmaxf(m[5], fabsf(bf16_hi(v[j].z)));
      m[6] = fmaxf(m[6], fabsf(bf16_lo(v[j].w)));
      m[7] = fmaxf(m[7], fabsf(bf16_hi(v[j].w)));
    }
  }
  // reduce over the row groups of the wave (lanes with equal lc)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int d = LPR; d < 64; d <<= 1) m[i] = fmaxf(m[i], __shfl_xor(m[i], d, 64));
  }
  if (lane < LPR) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
  }
  __syncthreads();
  if (tid < CW) {
    float cm = red[0][tid];
    for (int w = 1; w < nwaves; ++w) cm = fmaxf(cm, red[w][tid]);
    const int64_t c = strip * CW + tid;
    float s, iv;
    scale_from_amax(cm, fmax, eps, s, iv);
    s_scale[tid] = s;
    if (c < C) {
      scale[b * C + c] = s;
      if (inv) inv[b * C + c] = iv;
    }
  }
  __syncthreads();
  if (!rok) return;

  const float fm = (float)fmax;
  uint8_t* qs = qT + (b * C + strip * CW) * R;
  const uint32_t R32 = (uint32_t)R;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sc = s_scale[lc * 8 + i];
    float f[kColRPT];
#pragma unroll
    for (int j = 0; j < kColRPT; ++j) {
      const uint32_t w = (i < 2) ? v[j].x : (i < 4) ? v[j].y : (i < 6) ? v[j].z : v[j].w;
      f[j] = clampf(((i & 1) ? bf16_hi(w) : bf16_lo(w)) * sc, fm);
    }
    uint4 o;
    o.x = cvt4<E5>(f[0], f[1], f[2], f[3]);
    o.y = cvt4<E5>(f[4], f[5], f[6], f[7]);
    o.z = cvt4<E5>(f[8], f[9], f[10], f[11]);
    o.w = cvt4<E5>(f[12], f[13], f[14], f[15]);
    store_col16<PK>(qs, (uint32_t)(lc * 8 + i), (uint32_t)r0, R32, o);
  }
}

// Any shape: one workgroup per column, two passes (correct, slow).
template <bool E5>
__global__ __launch_bounds__(256) void k_quant_col_generic(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ qT, float* __restrict__ scale,
                                                           float* __restrict__ inv, double fmax, double eps) {
  __shared__ float red[4];
  const int64_t bc = blockIdx.x;
  const int64_t b = bc / C, c = bc % C;
  const uint16_t* xb = x + b * R * C + c;
  float m = 0.0f;
  for (int64_t r = threadIdx.x; r < R; r += 256) m = fmaxf(m, fabsf(__uint_as_float((uint32_t)xb[r * C] << 16)));
  m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (threadIdx.x == 0) {
    scale[bc] = s;
    if (inv) inv[bc] = iv;
  }
  const float fm = (float)fmax;
  for (int64_t r = threadIdx.x; r < R; r += 256)
    qT[bc * R + r] = cvt1<E5>(clampf(__uint_as_float((uint32_t)xb[r * C] << 16) * s, fm));
}

// ---------------------------------------------------------------------------
// Tensorwise: clear, amax with relaxed atomics, cast. The kernel boundary
// between the amax and the cast launches is the one ordering point.
__global__ void k_clear_words(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// max |x| over the 16-byte vectors [0, nvec) of x, for workgroup `blk` of
// `nblk` (256 threads each): kAmaxU loads in flight per thread, in chunks of
// kAmaxU * 256 vectors dealt round robin to the workgroups.
constexpr int kAmaxU = 8;
__device__ __forceinline__ float amax_vec_range(const uint16_t* __restrict__ x, int64_t nvec, int64_t blk,
                                                int64_t nblk) {
  float m = 0.0f;
  const int64_t stride = nblk * 256 * kAmaxU;
  int64_t i = blk * 256 * kAmaxU + threadIdx.x;
  for (; i + (kAmaxU - 1) * 256 < nvec; i += stride) {
    uint4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) v[u] = ld_nt16(x + 8 * (i + u * 256));
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) m = amax8(v[u], m);
  }
  // the partial chunk (later chunks of this thread start past nvec)
#pragma unroll
  for (int u = 0; u < kAmaxU; ++u)
    if (i + u * 256 < nvec) m = amax8(ld_nt16(x + 8 * (i + u * 256)), m);
  return m;
}

// workgroups for amax_vec_range over nvec vectors: one chunk each, at most 2048
static int64_t amax_blocks(int64_t nvec) {
  int64_t b = (nvec + 256 * kAmaxU - 1) / (256 * kAmaxU);
  return b < 1 ? 1 : (b > 2048 ? 2048 : b);
}

__global__ __launch_bounds__(256) void k_amax_tensor(const uint16_t* __restrict__ x, int64_t n,
                                                     uint32_t* __restrict__ amax_word) {
  __shared__ float red[4];
  const int64_t nvec = n / 8;
  float m = amax_vec_range(x, nvec, blockIdx.x, gridDim.x);
  // tail (n % 8 elements)
  if (blockIdx.x == 0)
    for (int64_t i = nvec * 8 + threadIdx.x; i < n; i += 256)
      m = fmaxf(m, fabsf(__uint_as_float((uint32_t)x[i] << 16)));
  m = block_max<256>(m, red);
  if (threadIdx.x == 0) atomic_max_relaxed(amax_word, m);
}

template <bool E5, bool NZ = false>
__global__ __launch_bounds__(256) void k_cast_tensor(const uint16_t* __restrict__ x, int64_t n,
                                                     const uint32_t* __restrict__ amax_word,
                                                     uint8_t* __restrict__ q, float* __restrict__ scale,
                                                     float* __restrict__ inv, double fmax, double eps) {
  const float amax = __uint_as_float(*amax_word);
  float s, iv;
  scale_from_amax(amax, fmax, eps, s, iv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scale[0] = s;
    if (inv) inv[0] = iv;
  }
  const float fm = (float)fmax;
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
    const uint4 v = ld_nt16(x + 8 * i);
    st_nt8(q + 8 * i, quant8<E5, NZ>(v, s, fm));
  }
  if (blockIdx.x == 0)
    for (int64_t i = nvec * 8 + threadIdx.x; i < n; i += 256)
      q[i] = cvt1x<E5, NZ>(clampf(__uint_as_float((uint32_t)x[i] << 16) * s, fm));
}

// ---------------------------------------------------------------------------
// 1 x G groups along the row, G in {128, 32}: G/8 lanes per group, one
// 16-byte chunk each; each lane set handles U groups per iteration so that
// U loads are in flight before the reductions (U = 4 for tensors small
// enough that the grid does not fill the chip several times over, else 1).
// MX=true: power-of-two scale, E8M0 byte per group.
template <bool E5, int G, bool MX, int U>
__global__ __launch_bounds__(256) void k_quant_group1d(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scale,
                                                       float* __restrict__ inv, uint8_t* __restrict__ e8m0,
                                                       double fmax, double eps, int mx_mode) {
  constexpr int LPG = G / 8;      // lanes per group
  constexpr int GPB = 256 / LPG;  // groups per workgroup per unrolled slot
  const int64_t ngc = (cols + G - 1) / G;
  const int64_t ngroups = rows * ngc;
  const bool flat = cols % G == 0;  // groups tile the flattened tensor exactly
  const int sub = threadIdx.x % LPG;
  const float fm = (float)fmax;
  const int64_t step = (int64_t)gridDim.x * GPB * U;
  for (int64_t g0 = (int64_t)blockIdx.x * GPB * U + threadIdx.x / LPG; g0 < ngroups; g0 += step) {
    uint4 v[U];
    int64_t off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + (int64_t)u * GPB;
      if (flat) {
        off[u] = g * G + sub * 8;
        ok[u] = g < ngroups;
      } else {
        const int64_t r = g / ngc, gc = g % ngc;
        const int64_t c = gc * G + sub * 8;
        off[u] = r * cols + c;
        ok[u] = g < ngroups && c < cols;
      }
      v[u] = ok[u] ? ld_nt16(x + off[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + (int64_t)u * GPB;
      float m = amax8(v[u], 0.0f);
#pragma unroll
      for (int o = 1; o < LPG; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float sc, iv;
      if constexpr (MX) {
        const int k = mx_exponent(m, fmax, eps, mx_mode);
        sc = exp2i(k);
        if (sub == 0 && g < ngroups) e8m0[g] = (uint8_t)(127 - k);
      } else {
        scale_from_amax(m, fmax, eps, sc, iv);
        if (sub == 0 && g < ngroups) {
          scale[g] = sc;
          if (inv) inv[g] = iv;
        }
      }
      if (ok[u]) st_nt8(q + off[u], quant8<E5>(v[u], sc, fm));
    }
  }
}

// 128 x 128 blocks: one workgroup of NB * 256 threads per NB neighbouring
// blocks of a 128-row band. 16 NB lanes cover NB * 256 contiguous bytes of a
// row (a thread: 8 columns of rows ro + 16 j, j < 8). On the 16 x 8192 x 5120
// MoE weights two blocks per workgroup (512-byte row pieces) measured 6% faster
// than one; four (1024 threads) leave one workgroup per CU and were slower.
template <bool E5, int NB>
__global__ __launch_bounds__(NB * 256) void k_quant_block128(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                             int64_t nbr, int64_t nbc, uint8_t* __restrict__ q,
                                                             float* __restrict__ scale, float* __restrict__ inv,
                                                             double fmax, double eps) {
  constexpr int LPR = NB * 16;  // lanes per row
  constexpr int NW = NB * 4;    // waves
  __shared__ float red[NW][NB];
  const int64_t ngrp = nbc / NB;
  int64_t blk = blockIdx.x;
  const int64_t cg = blk % ngrp;
  blk /= ngrp;
  const int64_t rb = blk % nbr;
  const int64_t b = blk / nbr;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % LPR, ro = tid / LPR;
  const int sub = cc >> 4;  // block of the group
  const int64_t c = cg * NB * 128 + cc * 8;
  const bool cok = c < C;
  const uint16_t* xb = x + b * R * C;
  uint4 v[8];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = rb * 128 + ro + 16 * j;
    if (cok && r < R) {
      v[j] = ld_nt16(xb + r * C + c);
      m = amax8(v[j], m);
    }
  }
  // the 16 lanes of one block in one row, then the rows a wave holds
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane < LPR && (lane & 15) == 0) red[wave][lane >> 4] = m;
  __syncthreads();
  m = red[0][sub];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, red[w][sub]);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  const int64_t si = (b * nbr + rb) * nbc + cg * NB + sub;
  if (ro == 0 && (cc & 15) == 0) {
    scale[si] = s;
    if (inv) inv[si] = iv;
  }
  const float fm = (float)fmax;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = rb * 128 + ro + 16 * j;
    if (cok && r < R)
      st_nt8(q + b * R * C + r * C + c, quant8<E5>(v[j], s, fm));
  }
}

// Generic block / MX (any alignment): one workgroup per group, two passes.
template <bool E5, bool MX>
__global__ __launch_bounds__(256) void k_quant_block_generic(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                             int64_t br, int64_t bc, int64_t nbr, int64_t nbc,
                                                             uint8_t* __restrict__ q, float* __restrict__ scale,
                                                             float* __restrict__ inv, uint8_t* __restrict__ e8m0,
                                                             double fmax, double eps, int mx_mode) {
  __shared__ float red[4];
  int64_t blk = blockIdx.x;
  const int64_t cbk = blk % nbc;
  blk /= nbc;
  const int64_t rbk = blk % nbr;
  const int64_t b = blk / nbr;
  const int64_t r0 = rbk * br, c0 = cbk * bc;
  const int64_t nr = R - r0 < br ? R - r0 : br;
  const int64_t nc = C - c0 < bc ? C - c0 : bc;
  const uint16_t* xb = x + b * R * C;
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < nr * nc; i += 256)
    m = fmaxf(m, fabsf(__uint_as_float((uint32_t)xb[(r0 + i / nc) * C + c0 + i % nc] << 16)));
  m = block_max<256>(m, red);
  float s, iv;
  if constexpr (MX) {
    const int k = mx_exponent(m, fmax, eps, mx_mode);
    s = exp2i(k);
    if (threadIdx.x == 0) e8m0[blockIdx.x] = (uint8_t)(127 - k);
  } else {
    scale_from_amax(m, fmax, eps, s, iv);
    if (threadIdx.x == 0) {
      scale[blockIdx.x] = s;
      if (inv) inv[blockIdx.x] = iv;
    }
  }
  const float fm = (float)fmax;
  for (int64_t i = threadIdx.x; i < nr * nc; i += 256) {
    const int64_t off = b * R * C + (r0 + i / nc) * C + c0 + i % nc;
    q[off] = cvt1<E5>(clampf(__uint_as_float((uint32_t)x[off] << 16) * s, fm));
  }
}

// ---------------------------------------------------------------------------
// Launchers.

static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <bool E5>
static hipError_t launch_row_t(const QuantArgs& a) {
  const int64_t R = a.batch * a.rows;
  if (R == 0 || a.cols == 0) return hipSuccess;
  const bool vec = a.cols % 8 == 0 && aligned16(a.x) && aligned16(a.q);
  dim3 grid((unsigned)R), block(256);
  if (a.fnuz) {
    hipLaunchKernelGGL((k_quant_row_generic<E5, true>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv,
                       a.fmax, a.eps);
    return hipGetLastError();
  }
  // rows up to 4096 elements: one wavefront per row; longer rows: one
  // workgroup per row (measured faster on MI355X for 7168 and 14336)
  if (vec && a.cols <= 512 * 8) {
    const int64_t J = (a.cols + 511) / 512;
    dim3 g4((unsigned)((R + 3) / 4));
    if (J <= 2)
      hipLaunchKernelGGL((k_quant_row_wave<2, E5>), g4, block, 0, a.stream, a.x, R, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
    else if (J <= 4)
      hipLaunchKernelGGL((k_quant_row_wave<4, E5>), g4, block, 0, a.stream, a.x, R, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
    else
      hipLaunchKernelGGL((k_quant_row_wave<8, E5>), g4, block, 0, a.stream, a.x, R, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
  } else if (vec && a.cols <= 2048 * 8) {
    const int64_t J = (a.cols + 2047) / 2048;
    if (J <= 1)
      hipLaunchKernelGGL((k_quant_row<1, E5>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
    else if (J <= 2)
      hipLaunchKernelGGL((k_quant_row<2, E5>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
    else if (J <= 4)
      hipLaunchKernelGGL((k_quant_row<4, E5>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
    else
      hipLaunchKernelGGL((k_quant_row<8, E5>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
  } else {
    hipLaunchKernelGGL((k_quant_row_generic<E5>), grid, block, 0, a.stream, a.x, a.cols, a.q, a.scale, a.inv, a.fmax, a.eps);
  }
  return hipGetLastError();
}

hipError_t launch_quant_row(const QuantArgs& a) { return a.e5 ? launch_row_t<true>(a) : launch_row_t<false>(a); }

// rows % G == 0 and cols % 64 == 0 (the caller checks), cols <= 16384
template <bool E5, int G>
static hipError_t launch_row_kpacked_t(const QuantArgs& a) {
  const int64_t R = a.batch * a.rows, C = a.cols;
  if (R == 0 || C == 0) return hipSuccess;
  dim3 grid((unsigned)R), block(256);
  // pair-interleaved rows up to 4096 elements: one wavefront per row, as the
  // row-major form (2048-column rows: 129 us against 156 us for a workgroup
  // per row, on the DeepSeek-V3-shaped MoE layer's grad_out, see the bench)
  if (G == 2 && C <= 512 * 8 && aligned16(a.x) && aligned16(a.q)) {
    const int64_t J = (C + 511) / 512;
    dim3 g4((unsigned)((R + 3) / 4));
    if (J <= 2)
      hipLaunchKernelGGL((k_quant_row_wave<2, E5, true>), g4, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                         a.eps);
    else if (J <= 4)
      hipLaunchKernelGGL((k_quant_row_wave<4, E5, true>), g4, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                         a.eps);
    else
      hipLaunchKernelGGL((k_quant_row_wave<8, E5, true>), g4, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                         a.eps);
    return hipGetLastError();
  }
  const int64_t J = (C + 2047) / 2048;
  if (J <= 1)
    hipLaunchKernelGGL((k_quant_row_kpacked<1, E5, G>), grid, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                       a.eps);
  else if (J <= 2)
    hipLaunchKernelGGL((k_quant_row_kpacked<2, E5, G>), grid, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                       a.eps);
  else if (J <= 4)
    hipLaunchKernelGGL((k_quant_row_kpacked<4, E5, G>), grid, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                       a.eps);
  else
    hipLaunchKernelGGL((k_quant_row_kpacked<8, E5, G>), grid, block, 0, a.stream, a.x, R, C, a.q, a.scale, a.inv, a.fmax,
                       a.eps);
  return hipGetLastError();
}

hipError_t launch_quant_row_kpacked(const QuantArgs& a, int group_rows) {
  if (group_rows == 2) return a.e5 ? launch_row_kpacked_t<true, 2>(a) : launch_row_kpacked_t<false, 2>(a);
  return a.e5 ? launch_row_kpacked_t<true, 16>(a) : launch_row_kpacked_t<false, 16>(a);
}

// The fused form (one workgroup per 64-column strip over all rows) when it
// gives enough workgroups to fill the chip, else the split form over row
// chunks of kColChunk rows, which needs one amax word per column.
static bool col_split(int64_t batch, int64_t rows, int64_t cols) {
  const int64_t strips = (cols + 63) / 64;
  return rows > 2048 && batch * strips < 1024;
}

size_t quant_col_ws_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (!col_split(batch, rows, cols)) return 0;
  return (size_t)(batch * cols) * sizeof(uint32_t);
}

template <bool E5, bool PK>
static hipError_t launch_col_t(const QuantArgs& a, uint32_t* colmax) {
  const int64_t B = a.batch, R = a.rows, C = a.cols;
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  // 32-bit in-slice offsets: one batch slice of x (2 B/elem) below 2^31 bytes
  const bool vec = C % 8 == 0 && R % 16 == 0 && aligned16(a.x) && aligned16(a.q) && R * C < ((int64_t)1 << 30);
  if (!vec) {
    hipLaunchKernelGGL((k_quant_col_generic<E5>), dim3((unsigned)(B * C)), dim3(256), 0, a.stream, a.x, R, C, a.q,
                       a.scale, a.inv, a.fmax, a.eps);
    return hipGetLastError();
  }
  if (R <= 2048) {
    const int64_t stripsw = (C + kColCW - 1) / kColCW;
    // kColCW / 8 threads per 16-row group, whole waves
    int64_t threads = (R / kColRPT) * (kColCW / 8);
    threads = (threads + 63) / 64 * 64;
    hipLaunchKernelGGL((k_quant_col_reg<E5, kColCW, PK>), dim3((unsigned)(B * stripsw)), dim3((unsigned)threads), 0,
                       a.stream, a.x, R, C, stripsw, a.q, a.scale, a.inv, a.fmax, a.eps);
    return hipGetLastError();
  }
  const int64_t strips = (C + 63) / 64;
  if (!col_split(B, R, C)) {
    hipLaunchKernelGGL((k_quant_col<E5, 0, PK>), dim3((unsigned)(B * strips)), dim3(256), 0, a.stream, a.x, R, C,
                       strips, (int64_t)1, R, a.q, a.scale, a.inv, (uint32_t*)nullptr, (int64_t)1, a.fmax, a.eps);
    return hipGetLastError();
  }
  const int64_t rchunks = (R + kColChunk - 1) / kColChunk;
  const int64_t nwords = B * C;
  hipLaunchKernelGGL(k_clear_words, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, a.stream, colmax, nwords);
  hipLaunchKernelGGL((k_quant_col<E5, 2>), dim3((unsigned)(B * strips * rchunks)), dim3(256), 0, a.stream, a.x, R, C,
                     strips, rchunks, (int64_t)kColChunk, a.q, a.scale, a.inv, colmax, (int64_t)1, a.fmax, a.eps);
  hipLaunchKernelGGL((k_quant_col<E5, 1, PK>), dim3((unsigned)(B * strips * rchunks)), dim3(256), 0, a.stream, a.x, R, C,
                     strips, rchunks, (int64_t)kColChunk, a.q, a.scale, a.inv, colmax, (int64_t)1, a.fmax, a.eps);
  return hipGetLastError();
}

// One scale for the whole tensor, written in the transposed layout
// qT[b][c][r] (the column-major operand of a tensorwise backward GEMM).
template <bool E5>
static hipError_t launch_tensor_t_t(const QuantArgs& a, uint32_t* amax_word) {
  const int64_t B = a.batch, R = a.rows, C = a.cols;
  const int64_t n = B * R * C;
  if (n == 0) return hipSuccess;
  const int64_t nvec = n / 8;
  const int64_t strips = (C + 63) / 64;
  const int64_t rchunks = (R + kColChunk - 1) / kColChunk;
  hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(64), 0, a.stream, amax_word, (int64_t)1);
  hipLaunchKernelGGL(k_amax_tensor, dim3((unsigned)amax_blocks(nvec)), dim3(256), 0, a.stream, a.x, n, amax_word);
  hipLaunchKernelGGL((k_quant_col<E5, 1>), dim3((unsigned)(B * strips * rchunks)), dim3(256), 0, a.stream, a.x, R, C,
                     strips, rchunks, (int64_t)kColChunk, a.q, a.scale, a.inv, amax_word, (int64_t)0, a.fmax,
                     a.eps);
  return hipGetLastError();
}

hipError_t launch_quant_tensor_transposed(const QuantArgs& a, void* ws) {
  // the cast pass's 32-bit in-slice offsets
  if (a.cols % 8 != 0 || a.rows % 16 != 0 || a.rows * a.cols >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
  return a.e5 ? launch_tensor_t_t<true>(a, (uint32_t*)ws) : launch_tensor_t_t<false>(a, (uint32_t*)ws);
}

hipError_t launch_quant_col(const QuantArgs& a, void* ws) {
  return a.e5 ? launch_col_t<true, false>(a, (uint32_t*)ws) : launch_col_t<false, false>(a, (uint32_t*)ws);
}

hipError_t launch_quant_col_kpacked(const QuantArgs& a, void* ws) {
  return a.e5 ? launch_col_t<true, true>(a, (uint32_t*)ws) : launch_col_t<false, true>(a, (uint32_t*)ws);
}

template <bool E5>
static hipError_t launch_tensor_t(const QuantArgs& a, uint32_t* amax_word) {
  const int64_t n = a.batch * a.rows * a.cols;
  if (n == 0) return hipSuccess;
  const int64_t nvec = n / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(64), 0, a.stream, amax_word, (int64_t)1);
  hipLaunchKernelGGL(k_amax_tensor, dim3((unsigned)amax_blocks(nvec)), dim3(256), 0, a.stream, a.x, n, amax_word);
  if (a.fnuz)
    hipLaunchKernelGGL((k_cast_tensor<E5, true>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x, n,
                       (const uint32_t*)amax_word, a.q, a.scale, a.inv, a.fmax, a.eps);
  else
  hipLaunchKernelGGL((k_cast_tensor<E5>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x, n,
                     (const uint32_t*)amax_word, a.q, a.scale, a.inv, a.fmax, a.eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tensorwise quantization of up to three tensors in two launches, for the
// all-FP8 backward of one Linear layer ("FP8 Training: Quantization,
// Autograd, Torchao", section 4: grad_weight = grad_output^T @ input needs
// grad_output transposed in row-major form and the input column-major; "FP8
// training on AMD GPUs with TorchTitan and TorchAO", Figure 4 caption: a
// companion kernel quantizes grad_output and the activation together).
//  - k_amax_multi: the amax of every tensor (one atomic word each);
//  - k_cast_multi_t: every tensor's transposed output qT [C][R] and, where
//    asked, its row-major output q [R][C] from the same registers, so
//    grad_output is read once for both layouts. Blocks are dealt to tensors by
//    ranges of blockIdx.x; a block casts 64 columns x up to kDualChunk rows
//    with the 16 x 8 register transpose of the column kernel above.
struct TJob {
  const uint16_t* x;  // [R][C], R % 16 == 0, C % 8 == 0, R * C < 2^30
  int64_t R, C;
  uint8_t* q;         // [R][C] or nullptr
  uint8_t* qT;        // [C][R]
  float* scale;
  float* inv;         // or nullptr
  uint32_t* amax;     // one word, cleared before k_amax_multi
  double fmax;
  int e5;
  int64_t amax_blk0, amax_blks;  // this tensor's blocks of k_amax_multi
  int64_t cast_blk0, rchunks;    // and of k_cast_multi_t (strips x rchunks)
};
struct TJobs {
  TJob j[kMaxTJobs];
  int n;
  double eps;
};

__device__ __forceinline__ int tjob_of(const TJobs& js, int64_t blk, bool cast) {
  int k = 0;
#pragma unroll
  for (int i = 1; i < kMaxTJobs; ++i)
    if (i < js.n && blk >= (cast ? js.j[i].cast_blk0 : js.j[i].amax_blk0)) k = i;
  return k;
}

__global__ __launch_bounds__(256) void k_amax_multi(const TJobs js) {
  __shared__ float red[4];
  const int k = tjob_of(js, blockIdx.x, false);
  const TJob& J = js.j[k];
  float m = amax_vec_range(J.x, J.R * J.C / 8, blockIdx.x - J.amax_blk0, J.amax_blks);
  m = block_max<256>(m, red);
  if (threadIdx.x == 0) atomic_max_relaxed(J.amax, m);
}

template <bool E5>
__device__ __forceinline__ void cast_strip_t(const TJob& J, int64_t strip, int64_t rc, float s) {
  const int tid = threadIdx.x;
  const int l8 = tid & 7, rg = tid >> 3;
  const int64_t R = J.R, C = J.C;
  if (strip * 64 + l8 * 8 >= C) return;
  const float fm = (float)J.fmax;
  const int64_t r_beg = rc * kDualChunk;
  const int64_t r_end = r_beg + kDualChunk < R ? r_beg + kDualChunk : R;
  // uniform bases plus 32-bit per-lane offsets (R * C < 2^30)
  const uint8_t* xs = reinterpret_cast<const uint8_t*>(J.x + strip * 64);
  uint8_t* qs = J.qT + strip * 64 * R;
  uint8_t* qr = J.q ? J.q + strip * 64 + l8 * 8 : nullptr;
  const uint32_t row_b = (uint32_t)(C * 2);
  const uint32_t R32 = (uint32_t)R, C32 = (uint32_t)C;
  const int64_t ngroups = (r_end - r_beg) / kColRPT;
  for (int64_t g = rg; g < ngroups; g += 32) {
    const uint32_t r0 = (uint32_t)(r_beg + g * kColRPT);
    const uint32_t xo = r0 * row_b + (uint32_t)(l8 * 16);
    // pk[i][d]: column i, rows r0 + 4d .. r0 + 4d + 3 as four fp8 bytes
    uint32_t pk[8][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ld_nt16(xs + xo + (uint32_t)(8 * h + j) * row_b);
      float f[8][8];  // [column i][row j]
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = (i < 2) ? v[j].x : (i < 4) ? v[j].y : (i < 6) ? v[j].z : v[j].w;
          f[i][j] = clampf(((i & 1) ? bf16_hi(w) : bf16_lo(w)) * s, fm);
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk[i][2 * h] = cvt4<E5>(f[i][0], f[i][1], f[i][2], f[i][3]);
        pk[i][2 * h + 1] = cvt4<E5>(f[i][4], f[i][5], f[i][6], f[i][7]);
      }
      if (qr) {
        // row-major: 8 columns of each of the 8 rows, the same conversions;
        // plain stores (a strip writes half of each 128-byte line, the
        // neighbouring strip the other half: L2 merges them)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint2*>(qr + (r0 + (uint32_t)(8 * h + j)) * C32) =
              make_uint2(cvt4<E5>(f[0][j], f[1][j], f[2][j], f[3][j]), cvt4<E5>(f[4][j], f[5][j], f[6][j], f[7][j]));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st_nt16(qs + (uint32_t)(l8 * 8 + i) * R32 + r0, make_uint4(pk[i][0], pk[i][1], pk[i][2], pk[i][3]));
  }
}

__global__ __launch_bounds__(256) void k_cast_multi_t(const TJobs js) {
  const int k = tjob_of(js, blockIdx.x, true);
  const TJob& J = js.j[k];
  const int64_t lb = blockIdx.x - J.cast_blk0;
  const int64_t rc = lb % J.rchunks, strip = lb / J.rchunks;
  float s, iv;
  scale_from_amax(__uint_as_float(*J.amax), J.fmax, js.eps, s, iv);
  if (lb == 0 && threadIdx.x == 0) {
    J.scale[0] = s;
    if (J.inv) J.inv[0] = iv;
  }
  if (J.e5)
    cast_strip_t<true>(J, strip, rc, s);
  else
    cast_strip_t<false>(J, strip, rc, s);
}

hipError_t launch_quant_tensor_multi_t(const TJobSpec* specs, int n, double eps, uint32_t* amax_words,
                                       hipStream_t stream) {
  if (n < 1 || n > kMaxTJobs) return hipErrorInvalidValue;
  TJobs js{};
  js.n = n;
  js.eps = eps;
  int64_t ab = 0, cb = 0;
  for (int i = 0; i < n; ++i) {
    const TJobSpec& t = specs[i];
    if (t.rows % 16 != 0 || t.cols % 8 != 0 || t.rows * t.cols >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
    TJob& J = js.j[i];
    J.x = t.x;
    J.R = t.rows;
    J.C = t.cols;
    J.q = t.q;
    J.qT = t.qT;
    J.scale = t.scale;
    J.inv = t.inv;
    J.amax = amax_words + i;
    J.fmax = t.fmax;
    J.e5 = t.e5 ? 1 : 0;
    const int64_t nvec = t.rows * t.cols / 8;
    // blocks in proportion to the tensor (about 4 chunks each), so that
    // tensors of different sizes finish together
    const int64_t blocks = (nvec + 4 * 256 * kAmaxU - 1) / (4 * 256 * kAmaxU);
    J.amax_blk0 = ab;
    J.amax_blks = blocks;
    ab += blocks;
    J.rchunks = (t.rows + kDualChunk - 1) / kDualChunk;
    if (J.rchunks < 1) J.rchunks = 1;
    J.cast_blk0 = cb;
    cb += J.rchunks * ((t.cols + 63) / 64);
  }
  hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(64), 0, stream, amax_words, (int64_t)n);
  hipLaunchKernelGGL(k_amax_multi, dim3((unsigned)ab), dim3(256), 0, stream, js);
  hipLaunchKernelGGL(k_cast_multi_t, dim3((unsigned)cb), dim3(256), 0, stream, js);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tensorwise quantization of two tensors in two launches with no cleared word
// (the Linear forward's x and w: "FP8 Training: Quantization, Autograd,
// Torchao", section 4, one scale per tensor from its amax; Figure 4 of "FP8
// training on AMD GPUs with TorchTitan and TorchAO" names the same pairing of
// two tensors in one kernel):
//  - k_amax_pair: the maximum of each workgroup's range into partials[block];
//  - k_cast_pair: each workgroup takes the maximum over its tensor's partials
//    (maxima of non-NaN magnitudes: the same value in any order, so the scale
//    is bit for bit the one of the single-tensor path), the tensor's first
//    workgroup writes scale and inverse, and every workgroup casts its share.
// For small layers the launch gaps dominate: this is two launches where the
// single-tensor path takes three per tensor.
struct PJob {
  const uint16_t* x;  // n elements, n % 8 == 0
  int64_t n;
  uint8_t* q;
  float* scale;
  float* inv;         // or nullptr
  int64_t amax_blk0, amax_blks, cast_blk0, cast_blks;
};
struct PJobs {
  PJob j[2];
  float* part;        // amax_blks of job 0, then of job 1
  double fmax, eps;
};

__global__ __launch_bounds__(256) void k_amax_pair(const PJobs js) {
  __shared__ float red[4];
  const PJob& J = js.j[blockIdx.x >= js.j[1].amax_blk0 ? 1 : 0];
  float m = amax_vec_range(J.x, J.n / 8, blockIdx.x - J.amax_blk0, J.amax_blks);
  m = block_max<256>(m, red);
  if (threadIdx.x == 0) js.part[blockIdx.x] = m;
}

template <bool E5>
__global__ __launch_bounds__(256) void k_cast_pair(const PJobs js) {
  __shared__ float red[4];
  const PJob& J = js.j[blockIdx.x >= js.j[1].cast_blk0 ? 1 : 0];
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < J.amax_blks; i += 256) m = fmaxf(m, js.part[J.amax_blk0 + i]);
  m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, js.fmax, js.eps, s, iv);
  const int64_t lb = blockIdx.x - J.cast_blk0;
  if (lb == 0 && threadIdx.x == 0) {
    J.scale[0] = s;
    if (J.inv) J.inv[0] = iv;
  }
  const float fm = (float)js.fmax;
  const int64_t nvec = J.n / 8;
  const int64_t stride = J.cast_blks * 256;
  for (int64_t i = lb * 256 + threadIdx.x; i < nvec; i += stride) st_nt8(J.q + 8 * i, quant8<E5>(ld_nt16(J.x + 8 * i), s, fm));
}

// partials: 2 * kPairMaxAmaxBlocks floats
hipError_t launch_quant_tensor_pair(const TPairSpec* specs, bool e5, double fmax, double eps, float* partials,
                                    hipStream_t stream) {
  PJobs js{};
  js.part = partials;
  js.fmax = fmax;
  js.eps = eps;
  int64_t ab = 0, cb = 0;
  for (int i = 0; i < 2; ++i) {
    const TPairSpec& t = specs[i];
    if (t.n <= 0 || t.n % 8 != 0) return hipErrorInvalidValue;
    PJob& J = js.j[i];
    J.x = t.x;
    J.n = t.n;
    J.q = t.q;
    J.scale = t.scale;
    J.inv = t.inv;
    const int64_t nvec = t.n / 8;
    J.amax_blk0 = ab;
    J.amax_blks = amax_blocks(nvec);  // at most kPairMaxAmaxBlocks
    ab += J.amax_blks;
    int64_t cblocks = (nvec + 255) / 256;
    if (cblocks > 4096) cblocks = 4096;
    J.cast_blk0 = cb;
    J.cast_blks = cblocks;
    cb += cblocks;
  }
  hipLaunchKernelGGL(k_amax_pair, dim3((unsigned)ab), dim3(256), 0, stream, js);
  if (e5)
    hipLaunchKernelGGL(k_cast_pair<true>, dim3((unsigned)cb), dim3(256), 0, stream, js);
  else
    hipLaunchKernelGGL(k_cast_pair<false>, dim3((unsigned)cb), dim3(256), 0, stream, js);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Normalization fused with the rowwise quantization of its output ("FP8
// Training: Quantization, Autograd, Torchao", section 8: the norm's output
// write and the next layer's amax pass become one memory pass). One
// 256-thread workgroup per row; the row stays in registers from the load to
// the FP8 store, so x is read once and y (bf16) is written only if asked.
//  1. s1 = sum x, s2 = sum x^2: the exact sums rounded once to fp64. Only
//     mean32 and rstd32 (step 2) reach the output, so the kernel sums the row
//     in fp64 (s2 with fused multiply-adds: x * x is exact) and bounds the
//     error: no term passes more than 72 additions (64 in a lane, 6 shuffle
//     levels, 2 across waves), so |error| <= 72 * 2^-53 * sum|terms|, below
//     2^-46 s2 for s2 and 2^-45 sqrt(n s2) for s1 (sum|x| <= sqrt(n s2)).
//     (LayerNorm: 0 when s1 is proven exact, below). Step 2 is monotone in
//     s2 (and in s1, in mean^2), so running it at both ends of those
//     intervals brackets the exact result: when both ends give the same
//     mean32 and rstd32, so does the exact sum. A row where they differ (a
//     rounding boundary inside the interval, about 2^-20 of random rows, or
//     sums that cancel) is summed again exactly: integer terms
//     M 2^(q + 133) and M^2 2^(2 q + 266) of x = +-M 2^q added with LDS atomics
//     into limbs of 32 bits held in 64-bit words, then rounded once to fp64;
//  2. mean, mean square, var (LayerNorm) and rstd = 1 / sqrt(var + norm_eps):
//     fp64 IEEE operations (no contraction: this file is built with
//     -ffp-contract=off, because hip's __fmul_rn / __fadd_rn are plain
//     operators that the compiler would otherwise fuse, and a fused
//     t * gamma + beta rounds once where the definition rounds twice);
//  3. y = ((x - mean32) * rstd32) * gamma + beta (LayerNorm) or
//     (x * rstd32) * gamma (RMSNorm), fp32 IEEE operations, stored as bf16
//     (RNE);
//  4. amax of the bf16 row, scale, clamp and cast as in k_quant_row.
constexpr int kS1Limbs = 10;  // sum x in units of 2^-133: below 2^275 for 2^14 terms
constexpr int kS2Limbs = 18;  // sum x^2 in units of 2^-266: below 2^536

// Exact row sums (the slow path of step 1): limbs L[0..n) hold 32-bit digits
// in 64-bit words; called by one lane after all the atomics landed. Carries
// go up (arithmetic shifts keep the sign in the top word), a negative total
// is negated, and the magnitude is rounded to the nearest fp64, ties to even.
__device__ __noinline__ double limbs_to_double(long long* L, int n, int unit_exp) {
  for (int i = 0; i < n - 1; ++i) {
    const long long c = L[i] >> 32;
    L[i] -= c * 4294967296LL;
    L[i + 1] += c;
  }
  const bool neg = L[n - 1] < 0;
  if (neg) {
    for (int i = 0; i < n; ++i) L[i] = -L[i];
    for (int i = 0; i < n - 1; ++i) {
      const long long c = L[i] >> 32;
      L[i] -= c * 4294967296LL;
      L[i + 1] += c;
    }
  }
  int h = n - 1;
  while (h >= 0 && L[h] == 0) --h;
  if (h < 0) return 0.0;
  const uint32_t top = (uint32_t)L[h];
  const int lead = 32 * h + 31 - __clz(top);
  // bits [32 (h - 1), 32 h + 32) of the magnitude, and the next digit below
  const uint64_t hi = ((uint64_t)top << 32) | (h >= 1 ? (uint64_t)(uint32_t)L[h - 1] : 0);
  const uint32_t lo = h >= 2 ? (uint32_t)L[h - 2] : 0u;
  const int sh = 63 - (lead - 32 * (h - 1));  // brings the leading one to bit 63
  const uint64_t w = sh ? (hi << sh) | ((uint64_t)lo >> (32 - sh)) : hi;
  bool sticky = (w & 0x3ffu) != 0 || (sh ? (uint32_t)(lo << sh) != 0u : lo != 0u);
  for (int i = h - 3; i >= 0 && !sticky; --i) sticky = L[i] != 0;
  uint64_t sig = w >> 11;
  const bool round = (w >> 10) & 1u;
  int e = lead - 52 + unit_exp;
  if (round && (sticky || (sig & 1u))) {
    sig += 1;
    if (sig == (1ull << 53)) {
      sig >>= 1;
      e += 1;
    }
  }
  const double v = ldexp((double)sig, e);
  return neg ? -v : v;
}

// Adds one bf16 value (and its square) as integers to the limbs.
template <bool LAYER>
__device__ __forceinline__ void exact_add(uint32_t b, long long* L1, long long* L2) {
  const uint32_t v = b & 0x7fffu;
  if (v == 0) return;
  const uint32_t E = v >> 7;
  const uint64_t M = E ? 128u + (v & 0x7fu) : (v & 0x7fu);
  const int sh = (E ? (int)E : 1) - 1;  // q + 133
  if constexpr (LAYER) {
    const uint64_t t = M << (sh & 31);
    const long long lo = (long long)(t & 0xffffffffu), hi = (long long)(t >> 32);
    const bool ng = (b & 0x8000u) != 0;
    atomicAdd(reinterpret_cast<unsigned long long*>(&L1[sh >> 5]), (unsigned long long)(ng ? -lo : lo));
    if (hi) atomicAdd(reinterpret_cast<unsigned long long*>(&L1[(sh >> 5) + 1]), (unsigned long long)(ng ? -hi : hi));
  }
  const int s2 = 2 * sh;
  const uint64_t t = (M * M) << (s2 & 31);
  atomicAdd(reinterpret_cast<unsigned long long*>(&L2[s2 >> 5]), (unsigned long long)(t & 0xffffffffu));
  if (t >> 32) atomicAdd(reinterpret_cast<unsigned long long*>(&L2[(s2 >> 5) + 1]), (unsigned long long)(t >> 32));
}

template <int TPR, int J, bool E5, bool LAYER>
__global__ __launch_bounds__(256) void k_norm_quant_row(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ beta, int64_t rows, int64_t cols,
                                                        double norm_eps, uint16_t* __restrict__ y,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale,
                                                        float* __restrict__ inv, double fmax, double eps) {
  // TPR threads per row: 64 (one wavefront per row, 4 rows per workgroup, no
  // barrier; LDS only in the exact-sum path) for rows up to 4096 elements,
  // else 256
  static_assert(TPR == 64 || TPR == 256, "threads per row");
  __shared__ double red_d[2][4];
  __shared__ uint32_t red_e[4];
  __shared__ float red[4];
  __shared__ long long s_limbs[TPR == 64 ? 4 : 1][kS1Limbs + kS2Limbs];
  __shared__ double s_exact[TPR == 64 ? 4 : 1][2];
  const int tid = threadIdx.x;
  const int t = TPR == 64 ? (tid & 63) : tid;
  const int slot = TPR == 64 ? (tid >> 6) : 0;
  const int64_t row = TPR == 64 ? (int64_t)blockIdx.x * 4 + (tid >> 6) : (int64_t)blockIdx.x;
  if (TPR == 64 && row >= rows) return;
  const uint16_t* xr = x + row * cols;
  uint4 v[J];
  double s1 = 0.0, s2 = 0.0;
  // LayerNorm: the smallest exponent field over the row's nonzero values (the
  // field of v - 1, never above the value's own) for the exactness test of s1
  uint32_t emin = 0x7f80u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = 8 * (t + TPR * j);
    v[j] = c < cols ? ld_nt16(xr + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double lo = bf16_lo(w[k]), hi = bf16_hi(w[k]);
      if constexpr (LAYER) s1 = __dadd_rn(__dadd_rn(s1, lo), hi);
      // x * x is exact in fp64, so the fused multiply-add rounds exactly as
      // s2 + x * x does, with one fp64 operation instead of two
      s2 = __fma_rn(hi, hi, __fma_rn(lo, lo, s2));
      if constexpr (LAYER) {
        const uint32_t a = w[k] & 0x7fffu, b = (w[k] >> 16) & 0x7fffu;
        emin = min(emin, min((a - 1u) & 0x7f80u, (b - 1u) & 0x7f80u));
      }
    }
  }
  // row sums (fp64): the wavefront, then (256 threads per row) the 4 waves
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    if constexpr (LAYER) {
      s1 = __dadd_rn(s1, __shfl_xor(s1, o, 64));
      emin = min(emin, (uint32_t)__shfl_xor((int)emin, o, 64));
    }
    s2 = __dadd_rn(s2, __shfl_xor(s2, o, 64));
  }
  if constexpr (TPR == 256) {
    if ((tid & 63) == 0) {
      red_d[0][tid >> 6] = s1;
      red_d[1][tid >> 6] = s2;
      red_e[tid >> 6] = emin;
    }
    __syncthreads();
    s1 = __dadd_rn(__dadd_rn(red_d[0][0], red_d[0][1]), __dadd_rn(red_d[0][2], red_d[0][3]));
    s2 = __dadd_rn(__dadd_rn(red_d[1][0], red_d[1][1]), __dadd_rn(red_d[1][2], red_d[1][3]));
    emin = min(min(red_e[0], red_e[1]), min(red_e[2], red_e[3]));
  }
  const double n = (double)cols;
  float mean32 = 0.0f, rstd32;
  // step 2 at the ends of the error intervals (row-uniform decision)
  bool settled;
  {
    const double e2 = __dmul_rn(s2, 0x1p-46);
    const double ms_lo = __ddiv_rn(__dsub_rn(s2, e2), n), ms_hi = __ddiv_rn(__dadd_rn(s2, e2), n);
    double v_lo = ms_lo, v_hi = ms_hi;
    if constexpr (LAYER) {
      // sum|x| <= sqrt(n s2); every term is a multiple of 2^qmin, qmin =
      // max(E, 1) - 134 over the nonzero values, so s1 is exact when that
      // bound stays below 2^(qmin + 53). The mean is then exact too whenever n
      // is a power of two, and often sits on an fp32 rounding midpoint, where
      // any interval around it would leave the rounding open
      const double bnd = __dmul_rn(__dsqrt_rn(__dmul_rn(n, __dadd_rn(s2, e2))), 1.0 + 0x1p-40);
      const int qmin = ((int)(emin >> 7) > 1 ? (int)(emin >> 7) : 1) - 134;
      const double e1 = bnd < ldexp(1.0, qmin + 53) ? 0.0 : __dmul_rn(bnd, 0x1p-45);
      const double m_lo = __ddiv_rn(__dsub_rn(s1, e1), n), m_hi = __ddiv_rn(__dadd_rn(s1, e1), n);
      const float m32 = __double2float_rn(m_lo);
      // the range of |mean| over the interval, then of var = ms - mean^2
      const double f_lo = fabs(m_lo), f_hi = fabs(m_hi);
      const double a_lo = m_lo <= 0.0 && m_hi >= 0.0 ? 0.0 : (f_lo < f_hi ? f_lo : f_hi);
      const double a_hi = f_lo > f_hi ? f_lo : f_hi;
      v_lo = __dsub_rn(ms_lo, __dmul_rn(a_hi, a_hi));
      v_hi = __dsub_rn(ms_hi, __dmul_rn(a_lo, a_lo));
      settled = m32 == __double2float_rn(m_hi);
      mean32 = m32;
    } else {
      settled = true;
    }
    const float r_small = __double2float_rn(__ddiv_rn(1.0, __dsqrt_rn(__dadd_rn(v_hi, norm_eps))));
    const float r_large = __double2float_rn(__ddiv_rn(1.0, __dsqrt_rn(__dadd_rn(v_lo, norm_eps))));
    settled = settled && r_small == r_large;  // false for NaN (var + norm_eps < 0)
    rstd32 = r_small;
  }
  if (!settled) {
    long long* L1 = s_limbs[slot];
    long long* L2 = s_limbs[slot] + kS1Limbs;
    if (t < kS1Limbs + kS2Limbs) s_limbs[slot][t] = 0;
    if constexpr (TPR == 256) __syncthreads();
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        exact_add<LAYER>(w[k] & 0xffffu, L1, L2);
        exact_add<LAYER>(w[k] >> 16, L1, L2);
      }
    }
    if constexpr (TPR == 256) __syncthreads();
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t == 0) {
      s_exact[slot][0] = LAYER ? limbs_to_double(L1, kS1Limbs, -133) : 0.0;
      s_exact[slot][1] = limbs_to_double(L2, kS2Limbs, -266);
    }
    if constexpr (TPR == 256) __syncthreads();
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    s1 = s_exact[slot][0];
    s2 = s_exact[slot][1];
    const double mean = __ddiv_rn(s1, n), ms = __ddiv_rn(s2, n);
    const double var = LAYER ? __dsub_rn(ms, __dmul_rn(mean, mean)) : ms;
    const double rstd = __ddiv_rn(1.0, __dsqrt_rn(__dadd_rn(var, norm_eps)));
    mean32 = __double2float_rn(mean);
    rstd32 = __double2float_rn(rstd);
  }
  // normalize, keep as bf16 in registers (and store to y)
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = 8 * (t + TPR * j);
    if (c >= cols) continue;
    const uint4 gv = *reinterpret_cast<const uint4*>(gamma + c);
    const uint4 bv = LAYER && beta ? *reinterpret_cast<const uint4*>(beta + c) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float t0, t1;
      if constexpr (LAYER) {
        t0 = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(bf16_lo(w[k]), mean32), rstd32), bf16_lo(gw[k])),
                       bf16_lo(bw[k]));
        t1 = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(bf16_hi(w[k]), mean32), rstd32), bf16_hi(gw[k])),
                       bf16_hi(bw[k]));
      } else {
        t0 = __fmul_rn(__fmul_rn(bf16_lo(w[k]), rstd32), bf16_lo(gw[k]));
        t1 = __fmul_rn(__fmul_rn(bf16_hi(w[k]), rstd32), bf16_hi(gw[k]));
      }
      // gfx950's packed convert, two values per instruction: round to
      // nearest even, the same bits as f32_to_bf16_rne for every non-NaN
      // value (subnormals included); a NaN stays a NaN
      const bf16x2_t h = {(__bf16)t0, (__bf16)t1};
      o[k] = __builtin_bit_cast(uint32_t, h);
    }
    v[j] = make_uint4(o[0], o[1], o[2], o[3]);
    m = amax8(v[j], m);
    if (y) *reinterpret_cast<uint4*>(y + row * cols + c) = v[j];
  }
  if (!q) return;
  if constexpr (TPR == 64)
    m = wave_max(m);
  else
    m = block_max<256>(m, red);
  float s, iv;
  scale_from_amax(m, fmax, eps, s, iv);
  if (t == 0) {
    scale[row] = s;
    if (inv) inv[row] = iv;
  }
  const float fm = (float)fmax;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t c = 8 * (t + TPR * j);
    if (c < cols) st_nt8(q + row * cols + c, quant8<E5>(v[j], s, fm));
  }
}

template <bool E5, bool LAYER>
static void launch_norm_quant_t(const NormQuantArgs& a) {
  const dim3 block(256);
  auto go = [&](auto kern, int64_t blocks) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), block, 0, a.stream, a.x, a.gamma, a.beta, a.rows, a.cols,
                       a.norm_eps, a.y, a.q, a.scale, a.inv, a.fmax, a.eps);
  };
  if (a.cols <= 512 * 8) {  // one wavefront per row
    const int64_t J = (a.cols + 511) / 512, blocks = (a.rows + 3) / 4;
    if (J <= 2)
      go(k_norm_quant_row<64, 2, E5, LAYER>, blocks);
    else if (J <= 4)
      go(k_norm_quant_row<64, 4, E5, LAYER>, blocks);
    else
      go(k_norm_quant_row<64, 8, E5, LAYER>, blocks);
  } else {
    const int64_t J = (a.cols + 2047) / 2048;
    if (J <= 4)
      go(k_norm_quant_row<256, 4, E5, LAYER>, a.rows);
    else
      go(k_norm_quant_row<256, 8, E5, LAYER>, a.rows);
  }
}

hipError_t launch_norm_quant_row(const NormQuantArgs& a) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.layer)
    a.e5 ? launch_norm_quant_t<true, true>(a) : launch_norm_quant_t<false, true>(a);
  else
    a.e5 ? launch_norm_quant_t<true, false>(a) : launch_norm_quant_t<false, false>(a);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const QuantArgs& a, void* ws) {
  return a.e5 ? launch_tensor_t<true>(a, (uint32_t*)ws) : launch_tensor_t<false>(a, (uint32_t*)ws);
}

// Grid of the looping 1-D quantizers: a grid of up to four resident rounds
// (8 workgroups of 256 threads per CU) runs as one round of workgroups that
// loop, which cut the 1 x 128 and MX activations of the Llama-4-style MoE
// ([8192, 5120]) from 26.6 to 25.3 us and 28.8 to 26.8 us; larger grids keep one
// workgroup per work item (capping the 16 x 8192 x 5120 MX weights at one round
// measured 10% slower).
static int64_t looping_grid(int64_t blocks) {
  if (blocks > 2048 && blocks <= 8192) return 2048;
  return blocks > 65536 ? 65536 : blocks;
}

template <bool E5>
static hipError_t launch_block_t(const QuantArgs& a, int br, int bc) {
  const int64_t B = a.batch, R = a.rows, C = a.cols;
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  const bool vec = C % 8 == 0 && aligned16(a.x) && aligned16(a.q);
  const int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
  if (vec && br == 1 && bc == 128) {
    const int64_t ngroups = B * R * nbc;
    const bool small = ngroups * 128 < ((int64_t)1 << 28);
    const int64_t blocks = looping_grid((ngroups + 16 * (small ? 4 : 1) - 1) / (16 * (small ? 4 : 1)));
    if (small)
      hipLaunchKernelGGL((k_quant_group1d<E5, 128, false, 4>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x,
                         B * R, C, a.q, a.scale, a.inv, (uint8_t*)nullptr, a.fmax, a.eps, 0);
    else
      hipLaunchKernelGGL((k_quant_group1d<E5, 128, false, 1>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x,
                         B * R, C, a.q, a.scale, a.inv, (uint8_t*)nullptr, a.fmax, a.eps, 0);
  } else if (vec && br == 128 && bc == 128 && C % 256 == 0) {
    hipLaunchKernelGGL((k_quant_block128<E5, 2>), dim3((unsigned)(B * nbr * nbc / 2)), dim3(512), 0, a.stream, a.x, R,
                       C, nbr, nbc, a.q, a.scale, a.inv, a.fmax, a.eps);
  } else if (vec && br == 128 && bc == 128) {
    hipLaunchKernelGGL((k_quant_block128<E5, 1>), dim3((unsigned)(B * nbr * nbc)), dim3(256), 0, a.stream, a.x, R, C,
                       nbr, nbc, a.q, a.scale, a.inv, a.fmax, a.eps);
  } else {
    hipLaunchKernelGGL((k_quant_block_generic<E5, false>), dim3((unsigned)(B * nbr * nbc)), dim3(256), 0, a.stream, a.x,
                       R, C, (int64_t)br, (int64_t)bc, nbr, nbc, a.q, a.scale, a.inv, (uint8_t*)nullptr, a.fmax, a.eps, 0);
  }
  return hipGetLastError();
}

hipError_t launch_quant_block(const QuantArgs& a, int br, int bc) {
  return a.e5 ? launch_block_t<true>(a, br, bc) : launch_block_t<false>(a, br, bc);
}

template <bool E5>
static hipError_t launch_mx_t(const QuantArgs& a, uint8_t* e8m0, int mode) {
  const int64_t B = a.batch, R = a.rows, C = a.cols;
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  const bool vec = aligned16(a.x) && aligned16(a.q);  // C % 32 == 0 is checked by the API
  if (vec) {
    const int64_t ngroups = B * R * (C / 32);
    const bool small = ngroups * 32 < ((int64_t)1 << 28);
    const int64_t blocks = looping_grid((ngroups + 64 * (small ? 4 : 1) - 1) / (64 * (small ? 4 : 1)));
    if (small)
      hipLaunchKernelGGL((k_quant_group1d<E5, 32, true, 4>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x,
                         B * R, C, a.q, (float*)nullptr, (float*)nullptr, e8m0, a.fmax, a.eps, mode);
    else
      hipLaunchKernelGGL((k_quant_group1d<E5, 32, true, 1>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x,
                         B * R, C, a.q, (float*)nullptr, (float*)nullptr, e8m0, a.fmax, a.eps, mode);
  } else {
    const int64_t nbc = C / 32;
    hipLaunchKernelGGL((k_quant_block_generic<E5, true>), dim3((unsigned)(B * R * nbc)), dim3(256), 0, a.stream, a.x,
                       B * R, C, (int64_t)1, (int64_t)32, B * R, nbc, a.q, (float*)nullptr, (float*)nullptr, e8m0,
                       a.fmax, a.eps, mode);
  }
  return hipGetLastError();
}

hipError_t launch_quant_mx(const QuantArgs& a, uint8_t* e8m0, int mode) {
  return a.e5 ? launch_mx_t<true>(a, e8m0, mode) : launch_mx_t<false>(a, e8m0, mode);
}

// MX groups as k_quant_group1d<E5, 32, true>, codes written in the packed
// layouts of the grouped GEMM's operands: GR = 16 k-packed (1 KB chunks of
// 16 rows x 64 columns), GR = 2 pair-interleaved (128-byte chunks of 2 rows
// x 64 columns); code (r, c) at ((r / GR) * (cols / 64) + c / 64) * 64 GR +
// (r % GR) * 64 + c % 64. A tile is GR rows x 2048 / GR columns, 8 columns
// per lane (a 32-column group is 4 neighbouring lanes), so a workgroup
// writes whole chunks: both halves of every 128-byte line come from one CU
// and meet in its L2 (with row-major work each half line would be written
// from another XCD). A workgroup takes U column-adjacent tiles per
// iteration, loads first, so it reads U * 4096 / GR contiguous bytes of each
// of its rows.
template <bool E5, int GR, int U>
__global__ __launch_bounds__(256) void k_quant_mx_packed(const uint16_t* __restrict__ x, int64_t nrows, int64_t cols,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ e8m0,
                                                         double fmax, double eps, int mx_mode) {
  constexpr int TC = 2048 / GR, LPR = TC / 8;
  const int lane_row = threadIdx.x / LPR, c8 = threadIdx.x % LPR;
  const int64_t ntc = (cols + TC - 1) / TC;
  const int64_t total = nrows / GR * ntc;
  const int64_t cb = cols / 64, g32 = cols / 32;
  const float fm = (float)fmax;
  for (int64_t t0 = (int64_t)blockIdx.x * U; t0 < total; t0 += (int64_t)gridDim.x * U) {
    uint4 v[U];
    int64_t r[U], c[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u;
      const int64_t band = t / ntc, tc = t % ntc;
      r[u] = band * GR + lane_row;
      c[u] = tc * TC + 8 * c8;
      ok[u] = t < total && c[u] < cols;
      v[u] = ok[u] ? ld_nt16(x + r[u] * cols + c[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float m = amax8(v[u], 0.0f);
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      const int k = mx_exponent(m, fmax, eps, mx_mode);
      if (ok[u]) {
        if ((c8 & 3) == 0) e8m0[r[u] * g32 + c[u] / 32] = (uint8_t)(127 - k);
        const int64_t o = ((r[u] / GR) * cb + c[u] / 64) * (64 * GR) + (r[u] % GR) * 64 + c[u] % 64;
        *reinterpret_cast<uint2*>(q + o) = quant8<E5>(v[u], exp2i(k), fm);
      }
    }
  }
}

template <bool E5, int GR>
static hipError_t launch_mx_packed_t(const QuantArgs& a, uint8_t* e8m0, int mode) {
  const int64_t R = a.batch * a.rows, C = a.cols;
  if (R == 0 || C == 0) return hipSuccess;
  constexpr int U = 4;
  const int64_t tiles = R / GR * ((C + 2048 / GR - 1) / (2048 / GR));
  const int64_t blocks = looping_grid((tiles + U - 1) / U);
  hipLaunchKernelGGL((k_quant_mx_packed<E5, GR, U>), dim3((unsigned)blocks), dim3(256), 0, a.stream, a.x, R, C, a.q,
                     e8m0, a.fmax, a.eps, mode);
  return hipGetLastError();
}

hipError_t launch_quant_mx_packed(const QuantArgs& a, uint8_t* e8m0, int mode, int group_rows) {
  if (group_rows == 2) return a.e5 ? launch_mx_packed_t<true, 2>(a, e8m0, mode) : launch_mx_packed_t<false, 2>(a, e8m0, mode);
  return a.e5 ? launch_mx_packed_t<true, 16>(a, e8m0, mode) : launch_mx_packed_t<false, 16>(a, e8m0, mode);
}

}  // namespace fp8dyn
