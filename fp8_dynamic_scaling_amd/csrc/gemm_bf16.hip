// gemm_bf16.hip -- the BF16 weight-gradient GEMM of a Linear layer,
// gw[n][k] = sum_m gy[m][n] * x[m][k] ("FP8 training on AMD GPUs with
// TorchTitan and TorchAO", Figure 1 caption: the weight-update GEMM stays in
// BF16 while the forward and grad-input GEMMs use FP8).
//
// Both operands are stored with the contracted index m as the row index
// ([M][N] and [M][K] row-major), which is the layout that forced
// transposed copies in the pages' baseline ("FP8 Training: Quantization,
// Autograd, Torchao", section 4). Here no copy is made: each thread loads an
// 8 x 8 bf16 block (8 rows of m, 8 adjacent columns) with 16-byte loads,
// transposes it in registers with 16-bit permutes, and writes it to LDS as
// 8 rows of 8 consecutive m values, the layout the bf16 matrix-core
// instruction (v_mfma_f32_16x16x32_bf16, 8 consecutive contracted values per
// lane) reads directly.
#include "common.hpp"
#include "internal.hpp"

namespace fp8dyn {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWNumXcd = 8;
constexpr int kWGroup = 4;

__device__ __forceinline__ uint16_t w_f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 8 x 8 transpose of 16-bit values: in[r] holds row r (8 values, 2 per word);
// out[c] receives column c (8 values, rows 0..7).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4& r0 = in[2 * p];
      const uint4& r1 = in[2 * p + 1];
      const uint32_t d0 = (c >> 1) == 0 ? r0.x : (c >> 1) == 1 ? r0.y : (c >> 1) == 2 ? r0.z : r0.w;
      const uint32_t d1 = (c >> 1) == 0 ? r1.x : (c >> 1) == 1 ? r1.y : (c >> 1) == 2 ? r1.z : r1.w;
      w[p] = (c & 1) ? ((d0 >> 16) | (d1 & 0xffff0000u)) : ((d0 & 0xffffu) | (d1 << 16));
    }
    out[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Tile: BN_ (rows of gw, i.e. n) x BK_ (columns of gw, i.e. k); contraction
// step of 64 m values (two 32-deep MFMAs). LDS rows are 128 bytes
// (64 bf16 of m), 16-byte chunks XOR-swizzled by row.
template <int BNT, int BKT, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, 1) void k_wgrad_bf16(const uint16_t* __restrict__ gy,
                                                               const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                               int64_t K, uint16_t* __restrict__ gw) {
  constexpr int NT = WM * WN * 64;
  constexpr int MS = 64;  // m values per step
  constexpr int TM = BNT / WM, TN = BKT / WN;
  constexpr int MI = TM / 16, NI = TN / 16;
  // transposing loaders: each owns an 8 (m) x 8 (col) block
  constexpr int GBLK = (MS / 8) * (BNT / 8);  // blocks of gy per step
  constexpr int XBLK = (MS / 8) * (BKT / 8);
  static_assert(GBLK + XBLK == NT, "one 8x8 block per thread");

  __shared__ __attribute__((aligned(16))) uint16_t lds_g[2][BNT * MS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[2][BKT * MS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lk = lane >> 4;
  const int64_t tn = (N + BNT - 1) / BNT, tk = (K + BKT - 1) / BKT;
  const int64_t total = tn * tk;
  const int64_t nsteps = (M + MS - 1) / MS;

  const int64_t G = gridDim.x;
  const int64_t per_xcd = G / kWNumXcd;
  const int64_t xcd = blockIdx.x % kWNumXcd, slot = blockIdx.x / kWNumXcd;
  int64_t t_begin, t_end, t_step;
  if (per_xcd > 0 && G % kWNumXcd == 0) {
    t_begin = xcd * total / kWNumXcd + slot;
    t_end = (xcd + 1) * total / kWNumXcd;
    t_step = per_xcd;
  } else {
    t_begin = blockIdx.x;
    t_end = total;
    t_step = G;
  }

  // loader role of this thread
  const bool is_g = tid < GBLK;
  const int lb = is_g ? tid : tid - GBLK;
  const int cols8 = is_g ? BNT / 8 : BKT / 8;
  const int blk_m = lb / cols8, blk_c = lb % cols8;  // m block (0..7), column block
  const uint16_t* src = is_g ? gy : x;
  const int64_t ld = is_g ? N : K;
  const int64_t limc = is_g ? N : K;

  for (int64_t t = t_begin; t < t_end; t += t_step) {
    // grouped order: kWGroup row-tiles, column tiles fastest
    const int64_t g = t / (kWGroup * tk), rem = t % (kWGroup * tk);
    const int64_t gm = (tn - g * kWGroup) < kWGroup ? (tn - g * kWGroup) : kWGroup;
    const int64_t n0 = (g * kWGroup + rem % gm) * BNT, k0 = (rem / gm) * BKT;
    const int64_t c0 = (is_g ? n0 : k0) + blk_c * 8;

    v4f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    uint4 rin[8];
    auto gload = [&](int64_t s) {
      const int64_t mb = s * MS + blk_m * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t m = mb + r;
        rin[r] = (m < M && c0 < limc) ? *reinterpret_cast<const uint4*>(src + m * ld + c0) : make_uint4(0, 0, 0, 0);
      }
    };
    auto lstore = [&](int buf) {
      uint4 tr[8];
      transpose8x8(rin, tr);
      uint16_t* dst = is_g ? lds_g[buf] : lds_x[buf];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int row = blk_c * 8 + c;  // n (or k) within the tile
        const int chunk = blk_m;        // which 8 m values (16 bytes) of the 64
        *reinterpret_cast<uint4*>(dst + row * MS + 8 * (chunk ^ (row & 7))) = tr[c];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int64_t s = 0; s < nsteps; ++s) {
      const int buf = (int)(s & 1);
      if (s + 1 < nsteps) gload(s + 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // two 32-deep halves of the 64 m values
        v8bf bfr[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int row = wn * TN + 16 * j + lr;
          const int chunk = 4 * h + lk;
          bfr[j] = *reinterpret_cast<const v8bf*>(&lds_x[buf][row * MS + 8 * (chunk ^ (row & 7))]);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int row = wm * TM + 16 * i + lr;
          const int chunk = 4 * h + lk;
          const v8bf af = *reinterpret_cast<const v8bf*>(&lds_g[buf][row * MS + 8 * (chunk ^ (row & 7))]);
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
            keep_live(af);
            keep_live(bfr[j]);
          }
        }
      }
      if (s + 1 < nsteps) lstore(buf ^ 1);
      __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t k = k0 + wn * TN + 16 * j + lr;
      if (k >= K) continue;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = n0 + wm * TM + 16 * i + 4 * lk + r;
          if (n < N) gw[n * K + k] = w_f32_to_bf16_rne(acc[i][j][r]);
        }
    }
  }
}

hipError_t launch_wgrad_bf16(const WgradArgs& w) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  constexpr int BNT = 256, BKT = 256;
  const int64_t total = ((w.N + BNT - 1) / BNT) * ((w.K + BKT - 1) / BKT);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  int64_t grid = cus < total ? cus : total;
  if (grid >= kWNumXcd) grid -= grid % kWNumXcd;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_wgrad_bf16<BNT, BKT, 2, 4>), dim3((unsigned)grid), dim3(512), 0, w.stream, w.gy, w.x, w.M, w.N,
                     w.K, w.gw);
  return hipGetLastError();
}

}  // namespace fp8dyn
