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
#include "gemm_common.hpp"

namespace fp8dyn {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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

  int64_t t_begin, t_end, t_step;
  xcd_range(total, t_begin, t_end, t_step);

  // loader role of this thread
  const bool is_g = tid < GBLK;
  const int lb = is_g ? tid : tid - GBLK;
  const int cols8 = is_g ? BNT / 8 : BKT / 8;
  const int blk_m = lb / cols8, blk_c = lb % cols8;  // m block (0..7), column block
  const uint16_t* src = is_g ? gy : x;
  const int64_t ld = is_g ? N : K;
  const int64_t limc = is_g ? N : K;

  for (int64_t t = t_begin; t < t_end; t += t_step) {
    // grouped order: kGroupM row-tiles, column tiles fastest
    const int64_t g = t / (kGroupM * tk), rem = t % (kGroupM * tk);
    const int64_t gm = (tn - g * kGroupM) < kGroupM ? (tn - g * kGroupM) : kGroupM;
    const int64_t n0 = (g * kGroupM + rem % gm) * BNT, k0 = (rem / gm) * BKT;
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
          if (n < N) gw[n * K + k] = f32_to_bf16_rne(acc[i][j][r]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined form for M % 64 == 0: no register transpose at all. Tiles of gy
// and x go from HBM into LDS as stored (rows of m) with the LDS DMA of the
// FP8 kernels, and the matrix-core fragments, which need consecutive m for a
// fixed n (or k), are read with gfx950's transposing LDS read
// ds_read_b64_tr_b16. Measured on MI355X: within each group of 16 lanes,
// lane r supplies the address of 4 consecutive 16-bit values (row r of a
// 16 x 4 block) and lane t receives rows 4e + t / 4 (e = 0..3) of column
// t % 4. With lane r pointing at (m0 + r / 4, n0 + 4 (r % 4)), lane t
// therefore receives the 4 consecutive m of column n0 + t; two such reads give
// the 8 consecutive m that v_mfma_f32_32x32x16_bf16 takes per lane (lane l:
// row l % 32, K [8 (l / 32), 8 (l / 32) + 8)).
//
//  - 256 (n) x 256 (k) output tile, 4 waves of 128 x 128 (accumulators in
//    AGPRs), stages of 32 m (16 KB of gy + 16 KB of x), a ring of 4 stages:
//    the loads of stage s + 4 are issued after the barrier of step s, the
//    fragments of stage s + 1 are read while stage s is multiplied, so each
//    load has three steps to land.
//  - LDS rows are 512 bytes (256 values of one m); their 16-byte chunks are
//    XOR-swizzled by 4 (m % 8), which spreads the 8 rows x 64 bytes of one
//    transposing read over all banks.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}

struct WgFrags {
  v8bf a[4][2], b[4][2];  // [32-row block][16-deep k step]
};

// per-tile cost beyond its stages (prologue, epilogue), in stages
constexpr int64_t kTileCost = 4;

// Grouped form (GR): expert e contracts over its own rows [off[e], off[e+1]):
// gw[e] = gy[rows]^T x[rows]. Its stages are padded to an even count; loads of
// rows past the expert's end fetch its last row (a valid address) and the wave
// that loaded them zeroes those LDS rows after its own loads landed and before
// the barrier that lets anyone read the stage. An empty expert gets a zero
// gradient.
// Dense form: tiles [t_lo, t_lo + t_cnt) of the grouped tile order. HALF:
// work item u is the k half u % 2 (128 columns) of tile t_lo + u / 2; it loads
// the whole tile's stages and runs half the products, each wave 128 x 64. A
// launch of half tiles takes the tiles that would otherwise leave most of the
// last round of workgroups idle (section on the launcher below).
template <bool GR, bool HALF = false>
__global__ __launch_bounds__(256, 1) void k_wgrad_pipe(const uint16_t* __restrict__ gy, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ offsets, int32_t E, int64_t M,
                                                      int64_t N, int64_t K, uint16_t* __restrict__ gw, int64_t t_lo,
                                                      int64_t t_cnt) {
  static_assert(!(GR && HALF), "half tiles: dense form");
  constexpr int BN = 256, BK = 256, MS = 32, NS = 4;
  constexpr int ROWB = 512;                    // bytes per LDS row (256 values)
  constexpr int SG = MS * ROWB, STAGE = 2 * SG;  // gy part, whole stage
  constexpr int NW = 4, WN = 2, TM = 128, TN = HALF ? 64 : 128, MI = 4, NI = TN / 32;
  constexpr int D = STAGE / 1024 / NW;  // wave-wide 1 KB loads per wave per stage
  static_assert(D == 8, "stage split");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];
  // grouped form: offsets and the cumulative cost of the experts' tiles
  __shared__ int32_t s_off[GR ? kMaxExperts + 1 : 1];
  __shared__ int64_t s_cum[GR ? kMaxExperts + 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tn = (N + BN - 1) / BN, tk = (K + BK - 1) / BK;
  const uint32_t lds0 = lds_addr(lds);
  // 8-byte output stores where gw allows (K % 8 == 0 keeps every row aligned)
  const bool vec_out = ((uintptr_t)gw & 7) == 0;
  // The XCD-aware split of the tile list (xcd_range). Grouped: the tiles of
  // an expert differ in length (its rows), so the XCDs get contiguous ranges
  // of equal total cost (stages + kTileCost per tile) rather than of equal
  // tile counts; within an XCD the workgroups still take neighbouring tiles
  // together, which share operand rows in that XCD's L2.
  const int64_t tpe = tn * tk;  // tiles per expert
  int64_t t_begin, t_end, t_step;
  auto stages_of = [&](int32_t e) -> int64_t {
    const int64_t me = (int64_t)s_off[e + 1] - s_off[e];
    return ((me + 2 * MS - 1) / (2 * MS)) * 2;
  };
  if constexpr (GR) {
    for (int i = tid; i <= E; i += 256) s_off[i] = offsets[i];
    __syncthreads();
    if (tid == 0) {
      clamp_offsets_serial(s_off, E, M);
      int64_t acc = 0;
      for (int32_t e = 0; e < E; ++e) {
        s_cum[e] = acc;
        acc += tpe * (stages_of(e) + kTileCost);
      }
      s_cum[E] = acc;
    }
    __syncthreads();
    // first tile whose start cost is >= w
    auto tile_at = [&](int64_t w) -> int64_t {
      if (w >= s_cum[E]) return (int64_t)E * tpe;
      int32_t lo = 0, hi = E;  // s_cum[lo] <= w < s_cum[hi]
      while (hi - lo > 1) {
        const int32_t mid = (lo + hi) / 2;
        if (s_cum[mid] <= w) lo = mid; else hi = mid;
      }
      const int64_t cost = stages_of(lo) + kTileCost;
      const int64_t j = (w - s_cum[lo] + cost - 1) / cost;
      return (int64_t)lo * tpe + j;  // j == tpe is the next expert's first tile
    };
    const int64_t G = gridDim.x, W = s_cum[E];
    if (G % kNumXcd == 0) {
      const int64_t xcd = blockIdx.x % kNumXcd;
      t_begin = uniform64(tile_at(W * xcd / kNumXcd) + blockIdx.x / kNumXcd);
      t_end = uniform64(tile_at(W * (xcd + 1) / kNumXcd));
      t_step = G / kNumXcd;
    } else {
      t_begin = blockIdx.x;
      t_end = (int64_t)E * tpe;
      t_step = G;
    }
  } else {
    xcd_range(HALF ? 2 * t_cnt : t_cnt, t_begin, t_end, t_step);
  }

  // loads: waves 0-1 take gy (16 pieces of 1 KB = 2 rows), waves 2-3 take x;
  // lane i of a piece fills row 2 q + i / 32, physical chunk i % 32
  const bool loads_g = wave < 2;
  const int q0 = (wave & 1) * D;
  const uint16_t* src = loads_g ? gy : x;
  const int64_t ld = loads_g ? N : K;
  const int64_t nchunk = ld / 8;  // valid 16-byte chunks per row

  // transposing-read address of this lane within a stage region, for row
  // block base rb (0..224), k step ks, half h: m = 16 ks + 8 (grp / 2) + 4 h +
  // r / 4, column = rb + 16 (grp % 2) + 4 (r % 4)
  const int grp = lane >> 4, rr4 = lane & 15;
  auto tr_off = [&](int rb, int ks, int h) -> uint32_t {
    const int m = 16 * ks + 8 * (grp >> 1) + 4 * h + (rr4 >> 2);
    const int c = rb + 16 * (grp & 1) + 4 * (rr4 & 3);
    const int chunk = (c >> 3) ^ ((m & 7) << 2);
    return (uint32_t)(m * ROWB + chunk * 16 + (c & 7) * 2);
  };
  uint32_t fa[MI][2][2], fb[NI][2][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) fa[i][ks][h] = tr_off(wm * TM + 32 * i, ks, h);
  // this wave's first column within the loaded tile (HALF: set per item)
  int cb = wn * TN;
  auto set_fb = [&]() {
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) fb[j][ks][h] = (uint32_t)SG + tr_off(cb + 32 * j, ks, h);
  };
  if constexpr (!HALF) set_fb();

  for (int64_t t0 = t_begin; t0 < t_end; t0 += t_step) {
    // expert (grouped form), then grouped order over its tiles: 4 row tiles
    // (n), column tiles (k) fastest
    int64_t t = t0, m_beg = 0, m_end = M;
    int32_t e = 0;
    if constexpr (HALF) {
      t = t_lo + t0 / 2;
      cb = (int)(t0 & 1) * 128 + wn * TN;
      set_fb();
    } else if constexpr (!GR) {
      t = t_lo + t0;
    }
    if constexpr (GR) {
      e = __builtin_amdgcn_readfirstlane((int32_t)(t0 / tpe));
      t = t0 - (int64_t)e * tpe;
      m_beg = __builtin_amdgcn_readfirstlane(s_off[e]);
      m_end = __builtin_amdgcn_readfirstlane(s_off[e + 1]);
    }
    const int64_t me = m_end - m_beg;
    // stages of 32 rows (even count: whole steady pairs); dense: M % 64 == 0
    const int64_t nk = GR ? ((me + 2 * MS - 1) / (2 * MS)) * 2 : M / MS;
    // (the column-tile count opaque per tile, so the divisions form their
    // reciprocal here rather than hold it in a register across the loop)
    int64_t tk_t = tk;
    asm volatile("" : "+s"(tk_t));
    const int64_t g = t / (kGroupM * tk_t), rem = t % (kGroupM * tk_t);
    const int64_t gm = (tn - g * kGroupM) < kGroupM ? (tn - g * kGroupM) : kGroupM;
    const int64_t n0 = uniform64((g * kGroupM + rem % gm) * BN), k0 = uniform64((rem / gm) * BK);
    const int64_t col0 = loads_g ? n0 : k0;
    uint32_t off[D];
    // the lane id opaque per tile: the offsets below (products row * ld
    // among them) are then formed per tile; hoisted out of the tile loop they
    // were spilled and each tile's reload waited for the previous tile's
    // stores
    int32_t ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int row = 2 * (q0 + d) + (ln >> 5);
      const int c = (ln & 31) ^ ((row & 7) << 2);
      int64_t cc = col0 / 8 + c;
      cc = cc < nchunk ? cc : nchunk - 1;  // columns past N (or K) load a valid chunk
      off[d] = (uint32_t)((row * ld + 8 * cc) * 2);
    }
    const uint32_t opnd_lds = loads_g ? 0u : (uint32_t)SG;

    auto issue = [&](int64_t s) {
      const uint32_t slot = lds0 + (uint32_t)((s % NS) * STAGE) + opnd_lds + (uint32_t)(q0 * 1024);
      if (!GR || MS * (s + 1) <= me) {
        const uint8_t* bs = reinterpret_cast<const uint8_t*>(src + (m_beg + s * MS) * ld);
#pragma unroll
        for (int d = 0; d < D; ++d) dma16(bs, off[d], slot + (uint32_t)(d * 1024));
      } else {
        // the expert ends inside (or before) this stage: rows past its end
        // load its last row, zeroed later by zero_tail
        const int64_t r0 = m_beg + s * MS < m_end - 1 ? m_beg + s * MS : m_end - 1;
        const int32_t rmax = (int32_t)(m_end - 1 - r0);
        const uint8_t* bs = reinterpret_cast<const uint8_t*>(src + r0 * ld);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int32_t row = 2 * (q0 + d) + (lane >> 5);
          const int32_t rc = row < rmax ? row : rmax;
          dma16(bs, off[d] - (uint32_t)((row - rc) * ld * 2), slot + (uint32_t)(d * 1024));
        }
      }
    };
    // zero this wave's LDS rows of stage s that lie past the expert's end
    // (after its own loads of the stage landed)
    auto zero_tail = [&](int64_t s) {
      if (!GR || MS * (s + 1) <= me) return;
      uint8_t* slot = lds + (s % NS) * STAGE + opnd_lds + q0 * 1024;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int row = 2 * (q0 + d) + (lane >> 5);
        if (m_beg + s * MS + row >= m_end)
          *reinterpret_cast<uint4*>(slot + d * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    };
    auto read = [&](int64_t s, WgFrags& f) {
      const uint8_t* st = lds + (s % NS) * STAGE;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v4s lo = lds_read_tr16(st + fa[i][ks][0]), hi = lds_read_tr16(st + fa[i][ks][1]);
          f.a[i][ks] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v4s lo = lds_read_tr16(st + fb[j][ks][0]), hi = lds_read_tr16(st + fb[j][ks][1]);
          f.b[j][ks] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    v16f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // transposed products (x fragment first): register 4 q + t of lane l in
    // block (i, j) is n = 32 i + l % 32, k = 32 j + 8 q + 4 (l / 32) + t, so a
    // lane stores 4 adjacent outputs at once
    auto mma = [&](const WgFrags& f) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j][ks], f.a[i][ks], acc[i][j], 0, 0, 0);
    };
    auto read_mma = [&](int64_t s_next, WgFrags& nxt, const WgFrags& cur) {
      read(s_next, nxt);
      mma(cur);
      if constexpr (HALF) {
        // 24 LDS reads, 16 MFMAs
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        }
      }
    };
    auto steady = [&](int64_t s, WgFrags& cur, WgFrags& nxt) {
      wait_vm_lgkm_and_barrier<2 * D>();
      issue(s + NS);
      read_mma(s + 1, nxt, cur);
    };

    // only the last two stages can hold rows past the expert's end: their
    // waits are split so each wave zeroes its own such rows in between
    WgFrags f0, f1;
    if (!GR || nk > 0) {
      if (nk >= NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) issue(s);
        wait_vm_and_barrier<(NS - 1) * D>();
      } else {  // nk == 2
        issue(0);
        issue(1);
        wait_vm<D>();
        zero_tail(0);
        wait_lgkm_and_barrier();
      }
      read(0, f0);
      for (int64_t s = 0; s + NS < nk; s += 2) {
        steady(s, f0, f1);
        steady(s + 1, f1, f0);
      }
      if (nk >= NS) {
        wait_vm_lgkm_and_barrier<2 * D>();
        read_mma(nk - 3, f1, f0);
        wait_vm<D>();
        zero_tail(nk - 2);
        wait_lgkm_and_barrier();
        read_mma(nk - 2, f0, f1);
      }
      wait_vm<0>();
      zero_tail(nk - 1);
      wait_lgkm_and_barrier();
      read_mma(nk - 1, f1, f0);
      wait_vm_lgkm_and_barrier<0>();
      mma(f1);
    }

    // ---- epilogue: block (i, j), register 4 q + t of lane l: n = 32 i + l % 32,
    // k = 32 j + 8 q + 4 (l / 32) + t of the wave's part; K % 8 == 0, so a
    // lane's 4 columns are all inside K or all past it ----
    int32_t nl0 = wm * TM + (lane & 31), kl0 = cb + 4 * (lane >> 5);
    asm volatile("" : "+v"(nl0), "+v"(kl0));
    uint16_t* const gwe = gw + (int64_t)e * N * K;
    if (vec_out) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t n = n0 + nl0 + 32 * i;
        if (n >= N) continue;
        uint16_t* const row = gwe + n * K + k0;
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int32_t kl = kl0 + 32 * j + 8 * q;
            if (k0 + kl >= K) continue;
            const v16f& a = acc[i][j];
            const v2bf h01 = {(__bf16)a[4 * q], (__bf16)a[4 * q + 1]}, h23 = {(__bf16)a[4 * q + 2], (__bf16)a[4 * q + 3]};
            *reinterpret_cast<uint2*>(row + kl) =
                make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t n = n0 + nl0 + 32 * i;
        if (n >= N) continue;
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int32_t kl = kl0 + 32 * j + 8 * q;
            if (k0 + kl >= K) continue;
#pragma unroll
            for (int t = 0; t < 4; ++t) gwe[n * K + k0 + kl + t] = f32_to_bf16_rne(acc[i][j][4 * q + t]);
          }
      }
    }
  }
}

hipError_t launch_wgrad_bf16(const WgradArgs& w) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  constexpr int BNT = 256, BKT = 256;
  const int64_t total = ((w.N + BNT - 1) / BNT) * ((w.K + BKT - 1) / BKT);
  const int cus = device_cus();
  // pipelined form: whole 64-row steps of m; a stage (32 rows) of either
  // operand addressed with 32-bit offsets
  const int64_t ldmax = w.N > w.K ? w.N : w.K;
  if (w.M >= 64 && w.M % 64 == 0 && 32 * ldmax * 2 < ((int64_t)1 << 31)) {
    int64_t grid = cus < total ? cus : total;
    if (grid >= kNumXcd) grid -= grid % kNumXcd;
    if (grid < 1) grid = 1;
    // Whole rounds of tiles, then the rest. When the rest would occupy at
    // most half the workgroups for a whole extra round (896 tiles on 256 CUs:
    // 128 left over), a second launch splits each leftover tile into its two
    // 128-column halves, one per workgroup, and the extra round takes about
    // half as long.
    const int64_t full = (total / grid) * grid, rest = total - full;
    const bool halves = full > 0 && rest > 0 && 2 * rest <= grid;
    hipLaunchKernelGGL((k_wgrad_pipe<false, false>), dim3((unsigned)grid), dim3(256), 0, w.stream, w.gy, w.x,
                       (const int32_t*)nullptr, 1, w.M, w.N, w.K, w.gw, (int64_t)0, halves ? full : total);
    if (halves) {
      int64_t g2 = 2 * rest;
      if (g2 >= kNumXcd) g2 -= g2 % kNumXcd;
      hipLaunchKernelGGL((k_wgrad_pipe<false, true>), dim3((unsigned)g2), dim3(256), 0, w.stream, w.gy, w.x,
                         (const int32_t*)nullptr, 1, w.M, w.N, w.K, w.gw, full, rest);
    }
    return hipGetLastError();
  }
  int64_t grid = cus < total ? cus : total;
  if (grid >= kNumXcd) grid -= grid % kNumXcd;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_wgrad_bf16<BNT, BKT, 2, 4>), dim3((unsigned)grid), dim3(512), 0, w.stream, w.gy, w.x, w.M, w.N,
                     w.K, w.gw);
  return hipGetLastError();
}

hipError_t launch_grouped_wgrad_bf16(const GroupedWgradArgs& w) {
  if (w.E == 0 || w.N == 0 || w.K == 0) return hipSuccess;
  constexpr int BNT = 256, BKT = 256;
  const int64_t total = (int64_t)w.E * ((w.N + BNT - 1) / BNT) * ((w.K + BKT - 1) / BKT);
  const int cus = device_cus();
  int64_t grid = cus < total ? cus : total;
  if (grid >= kNumXcd) grid -= grid % kNumXcd;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_wgrad_pipe<true, false>), dim3((unsigned)grid), dim3(256), 0, w.stream, w.gy, w.x, w.offsets,
                     w.E, w.Mtot, w.N, w.K, w.gw, (int64_t)0, total);
  return hipGetLastError();
}

}  // namespace fp8dyn
