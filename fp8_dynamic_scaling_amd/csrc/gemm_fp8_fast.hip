// gemm_fp8_fast.hip -- the main FP8 GEMM kernel for gfx950 (dense and MoE
// grouped; tensorwise, rowwise, 128-blockwise and MX scales) for K a multiple
// of 128 and 16-byte aligned operands; other shapes use the generic kernel in
// gemm_fp8.hip.
//
// What it computes is the scaled GEMM of "FP8 Training: Quantization,
// Autograd, Torchao", section 4 (A row-major, B column-major, multiply by the
// inverse scales) over the expert row ranges of "FP8 training on AMD GPUs with
// TorchTitan and TorchAO", section "Scaling FP8 to MoE Architectures".
//
// Design:
//  - Tensorwise, rowwise and MX scales: the pipelined kernel below (the
//    header comment there has the details).
//  - 128-blockwise scales: k_gemm_fp8_fast, a two-buffer kernel with
//    v_mfma_scale_f32_16x16x128_f8f6f4 and 8 waves of 128 x 64: each 128-deep
//    product is scaled by inv_a[m][kb] * inv_b[nb][kb] and accumulated in fp32
//    registers, which needs a second accumulator set.
//  - Both: 256 x 256 output tiles walked persistently (one workgroup per CU,
//    XCD-aware order; see gemm_common.hpp); operands go from HBM straight into
//    LDS with global_load_lds_dwordx4 (lane i lands at base + 16 i, measured on
//    MI355X), each lane fetching the 16-byte chunk that belongs at its slot
//    under the row-XOR swizzle; rows past the end of an expert (or of N) load
//    a valid clamped row and their outputs are never stored; K % 128 == 0
//    means no K tail.
#include "gemm_common.hpp"

namespace fp8dyn {

// ---------------------------------------------------------------------------
// Pipelined kernel for tensorwise, rowwise and MX scales (the dense Linear
// GEMMs, the rowwise MoE grouped GEMM and the MX grouped GEMM).
//
//  - 256 x 256 output tile, 4 waves of 128 x 128, v_mfma_scale_f32_32x32x64_f8f6f4
//    (64-deep K per instruction; measured lane layout: lane l feeds row l % 32,
//    its low 16 bytes are K [16g, 16g + 16) and its high 16 bytes are
//    K [32 + 16g, 32 + 16g + 16), g = l / 32; so each lane loads 16-byte chunks
//    g and g + 2 of a 64-byte row and the instruction's K order is memory order;
//    the scale operand of lane l covers row l % 32, K block g).
//  - LDS holds a ring of 4 stages of 64-deep K (A and B, 32 KB per stage).
//    At step s, after the barrier that proves stage s + 1 has landed and
//    everyone has finished reading stage s, the HBM -> LDS loads of stage
//    s + 4 go into stage s's slot, so each load has three steps to land.
//    The loads are issued from inline assembly with explicit vmcnt waits: the
//    compiler cannot tell those LDS writes apart from the fragment reads and
//    would otherwise wait for all of them before every read.
//  - Fragments are double-buffered in registers: the 16 LDS reads of stage
//    s + 1 alternate with the 16 MFMAs of stage s. Rows of 64 bytes are
//    XOR-swizzled in 16-byte chunks by (row / 4) so a wave's reads hit
//    distinct banks.
//  - MX: the E8M0 bytes of a stage pair (one dword per row) ride in a small
//    LDS ring of their own, one wave-wide dword load per stage, and each lane
//    reads its byte straight into the MFMA's scale operand.
constexpr int kPipeStages = 4;

// Fragments of one 64-deep stage for one wave: 4 row blocks of A, 4 of B,
// and (MX) this lane's E8M0 scale byte for each of them.
struct PipeFrags {
  v8i a[4], b[4];
  int sa[4], sb[4];
};

template <bool AE5, bool BE5, int SK, bool OF32, bool GR>
__global__ __launch_bounds__(256, 1) void k_gemm_fp8_pipe(GemmParams p) {
  constexpr int BM = 256, BN = 256, BK = 64, NS = kPipeStages;
  constexpr int NW = 4, WN = 2;
  constexpr int TM = 128, TN = 128, MI = TM / 32, NI = TN / 32;
  constexpr int SA_BYTES = BM * BK, SB_BYTES = BN * BK, STAGE = SA_BYTES + SB_BYTES;
  constexpr int D = STAGE / 1024 / NW;  // wave-wide loads per wave per stage
  static_assert(D == 8 && MI == 4 && NI == 4, "stage split");
  typedef float v16f __attribute__((ext_vector_type(16)));

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];
  __shared__ int32_t s_off[GR ? kMaxExperts + 1 : 2];
  __shared__ int64_t s_pref[GR ? kMaxExperts + 1 : 2];
  // MX: E8M0 scales of a stage pair (128-deep K: one dword = 4 K blocks per
  // row), A rows then B rows, in a ring of 4 pairs
  constexpr bool MXS = SK == kScaleMX;
  __shared__ __attribute__((aligned(16))) uint32_t s_scl[MXS ? 4 : 1][MXS ? BM + BN : 1];
  // epilogue: each wave's 128 row scales (rowwise)
  __shared__ __attribute__((aligned(16))) float s_rs[SK == kScaleRow ? NW : 1][SK == kScaleRow ? TM : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 31, lg = lane >> 5;
  const int64_t N = p.N, K = p.K;
  const int64_t nt = (N + BN - 1) / BN;
  const int64_t nk = K / BK;
  const uint32_t lds0 = lds_addr(lds);

  int64_t total;
  if constexpr (GR) {
    total = build_tile_prefix<BM, 256>(p, nt, s_off, s_pref);
  } else {
    total = ((p.M + BM - 1) / BM) * nt;
  }
  int64_t t_begin, t_end, t_step;
  xcd_range(total, t_begin, t_end, t_step);

  // this lane's part of each wave-wide load: 16 rows of 64 bytes per load
  const int ld_row = lane >> 2;    // row within the 16
  const int ld_pch = lane & 3;     // physical 16-byte chunk in the row
  // the waves split a stage: waves 0-1 load A (8 loads each), waves 2-3 load B
  const bool loads_a = wave < 2;
  const int q0 = (wave & 1) * D;   // first 1 KB piece of the operand this wave loads

  // fragment read offsets within a stage (constant over the whole kernel):
  // lane l reads row r = 32 i + l % 32 of its wave's block, 16-byte chunks
  // g and g + 2 (g = l / 32), each XOR-swizzled by (r / 4) % 4
  uint32_t fa_lo[MI], fa_hi[MI], fb_lo[NI], fb_hi[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * TM + 32 * i + lrow, sw = (r >> 2) & 3;
    fa_lo[i] = (uint32_t)(r * BK + 16 * (lg ^ sw));
    fa_hi[i] = (uint32_t)(r * BK + 16 * ((lg + 2) ^ sw));
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = wn * TN + 32 * j + lrow, sw = (r >> 2) & 3;
    fb_lo[j] = (uint32_t)(SA_BYTES + r * BK + 16 * (lg ^ sw));
    fb_hi[j] = (uint32_t)(SA_BYTES + r * BK + 16 * ((lg + 2) ^ sw));
  }

  for (int64_t t = t_begin; t < t_end; t += t_step) {
    TileInfo ti;
    if constexpr (GR) {
      tile_of<BM, BN>(t, s_off, s_pref, p.E, nt, ti);
    } else {
      // grouped-M order over the dense tile grid (same walk as one expert)
      const int64_t mt = (p.M + BM - 1) / BM;
      const int64_t g = t / (kGroupM * nt), rem = t % (kGroupM * nt);
      const int64_t gm = (mt - g * kGroupM) < kGroupM ? (mt - g * kGroupM) : kGroupM;
      ti.e = 0;
      ti.m0 = (g * kGroupM + rem % gm) * BM;
      ti.m_end = p.M;
      ti.n0 = (rem / gm) * BN;
    }
    ti.m0 = uniform64(ti.m0);
    ti.m_end = uniform64(ti.m_end);
    ti.n0 = uniform64(ti.n0);
    ti.e = __builtin_amdgcn_readfirstlane(ti.e);
    const int32_t K32 = (int32_t)K;
    const int32_t a_rows = (int32_t)(ti.m_end - ti.m0);
    const int32_t b_rows = (int32_t)(N - ti.n0 < BN ? N - ti.n0 : BN);
    const uint8_t* base = loads_a ? p.a + ti.m0 * K : p.b + ((int64_t)ti.e * N + ti.n0) * K;
    const int32_t rows = loads_a ? a_rows : b_rows;
    uint32_t off[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int r = 16 * (q0 + d) + ld_row;
      const int c = ld_pch ^ ((r >> 2) & 3);
      const int32_t rr = r < rows ? r : rows - 1;  // rows past the expert / N load a valid row
      off[d] = (uint32_t)(rr * K32 + 16 * c);
    }
    const uint32_t opnd_lds = loads_a ? 0u : (uint32_t)SA_BYTES;

    // MX scale loads: one wave-wide dword load per stage, chunk c = 2 wave +
    // (stage parity) of the pair's 8 chunks of 64 rows (0-3: A, 4-7: B); each
    // lane fetches its row's 4 E8M0 bytes of the pair (rows past the expert /
    // N fetch a valid row)
    const int64_t kb32 = K / 32;
    // per stage parity: the wave's chunk (uniform base, lane offset, LDS offset)
    const uint8_t* sc_base0 = nullptr;
    const uint8_t* sc_base1 = nullptr;
    uint32_t sc_off0 = 0u, sc_off1 = 0u, sc_lds0 = 0u, sc_lds1 = 0u;
    if constexpr (MXS) {
      auto chunk = [&](int par, const uint8_t*& bp, uint32_t& o, uint32_t& l) {
        const int c = 2 * wave + par;
        const bool ca = c < 4;
        const int r = 64 * (c & 3) + lane;
        const int32_t lim = ca ? a_rows : b_rows;
        const int32_t rr = r < lim ? r : lim - 1;
        bp = ca ? reinterpret_cast<const uint8_t*>(p.sa) + ti.m0 * kb32
                : reinterpret_cast<const uint8_t*>(p.sb) + ((int64_t)ti.e * N + ti.n0) * kb32;
        o = (uint32_t)(rr * (int32_t)kb32);
        l = (uint32_t)(4 * ((ca ? 0 : BM) + 64 * (c & 3)));
      };
      chunk(0, sc_base0, sc_off0, sc_lds0);
      chunk(1, sc_base1, sc_off1, sc_lds1);
    }
    auto scale_dma = [&](int64_t pair, bool odd) {
      const int64_t pc = pair < nk / 2 ? pair : nk / 2 - 1;  // past the end: a valid address
      const uint8_t* bp = odd ? sc_base1 : sc_base0;
      const uint32_t o = (odd ? sc_off1 : sc_off0) + (uint32_t)(4 * pc);
      const uint32_t l = lds_addr(&s_scl[pair & 3][0]) + (odd ? sc_lds1 : sc_lds0);
      asm volatile("global_load_lds_dword %0, %1" ::"v"(o), "s"(bp), "{m0}"(l) : "memory");
    };

    // unit s: the D loads of stage s, then (MX) one scale load of pair s / 2 + 1
    auto issue = [&](int64_t s) {
      const uint32_t slot = lds0 + (uint32_t)((s % NS) * STAGE) + opnd_lds + (uint32_t)(q0 * 1024);
      const uint8_t* bk = base + s * BK;
#pragma unroll
      for (int d = 0; d < D; ++d) dma16(bk, off[d], slot + (uint32_t)(d * 1024));
      if constexpr (MXS) scale_dma(s / 2 + 1, (s & 1) != 0);
    };
    constexpr int U = D + (MXS ? 1 : 0);  // loads per unit
    constexpr int X = U - D;              // loads of a unit after its stage's data
    auto read = [&](int64_t s, PipeFrags& f) {
      if constexpr (MXS) {
        // this lane's E8M0 byte: K block 2 s + g of its row (byte (s % 2) * 2 + g
        // of the row's pair dword), read straight into the scale register
        const uint8_t* sp = reinterpret_cast<const uint8_t*>(&s_scl[(s / 2) & 3][0]) + 2 * (int)(s & 1) + lg;
#pragma unroll
        for (int i = 0; i < MI; ++i) f.sa[i] = sp[4 * (wm * TM + 32 * i + lrow)];
#pragma unroll
        for (int j = 0; j < NI; ++j) f.sb[j] = sp[4 * (BM + wn * TN + 32 * j + lrow)];
      }
      const uint8_t* st = lds + (s % NS) * STAGE;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + fa_lo[i]);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + fa_hi[i]);
        f.a[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + fb_lo[j]);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + fb_hi[j]);
        f.b[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    };

    v16f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto mma = [&](const PipeFrags& f) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if constexpr (MXS)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], AE5 ? 1 : 0,
                                                                        BE5 ? 1 : 0, 0, f.sa[i], 0, f.sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], AE5 ? 1 : 0,
                                                                        BE5 ? 1 : 0, 0, 127, 0, 127);
        }
    };

    // One step s: stage s is in registers (cur). Wait until stage s + 1 has
    // landed (W = stages allowed to stay in flight behind it) and every wave
    // has finished reading stage s, whose slot is then free; refill that slot
    // with stage s + 4 (steady state only), read stage s + 1 into nxt while the
    // matrix cores work on cur. K % 128 == 0 makes nk even, so the steady
    // state runs in pairs and a tail of 4 (or 2) steps closes the tile.
    // the 16 fragment reads of the next stage alternate with the 16 MFMAs of
    // this one, so the reads are in flight while the matrix cores are busy
    auto read_mma = [&](int64_t s_next, PipeFrags& nxt, const PipeFrags& cur) {
      read(s_next, nxt);
      mma(cur);
      if constexpr (MXS) {
        // 8 scale reads ride along with the first 8 fragment reads
#pragma unroll
        for (int k = 0; k < MI + NI; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        }
      }
#pragma unroll
      for (int k = MXS ? MI + NI : 0; k < 2 * (MI + NI); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
    };
    auto steady = [&](int64_t s, PipeFrags& cur, PipeFrags& nxt) {
      wait_vm_lgkm_and_barrier<2 * U + X>();
      issue(s + NS);
      read_mma(s + 1, nxt, cur);
    };

    // prologue: (MX) the scales of pair 0, then units 0 .. min(nk, 4) - 1 in
    // flight; stage 0 (and its scales) read into f0
    PipeFrags f0, f1;
    if constexpr (MXS) {
      scale_dma(0, false);
      scale_dma(0, true);
    }
    if (nk >= NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s) issue(s);
      wait_vm_and_barrier<(NS - 1) * U + X>();
    } else {  // nk == 2
      issue(0);
      issue(1);
      wait_vm_and_barrier<U + X>();
    }
    read(0, f0);

    for (int64_t s = 0; s + NS < nk; s += 2) {
      steady(s, f0, f1);
      steady(s + 1, f1, f0);
    }
    if (nk >= NS) {
      wait_vm_lgkm_and_barrier<2 * U + X>();
      read_mma(nk - 3, f1, f0);
      wait_vm_lgkm_and_barrier<U + X>();
      read_mma(nk - 2, f0, f1);
    }
    wait_vm_lgkm_and_barrier<X>();
    read_mma(nk - 1, f1, f0);
    wait_vm_lgkm_and_barrier<0>();
    mma(f1);

    // ---- epilogue: 32 x 32 tile (i, j), register r of lane l holds
    // row 32 i + 8 (r / 4) + 4 g + r % 4, column 32 j + l % 32. The scales are
    // gathered first so their loads overlap, then the products are scaled,
    // rounded and stored. ----
    const float* SA = reinterpret_cast<const float*>(p.sa);
    const float* SB = reinterpret_cast<const float*>(p.sb);
    float cs[NI];
    float st = 1.0f;
    if constexpr (SK == kScaleTensor || MXS) {
      if constexpr (!MXS) st = SA[0] * SB[0];
#pragma unroll
      for (int j = 0; j < NI; ++j) cs[j] = 1.0f;
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        int64_t n = ti.n0 + wn * TN + 32 * j + lrow;
        n = n < N ? n : N - 1;
        cs[j] = SB[(int64_t)ti.e * N + n];
      }
    }
    const int32_t m_lim = (int32_t)(ti.m_end - ti.m0);
    const int32_t n_lim = (int32_t)(N - ti.n0);
    // the row scales of the wave's 128 rows go through LDS and are all loaded
    // before the first store: stores and loads share one counter, so a load
    // issued after stores would make its wait cover the stores too
    if constexpr (SK == kScaleRow) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = ti.m0 + wm * TM + 64 * h + lane;
        m = m < ti.m_end ? m : ti.m_end - 1;
        s_rs[wave][64 * h + lane] = SA[m];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    // direct stores relative to the tile's corner (32-bit offsets: 256 rows *
    // N < 2^31)
    int32_t N32 = (int32_t)N;
    // opaque per tile: keeps the compiler from hoisting every store address
    // out of the tile loop (256 precomputed addresses would spill)
    asm volatile("" : "+s"(N32));
    // this lane's first row and column in the tile, also opaque per tile
    int32_t ml0 = wm * TM + 4 * lg, nl0 = wn * TN + lrow;
    asm volatile("" : "+v"(ml0), "+v"(nl0));
    const int64_t corner = ti.m0 * N + ti.n0;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // rows 32 i + 8 q + 4 g + t, t < 4: the four row scales in one LDS read
        float4 rs4 = make_float4(st, st, st, st);
        if constexpr (SK == kScaleRow)
          rs4 = *reinterpret_cast<const float4*>(&s_rs[wave][32 * i + 8 * q + 4 * lg]);
        const float rsv[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int32_t nl = nl0 + 32 * j;
          if (nl >= n_lim) continue;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int32_t ml = ml0 + 32 * i + 8 * q + t;
            if (ml >= m_lim) continue;
            const uint32_t o = (uint32_t)(ml * N32 + nl);
            const float v = acc[i][j][4 * q + t] * rsv[t] * cs[j];
            if constexpr (OF32)
              (reinterpret_cast<float*>(p.out) + corner)[o] = v;
            else
              (reinterpret_cast<uint16_t*>(p.out) + corner)[o] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  }
}

template <bool AE5, bool BE5, bool OF32>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8_block(GemmParams p) {
  constexpr int BM = 256, BN = 256, BK = 128;
  constexpr int NW = 8, WN = 4;
  constexpr int TM = 128, TN = 64, MI = TM / 16, NI = TN / 16;
  constexpr int SA_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int D = STAGE / 1024 / NW;  // wave-wide 1 KB loads per wave per stage
  static_assert(D == 8, "stage split");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float s_sa[2][BM];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int64_t s_pref[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t N = p.N, K = p.K;
  const int64_t nt = (N + BN - 1) / BN;
  const int64_t nk = K / BK;
  const int64_t nbt = N / 128;
  const uint32_t lds0 = lds_addr(lds);

  const int64_t total = build_tile_prefix<BM, 512>(p, nt, s_off, s_pref);
  int64_t t_begin, t_end, t_step;
  xcd_range(total, t_begin, t_end, t_step);

  // wave w loads 1 KB pieces 8w .. 8w + 7 of a stage: 0-31 are A (8 rows of
  // 128 bytes each), 32-63 are B; lane -> row lane / 8, chunk lane % 8
  const bool loads_a = wave < 4;
  const int q0 = (wave & 3) * D;
  const int ld_row = lane >> 3, ld_pch = lane & 7;

  // fragment read offsets within a stage (16-row block i of A, j of B)
  uint32_t fa_lo[MI], fa_hi[MI], fb_lo[NI], fb_hi[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * TM + 16 * i + lr;
    fa_lo[i] = (uint32_t)(r * BK + 16 * (lg ^ (r & 7)));
    fa_hi[i] = (uint32_t)(r * BK + 16 * ((lg + 4) ^ (r & 7)));
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = wn * TN + 16 * j + lr;
    fb_lo[j] = (uint32_t)(SA_BYTES + r * BK + 16 * (lg ^ (r & 7)));
    fb_hi[j] = (uint32_t)(SA_BYTES + r * BK + 16 * ((lg + 4) ^ (r & 7)));
  }

  for (int64_t t = t_begin; t < t_end; t += t_step) {
    TileInfo ti;
    tile_of<BM, BN>(t, s_off, s_pref, p.E, nt, ti);
    ti.m0 = uniform64(ti.m0);
    ti.m_end = uniform64(ti.m_end);
    ti.n0 = uniform64(ti.n0);
    ti.e = __builtin_amdgcn_readfirstlane(ti.e);
    const int32_t K32 = (int32_t)K;
    const int32_t a_rows = (int32_t)(ti.m_end - ti.m0);
    const int32_t b_rows = (int32_t)(N - ti.n0 < BN ? N - ti.n0 : BN);
    const uint8_t* base = loads_a ? p.a + ti.m0 * K : p.b + ((int64_t)ti.e * N + ti.n0) * K;
    const int32_t rows = loads_a ? a_rows : b_rows;
    uint32_t off[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int r = 8 * (q0 + d) + ld_row;
      const int c = ld_pch ^ (r & 7);
      const int32_t rr = r < rows ? r : rows - 1;  // rows past the expert / N load a valid row
      off[d] = (uint32_t)(rr * K32 + 16 * c);
    }
    const uint32_t opnd_lds = loads_a ? 0u : (uint32_t)SA_BYTES;
    // A-block scales: wave w (and its twin w + 4, same bytes) loads rows
    // 64 (w % 4) .. + 63 of inv_a[m][kb]
    const float* sa_base = reinterpret_cast<const float*>(p.sa) + ti.m0 * nk;
    int32_t sr = 64 * (wave & 3) + lane;
    sr = sr < a_rows ? sr : a_rows - 1;
    const uint32_t sa_off = (uint32_t)(sr * (int32_t)nk) * 4u;
    // this wave's B-block scales: inv_b[e][nb][kb], nb of its 64 columns
    const int64_t nb = (ti.n0 + wn * TN) / 128;
    const float* sb_row = reinterpret_cast<const float*>(p.sb) + ((int64_t)ti.e * nbt + (nb < nbt ? nb : nbt - 1)) * nk;

    auto issue = [&](int64_t k) {
      const uint32_t slot = lds0 + (uint32_t)((k & 1) * STAGE) + opnd_lds + (uint32_t)(q0 * 1024);
      const uint8_t* bk = base + k * BK;
#pragma unroll
      for (int d = 0; d < D; ++d) dma16(bk, off[d], slot + (uint32_t)(d * 1024));
      const uint32_t sl = lds_addr(&s_sa[k & 1][64 * (wave & 3)]);
      asm volatile("global_load_lds_dword %0, %1" ::"v"(sa_off + (uint32_t)(4 * k)),
                   "s"(reinterpret_cast<const uint8_t*>(sa_base)), "{m0}"(sl)
                   : "memory");
    };

    v4f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    issue(0);
    float sbk = sb_row[0];
    for (int64_t k = 0; k < nk; ++k) {
      // stage k landed everywhere and every wave is done with stage k - 1,
      // whose slot the loads of stage k + 1 now fill
      wait_vm_lgkm_and_barrier<0>();
      if (k + 1 < nk) issue(k + 1);
      const float sbk_next = sb_row[k + 1 < nk ? k + 1 : k];
      const uint8_t* st = lds + (k & 1) * STAGE;
      v8i bf[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + fb_lo[j]);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + fb_hi[j]);
        bf[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + fa_lo[i]);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + fa_hi[i]);
        const v8i af = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        // rows 16 i + 4 g + r (r < 4) of this lane's output block
        const float4 sv = *reinterpret_cast<const float4*>(&s_sa[k & 1][wm * TM + 16 * i + 4 * lg]);
        const float f0 = sv.x * sbk, f1 = sv.y * sbk, f2 = sv.z * sbk, f3 = sv.w * sbk;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
          const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], z, AE5 ? 1 : 0, BE5 ? 1 : 0,
                                                                          0, 127, 0, 127);
          // sources stay live until the result is used, so the compiler cannot
          // hand their registers to the destination (not allowed for this MFMA)
          asm volatile("" ::"v"(af), "v"(bf[j]), "v"(pr));
          acc[i][j][0] += pr[0] * f0;
          acc[i][j][1] += pr[1] * f1;
          acc[i][j][2] += pr[2] * f2;
          acc[i][j][3] += pr[3] * f3;
        }
      }
      sbk = sbk_next;
    }
    // every wave is done reading the last stage before the next tile's loads
    // refill its slot
    wait_vm_lgkm_and_barrier<0>();

    // ---- epilogue: lane l holds rows 16 i + 4 g + r, column 16 j + l % 16 ----
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t n = ti.n0 + wn * TN + 16 * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = ti.m0 + wm * TM + 16 * i + 4 * lg + r;
          if (m >= ti.m_end) continue;
          if constexpr (OF32)
            reinterpret_cast<float*>(p.out)[m * N + n] = acc[i][j][r];
          else
            reinterpret_cast<uint16_t*>(p.out)[m * N + n] = f32_to_bf16_rne(acc[i][j][r]);
        }
      }
    }
  }
}

template <bool AE5, bool BE5, int SK, bool OF32>
static hipError_t launch_fast_cfg(const GemmArgs& g) {
  GemmParams p{g.a, g.b, g.sa, g.sb, g.offsets, g.E, g.M, g.N, g.K, g.out};
  constexpr int BM = 256, BN = 256;
  const int64_t nt = (g.N + BN - 1) / BN;
  const int64_t tiles_ub = g.offsets ? ((g.M + BM - 1) / BM + g.E) * nt : ((g.M + BM - 1) / BM) * nt;
  int64_t grid = device_cus();
  if (tiles_ub < grid) grid = tiles_ub;
  if (grid >= kNumXcd) grid -= grid % kNumXcd;
  if (grid < 1) grid = 1;
  if constexpr (SK == kScaleBlock) {
    hipLaunchKernelGGL((k_gemm_fp8_block<AE5, BE5, OF32>), dim3((unsigned)grid), dim3(512), 0, g.stream, p);
  } else if constexpr (SK == kScaleTensor || SK == kScaleRow || SK == kScaleMX) {
    if (g.offsets)
      hipLaunchKernelGGL((k_gemm_fp8_pipe<AE5, BE5, SK, OF32, true>), dim3((unsigned)grid), dim3(256), 0, g.stream, p);
    else
      hipLaunchKernelGGL((k_gemm_fp8_pipe<AE5, BE5, SK, OF32, false>), dim3((unsigned)grid), dim3(256), 0, g.stream, p);
  }
  return hipGetLastError();
}

template <bool AE5, bool BE5>
static hipError_t launch_fast_fmt(const GemmArgs& g) {
  switch (g.scale_kind) {
    case kScaleTensor:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleTensor, true>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleTensor, false>(g);
    case kScaleRow:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleRow, true>(g) : launch_fast_cfg<AE5, BE5, kScaleRow, false>(g);
    case kScaleBlock:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleBlock, true>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleBlock, false>(g);
    default:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleMX, true>(g) : launch_fast_cfg<AE5, BE5, kScaleMX, false>(g);
  }
}

bool gemm_fp8_fast_eligible(const GemmArgs& g) {
  const auto al = [](const void* q, uintptr_t a) { return ((uintptr_t)q % a) == 0; };
  if (g.N > (1 << 22)) return false;  // 32-bit in-tile output offsets
  if (g.K % 128 != 0 || g.K == 0) return false;
  if (g.K > (1 << 23)) return false;  // 32-bit in-tile offsets: 256 rows * K < 2^31
  if (!al(g.a, 16) || !al(g.b, 16)) return false;
  if (g.scale_kind == kScaleMX && (!al(g.sa, 4) || !al(g.sb, 4))) return false;
  return true;
}

hipError_t launch_gemm_fp8_fast(const GemmArgs& g) {
  if (g.a_e5) return g.b_e5 ? launch_fast_fmt<true, true>(g) : launch_fast_fmt<true, false>(g);
  return g.b_e5 ? launch_fast_fmt<false, true>(g) : launch_fast_fmt<false, false>(g);
}

}  // namespace fp8dyn
