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
//  - Tensorwise, rowwise and MX scales: k_gemm_fp8_pp, an 8-wave ping-pong
//    kernel (the header comment there has the details).
//  - 128-blockwise scales: k_gemm_fp8_block, the same ping-pong over 128-deep
//    K blocks with v_mfma_scale_f32_16x16x128_f8f6f4: each 128-deep product
//    goes into a zeroed accumulator and is added to the fp32 result scaled by
//    inv_a[m][kb] * inv_b[nb][kb].
//  - Both: 256 x 256 output tiles walked persistently (one workgroup per CU,
//    XCD-aware order; see gemm_common.hpp); operands go from HBM straight into
//    LDS with global_load_lds_dwordx4 (lane i lands at base + 16 i, measured on
//    MI355X), each lane fetching the 16-byte chunk that belongs at its slot
//    under the row-XOR swizzle; rows past the end of an expert (or of N) load
//    a valid clamped row and their outputs are never stored; K % 128 == 0
//    means no K tail.
#include <type_traits>

#include "gemm_common.hpp"

namespace fp8dyn {

// ---------------------------------------------------------------------------
// Ping-pong kernel (tensorwise, rowwise and MX scales): 256 x 256 tile, 8 waves
// of 128 x 64 in two groups of four, one wave of each group per SIMD. The
// groups alternate between a memory phase (fragment reads of one 64-deep stage
// from LDS, LDS DMA of a later stage) and a compute phase (the 8 MFMAs of the
// stage read before), one s_barrier per phase, so each SIMD's matrix core is
// fed by one wave while the other waits on LDS and HBM. With one wave per
// SIMD doing both in turn (4 waves of 128 x 128), the in-order issue left the
// matrix cores idle whenever that wave waited on LDS: on the Llama3-8B and
// DeepSeek-V3-shaped GEMMs this kernel is 5-17% faster.
//  - v_mfma_scale_f32_32x32x64_f8f6f4, 64-deep K per instruction; measured
//    lane layout: lane l feeds row l % 32, its low 16 bytes are
//    K [16g, 16g + 16) and its high 16 bytes K [32 + 16g, 32 + 16g + 16),
//    g = l / 32, so the instruction's K order is memory order; the scale
//    operand of lane l covers row l % 32, K block g.
//  - LDS stage: 256 rows of A then 256 rows of B, 64 bytes each, 16-byte
//    chunks XOR-swizzled by (row / 4) % 4 so a wave's reads hit distinct
//    banks; the loads are global_load_lds_dwordx4 issued from inline assembly
//    with explicit vmcnt waits (the compiler cannot tell those LDS writes from
//    the fragment reads).
//  - group 0: output rows 0-127, loads the A half of every stage;
//    group 1: rows 128-255, loads the B half; wave w % 4 = column block.
//  - phase 2u: group 0 reads stage u, group 1 computes stage u - 1;
//    phase 2u + 1: group 0 computes stage u, group 1 reads stage u.
//  - ring of 4 stages; in its memory phase for stage u a wave issues its part
//    of stage u + 3 into the slot of stage u - 1 (free once group 1 read it at
//    the end of phase 2u - 1); stage u + 1 has landed (each wave waits for its
//    own loads before the barrier that ends phase 2u + 1).
//  - MX: when K % 512 == 0 and the scale pointers are 16-byte aligned, a row's
//    E8M0 bytes for four stage pairs (512-deep K) come in one 16-byte load per
//    lane with one stage in eight, into an LDS ring of two such blocks;
//    otherwise a stage pair's bytes (one dword per row, 128-deep K) ride in a
//    ring of 4 pairs with each even stage's loads. In an even stage's memory
//    phase each lane reads its rows' dwords of the pair (bytes: K blocks
//    4 p .. 4 p + 3) and shifts them right by 8 g, so byte 0 is its K block
//    of the even stage and byte 2 that of the odd one; the instruction's byte
//    select picks it. A per-stage byte read and mask cost about a sixth of
//    the MX GEMM's time on the Llama-4-style MoE shape.
//  - EX (tensorwise and rowwise scales): full-precision accumulation. The
//    compute phase decodes each 32-byte fragment to bf16 once and runs four
//    v_mfma_f32_32x32x16_bf16 per pair instead of one FP8 instruction: bytes
//    [8 q, 8 q + 8) of every lane feed instruction q, on both operands, so
//    the four instructions together take each K of the stage exactly once.
template <bool AE5, bool BE5, int SK, bool OF32, bool GR, bool PKB, bool EX = false>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8_pp(GemmParams p) {
  constexpr int BM = 256, BN = 256, BK = 64, NS = 4;
  constexpr int TM = 128, TN = 64, MI = TM / 32, NI = TN / 32;
  constexpr int SA_BYTES = BM * BK, STAGE = 2 * SA_BYTES;
  constexpr int DH = 4;  // wave-wide loads per wave per stage: its group's half over 4 waves
  typedef float v16f __attribute__((ext_vector_type(16)));
  constexpr bool MXS = SK == kScaleMX;
  constexpr int X = MXS ? 1 : 0;  // scale loads of an even stage
  static_assert(SK == kScaleTensor || SK == kScaleRow || MXS, "tensorwise, rowwise or MX");
  static_assert(!(EX && MXS), "full-precision accumulation: tensorwise or rowwise scales");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];
  __shared__ int32_t s_off[GR ? kMaxExperts + 1 : 2];
  __shared__ int64_t s_pref[GR ? kMaxExperts + 1 : 2];
  // MX: E8M0 scales, A rows then B rows. Either a ring of 4 stage pairs, one
  // dword per row each, or (K % 512 == 0, 16-byte aligned scales) a ring of 2
  // blocks of 4 pairs, 16 bytes per row each
  __shared__ __attribute__((aligned(16))) uint32_t s_scl[MXS ? 4 * (BM + BN) * 2 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3, wm = grp;
  const int lrow = lane & 31, lg = lane >> 5;
  const int64_t N = p.N, K = p.K;
  const int64_t nt = (N + BN - 1) / BN;
  const int64_t nk = K / BK;
  const uint32_t lds0 = lds_addr(lds);
  // MX scales 16 bytes per row at a time: a dword per row touches a cache
  // line per lane, and the DMA pays per line touched
  const bool scl16 = MXS && nk % 8 == 0 && ((uintptr_t)p.sa % 16) == 0 && ((uintptr_t)p.sb % 16) == 0;

  int64_t total;
  if constexpr (GR) {
    total = build_tile_prefix<BM, 512>(p, nt, s_off, s_pref);
  } else {
    total = ((p.M + BM - 1) / BM) * nt;
  }
  int64_t t_begin, t_end, t_step;
  xcd_range(total, t_begin, t_end, t_step);

  const int ld_row = lane >> 2, ld_pch = lane & 3;
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
    // the column-tile count opaque per tile: the divisions below then form
    // their reciprocal per tile instead of holding it in a register across the
    // K loop (the MX form spilled it, and the reload waited for the previous
    // tile's stores)
    int64_t nt_t = nt;
    asm volatile("" : "+s"(nt_t));
    if constexpr (GR) {
      tile_of<BM, BN>(t, s_off, s_pref, p.E, nt_t, ti);
    } else {
      const int64_t mt = (p.M + BM - 1) / BM;
      const int64_t g = t / (kGroupM * nt_t), rem = t % (kGroupM * nt_t);
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
    // B k-packed: the expert's (or the dense) [N][K] codes as 1 KB chunks of
    // 16 rows x 64 K, chunk (n / 16, k / 64) at ((n / 16) * (K / 64) + k / 64)
    // * 1024, so one
    // stage's load of 16 rows is one contiguous KB (whole cache lines) and the
    // next stage is 1 KB further
    // Grouped k-packed: A pair-interleaved, rows 2i and 2i + 1 sharing a
    // 128-byte line per 64-deep K block (row m, block s at (m / 2) * 2K +
    // s * 128 + (m % 2) * 64), so a 16-row load touches 8 or 9 whole lines
    // however the expert's rows start
    const bool pk = PKB && grp == 1;
    const bool pa = PKB && GR && grp == 0;
    const int64_t m0e = ti.m0 & ~(int64_t)1;
    const uint8_t* base = pa ? p.a + m0e * K
                          : grp == 0 ? p.a + ti.m0 * K
                          : pk       ? p.b + (int64_t)ti.e * N * K
                                     : p.b + ((int64_t)ti.e * N + ti.n0) * K;
    const int64_t sstride = pk ? 1024 : pa ? 128 : BK;
    const int32_t rows = grp == 0 ? a_rows : b_rows;
    uint32_t off[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      const int r = 64 * wn + 16 * d + ld_row;
      const int c = ld_pch ^ ((r >> 2) & 3);
      if (pk) {
        // groups past N (N % 16 == 0) fetch the last group; never stored
        int64_t gi = ti.n0 / 16 + 4 * wn + d;
        gi = gi < N / 16 ? gi : N / 16 - 1;
        off[d] = (uint32_t)(gi * (K / 64) * 1024 + ld_row * 64 + 16 * c);
      } else if (pa) {
        const int32_t rr = r < rows ? r : rows - 1;
        const int64_t m = ti.m0 + rr;
        off[d] = (uint32_t)(((m >> 1) - (m0e >> 1)) * 2 * K + (m & 1) * 64 + 16 * c);
      } else {
        const int32_t rr = r < rows ? r : rows - 1;
        off[d] = (uint32_t)(rr * K32 + 16 * c);
      }
    }
    const uint32_t part_lds = (grp == 0 ? 0u : (uint32_t)SA_BYTES) + (uint32_t)(wn * 4096);
    // MX: this wave's 64 rows (those of its stage loads) of its operand's
    // E8M0 bytes, 4 per row per stage pair (rows past the expert / N fetch a
    // valid row)
    const uint8_t* sc_base = nullptr;
    uint32_t sc_off = 0u, sc_lds = 0u;
    if constexpr (MXS) {
      const int64_t kb32 = K / 32;
      const int r = 64 * wn + lane;
      const int32_t rr = r < rows ? r : rows - 1;
      sc_base = grp == 0 ? reinterpret_cast<const uint8_t*>(p.sa) + ti.m0 * kb32
                         : reinterpret_cast<const uint8_t*>(p.sb) + ((int64_t)ti.e * N + ti.n0) * kb32;
      sc_off = (uint32_t)(rr * (int32_t)kb32);
      sc_lds = (uint32_t)(4 * ((grp == 0 ? 0 : BM) + 64 * wn));
    }

    // the loads of stage s (and, s even, the scales of its pair)
    auto issue = [&](int64_t s) {
      const uint32_t slot = lds0 + (uint32_t)((s & (NS - 1)) * STAGE) + part_lds;
      const uint8_t* bk = base + s * sstride;
#pragma unroll
      for (int d = 0; d < DH; ++d) dma16(bk, off[d], slot + (uint32_t)(d * 1024));
      if constexpr (MXS) {
        const uint32_t o = sc_off + (uint32_t)(2 * s);  // byte 4 (s / 2) of the row
        if (scl16) {
          if ((s & 7) == 0) {  // pairs s / 2 .. s / 2 + 3
            const uint32_t l = lds_addr(&s_scl[((s >> 3) & 1) * 4 * (BM + BN)]) + 4 * sc_lds;
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(o), "s"(sc_base), "{m0}"(l) : "memory");
          }
        } else if ((s & 1) == 0) {
          const uint32_t l = lds_addr(&s_scl[((s >> 1) & 3) * (BM + BN)]) + sc_lds;
          asm volatile("global_load_lds_dword %0, %1" ::"v"(o), "s"(sc_base), "{m0}"(l) : "memory");
        }
      }
    };
    v8i fa[MI], fb[NI];
    int sa[MI], sb[NI];
    // P: the stage's parity where MX reads scales (even stages only), else 0
    auto read = [&](int64_t s, auto par) {
      constexpr int P = decltype(par)::value;
      // slot offset opaque per call: the 12 addresses are formed per read, not
      // precomputed for all 4 slots (48 registers)
      uint32_t so = (uint32_t)((s & (NS - 1)) * STAGE);
      asm volatile("" : "+s"(so));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(lds + so + fa_lo[i]);
        const uint4 hi = *reinterpret_cast<const uint4*>(lds + so + fa_hi[i]);
        fa[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(lds + so + fb_lo[j]);
        const uint4 hi = *reinterpret_cast<const uint4*>(lds + so + fb_hi[j]);
        fb[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if constexpr (MXS && P == 0) {
        // the row's dword of the pair s / 2 (16-byte rows: dword (s / 2) % 4),
        // shifted so this lane's K block 2 s + g sits in byte 0 and 2 s + 2 + g
        // in byte 2
        const uint32_t* dp;
        int rs;  // dwords per row
        if (scl16) {
          dp = &s_scl[((s >> 3) & 1) * 4 * (BM + BN) + (int)((s >> 1) & 3)];
          rs = 4;
        } else {
          dp = &s_scl[((s >> 1) & 3) * (BM + BN)];
          rs = 1;
        }
        const int sh = 8 * lg;
#pragma unroll
        for (int i = 0; i < MI; ++i) sa[i] = (int)(dp[rs * (wm * TM + 32 * i + lrow)] >> sh);
#pragma unroll
        for (int j = 0; j < NI; ++j) sb[j] = (int)(dp[rs * (BM + wn * TN + 32 * j + lrow)] >> sh);
      }
    };
    // MX: the scale operands take their final values here, in the memory
    // phase, so no VALU op on one can sit right before its MFMA. Called after
    // the fragment reads and the DMA issue: the wait these pins imply then
    // costs one LDS round trip for all reads of the phase.
    auto pin_scales = [&]() {
      if constexpr (MXS) {
#pragma unroll
        for (int i = 0; i < MI; ++i) asm volatile("" : "+v"(sa[i]));
#pragma unroll
        for (int j = 0; j < NI; ++j) asm volatile("" : "+v"(sb[j]));
      }
    };
    v16f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // EX: the stage's B fragments and first A row block decoded to bf16 in
    // the memory phase, where the converts overlap the other group's
    // products; pinned there (converts have no side effects and would
    // otherwise sink past the barrier into the compute phase)
    v8bf bd[NI][4], ad[2][4];
    auto predecode = [&]() {
      if constexpr (EX) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) bd[j][q] = bf16x8<BE5>(fb[j], q);
#pragma unroll
        for (int q = 0; q < 4; ++q) ad[0][q] = bf16x8<AE5>(fa[0], q);
        asm volatile("" : "+v"(ad[0][0]), "+v"(ad[0][1]), "+v"(ad[0][2]), "+v"(ad[0][3]));
#pragma unroll
        for (int j = 0; j < NI; ++j)
          asm volatile("" : "+v"(bd[j][0]), "+v"(bd[j][1]), "+v"(bd[j][2]), "+v"(bd[j][3]));
      }
    };
    auto mma = [&](auto par) {
      constexpr int SEL = decltype(par)::value ? 2 : 0;  // MX: byte of the scale operands
      __builtin_amdgcn_s_setprio(1);
      if constexpr (EX) {
        // Each fragment decoded once per stage: both B column blocks and the
        // first A row block in the memory phase (predecode), then every
        // further A row block between the previous one's eight instructions
        // (two converts after each), into the other of two buffers, so the
        // matrix core runs while the converts issue. Every decoded fragment
        // stays live to the end of the phase, so no decode reuses a register
        // an issued instruction may still read.
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int b = i & 1;
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad[b][q], bd[j][q], acc[i][j], 0, 0, 0);
          if (i + 1 < MI) {
#pragma unroll
            for (int q = 0; q < 4; ++q) ad[b ^ 1][q] = bf16x8<AE5>(fa[i + 1], q);
            // 4 NI instructions, 16 converts
#pragma unroll
            for (int k = 0; k < 4 * NI; ++k) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" ::"v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[0][2]), "v"(ad[0][3]), "v"(ad[1][0]), "v"(ad[1][1]),
                     "v"(ad[1][2]), "v"(ad[1][3]));
#pragma unroll
        for (int j = 0; j < NI; ++j)
          asm volatile("" ::"v"(bd[j][0]), "v"(bd[j][1]), "v"(bd[j][2]), "v"(bd[j][3]));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        return;
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          if constexpr (MXS)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AE5 ? 1 : 0,
                                                                        BE5 ? 1 : 0, SEL, sa[i], SEL, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AE5 ? 1 : 0,
                                                                        BE5 ? 1 : 0, 0, 127, 0, 127);
      if constexpr (SEL == 0 && MXS) {
        // an even stage's products stay before the barrier that follows: they
        // have no side effects, and the compiler would otherwise sink them
        // into the odd stage's compute phase (their first use)
        asm volatile(""
                     : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[2][0]),
                       "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1]));
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // this wave's loads of stage u + 1 have landed: those issued after it
    // (stages u + 2 .. min(u + 3, nk - 1); one of two consecutive stages is
    // even and carries a scale load) may stay in flight
    // (16-byte scale rows: a scale load rides with the stages s, s % 8 == 0,
    // so it is among the later ones when u % 8 is 5 or 6; counting it there
    // keeps the wait from taking one of stage u + 2's loads early, which cost
    // about a tenth of the MX GEMM's time on the Llama-4-style MoE shape)
    auto wait_next = [&](int64_t u) {
      if (u + 3 < nk) {
        if (scl16) {
          if ((u & 7) == 5 || (u & 7) == 6) wait_vm_lgkm_and_barrier<2 * DH + 1>();
          else wait_vm_lgkm_and_barrier<2 * DH>();
        } else {
          wait_vm_lgkm_and_barrier<2 * DH + X>();
        }
      } else if (u + 2 < nk) {
        wait_vm_lgkm_and_barrier<DH>();  // stage nk - 1 is odd
      } else {
        wait_vm_lgkm_and_barrier<0>();
      }
    };

    // prologue: stages 0 .. min(nk, 3) - 1; then stage 0 has landed
    issue(0);
    issue(1);
    if (nk >= 4) {
      issue(2);
      if (scl16) wait_vm_lgkm_and_barrier<2 * DH>();
      else wait_vm_lgkm_and_barrier<2 * DH + X>();
    } else {
      wait_vm_lgkm_and_barrier<DH>();
    }
    // both groups run the same loop, group 1 one phase behind: memory phase
    // (reads of stage u, loads of stage u + 3, own loads of stage u + 1
    // landed), barrier, compute phase (MFMAs of stage u), barrier
    if (grp == 1) wait_vm_lgkm_and_barrier<63>();
    auto phase = [&](int64_t u, auto par) {
      read(u, par);
      if (u + 3 < nk) issue(u + 3);
      pin_scales();
      predecode();
      wait_next(u);
      __builtin_amdgcn_sched_barrier(0);
      mma(par);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
    };
    if constexpr (MXS) {
      // stage pairs (nk is even): the odd stage reuses the pair's scale dwords
      for (int64_t u = 0; u < nk; u += 2) {
        phase(u, std::integral_constant<int, 0>{});
        phase(u + 1, std::integral_constant<int, 1>{});
      }
    } else {
      for (int64_t u = 0; u < nk; ++u) phase(u, std::integral_constant<int, 0>{});
    }
    if (grp == 0) asm volatile("s_barrier" ::: "memory");

    // ---- epilogue (the ring is idle: every wave passed the last barrier) ----
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
    float* s_rs = reinterpret_cast<float*>(lds) + wave * TM;
    if constexpr (SK == kScaleRow) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = ti.m0 + wm * TM + 64 * h + lane;
        m = m < ti.m_end ? m : ti.m_end - 1;
        s_rs[64 * h + lane] = SA[m];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    int32_t N32 = (int32_t)N;
    asm volatile("" : "+s"(N32));
    int32_t ml0 = wm * TM + 4 * lg, nl0 = wn * TN + lrow;
    asm volatile("" : "+v"(ml0), "+v"(nl0));
    const int64_t corner = ti.m0 * N + ti.n0;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 rs4 = make_float4(st, st, st, st);
        if constexpr (SK == kScaleRow) rs4 = *reinterpret_cast<const float4*>(&s_rs[32 * i + 8 * q + 4 * lg]);
        const float rsv[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int32_t nl = nl0 + 32 * j;
          if (nl >= n_lim) continue;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            const int32_t ml = ml0 + 32 * i + 8 * q + t2;
            if (ml >= m_lim) continue;
            const uint32_t o = (uint32_t)(ml * N32 + nl);
            const float v = acc[i][j][4 * q + t2] * rsv[t2] * cs[j];
            if constexpr (OF32)
              (reinterpret_cast<float*>(p.out) + corner)[o] = v;
            else
              (reinterpret_cast<uint16_t*>(p.out) + corner)[o] = f32_to_bf16_rne(v);
          }
        }
      }
    }
    // the next tile's first loads refill slot 0, which holds the row scales
    if constexpr (SK == kScaleRow) __syncthreads();
  }
}


// ---------------------------------------------------------------------------
// Kernel for 128-blockwise scales. Every 128-deep partial product carries its
// own scale inv_a[m][kb] * inv_b[nb][kb], so partial sums cannot stay in the
// matrix-core accumulator: each 128-deep product of a 32 x 32 block is two
// v_mfma_scale_f32_32x32x64_f8f6f4 into a fresh register, and an fp32 FMA
// per output adds it, scaled, into the result.
//  - Transposed products: the instruction's rows are B rows (n), its columns
//    A rows (m), so a lane holds one m and 16 n of each block. The A-block
//    scale is then one value per lane and block, and the B-block scale one
//    per wave (its 64 columns lie in one 128-column block): a single factor
//    per lane scales a whole product. Measured on MI355X, this instruction
//    sustains about 94% of the nominal FP8 rate back to back; the 16 x 16 x
//    128 one, about 75%.
//  - 256 x 256 tile, 8 waves of 128 m x 64 n, two per SIMD, both computing:
//    while one wave runs the FMAs of a product or waits on LDS, the other
//    keeps the matrix core busy. (A ping-pong split, one wave computing while
//    the other reads, measured slower here: the FMAs then stall the only
//    wave that could feed the matrix core, and every phase boundary idles
//    it.) Per K block a wave runs 8 products (4 row blocks x 2 column
//    blocks); the FMAs of product n follow the first instruction of product
//    n + 1, and each row block's A fragments are read while the previous row
//    block's products run.
//  - LDS: a ring of two 128-deep K blocks, each 256 rows of A then 256 rows
//    of B, 128 bytes per row, so every DMA lane group fetches whole cache
//    lines; 16-byte chunks XOR-swizzled by (row / 2) % 8: two rows share a
//    line of the 64 four-byte banks, and a 16-lane group of a 16-byte read
//    (16 consecutive rows) then hits 16 distinct bank quads. Lane l's 32-byte
//    operand for K half kh of a block is chunks 4 kh + g and 4 kh + 2 + g of
//    row l % 32, g = l / 32 (the instruction's measured operand layout).
//  - Two barriers per K block kb. After the first (kb has landed, every wave
//    is done with kb - 1), waves 0-3 load A of kb + 1 into kb - 1's slot.
//    After the second (every wave holds its B fragments of kb), waves 4-7
//    load B of kb + 2 into the B half of kb's slot: B, mostly fetched from
//    HBM (a B tile serves few row tiles), gets about 1.75 K blocks to land,
//    A (row tiles are shared by the whole tile row, mostly L2 hits) one.
//  - Scales (SC4: K % 512 == 0 and 16-byte aligned scale arrays): one
//    16-byte load per row brings the A-block scales of four K blocks, and one
//    per column block those of B. Otherwise one 4-byte load per row per K
//    block; that form touches a cache line per lane for 4 bytes.
template <bool AE5, bool BE5, bool OF32, bool SC4>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8_block(GemmParams p) {
  constexpr int BM = 256, BN = 256, BK = 128;
  constexpr int TM = 128, TN = 64;
  constexpr int SA_BYTES = BM * BK, STAGE = 2 * SA_BYTES;
  constexpr int D = SA_BYTES / 1024 / 4;  // wave-wide 1 KB loads per wave per K block
  typedef float v16f __attribute__((ext_vector_type(16)));
  static_assert(D == 8, "stage split");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];
  // A-block scales of four K blocks: SC4 [slot][row][kb % 4], else
  // [slot][kb % 4][row]; slot (kb / 4) % 2
  __shared__ __attribute__((aligned(16))) float s_sa[2][4 * BM];
  // B-block scales of four K blocks per 64-column block: [slot][wn][kb % 4]
  __shared__ __attribute__((aligned(16))) float s_sb[2][4][4];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int64_t s_pref[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3;
  const int lrow = lane & 31, g = lane >> 5;
  const int64_t N = p.N, K = p.K;
  const int64_t nt = (N + BN - 1) / BN;
  const int64_t nk = K / BK;
  const int64_t nbt = N / 128;
  const uint32_t lds0 = lds_addr(lds);

  const int64_t total = build_tile_prefix<BM, 512>(p, nt, s_off, s_pref);
  int64_t t_begin, t_end, t_step;
  xcd_range(total, t_begin, t_end, t_step);

  // fragment byte offsets within a slot, lane part: row lrow, chunk
  // (4 kh + 2 s + g) ^ ((row / 2) % 8) for K half kh, low (s = 0) or high 16
  // bytes; row block i of A starts 16384 grp + 4096 i further, column block
  // j of B SA_BYTES + 8192 wn + 4096 j further
  uint32_t fo[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      fo[kh][s] = (uint32_t)(lrow * BK) + 16u * ((uint32_t)(4 * kh + 2 * s + g) ^ (uint32_t)((lrow >> 1) & 7));
  const uint32_t a_part = (uint32_t)(grp * TM * BK);
  const uint32_t b_part = (uint32_t)(SA_BYTES + wn * TN * BK);

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
    // waves 0-3 load A rows 64 wn .. 64 wn + 63 of the tile, waves 4-7 those
    // B rows; rows past the expert (or N) load a valid row, never stored
    const uint8_t* base = grp == 0 ? p.a + ti.m0 * K : p.b + ((int64_t)ti.e * N + ti.n0) * K;
    const int32_t rows = grp == 0 ? a_rows : b_rows;
    const uint32_t part = (grp == 0 ? 0u : (uint32_t)SA_BYTES) + (uint32_t)(wn * D * 1024);
    // scales: waves 0-3 those of A rows 64 wn + lane, waves 4-7 (one lane)
    // those of B column block (n0 + 64 wn) / 128
    const uint8_t* sa_bytes = reinterpret_cast<const uint8_t*>(reinterpret_cast<const float*>(p.sa) + ti.m0 * nk);
    int64_t nb = (ti.n0 + wn * TN) / 128;
    nb = nb < nbt ? nb : nbt - 1;
    const uint8_t* sb_bytes =
        reinterpret_cast<const uint8_t*>(reinterpret_cast<const float*>(p.sb) + ((int64_t)ti.e * nbt + nb) * nk);

    // K block kb starts a scale load: SC4 one in four, else every one
    auto has_scale = [&](int64_t kb) { return SC4 ? (kb & 3) == 0 : true; };
    // the offsets are formed per call from opaque inputs: held across the
    // K loop they would take 16 registers the loop does not have
    auto issue_ops = [&](int64_t kb) {
      const uint32_t slot = lds0 + (uint32_t)((kb & 1) * STAGE) + part;
      const uint8_t* bk = base + kb * BK;
      // lane: row 8 d + lane / 8 of the wave's 64, LDS chunk lane % 8, which
      // holds chunk (lane % 8) ^ ((row / 2) % 8) of the row; (8 d + lane / 8)
      // / 2 % 8 is lane / 16 + 4 (d % 2)
      uint32_t l = (uint32_t)lane;
      asm volatile("" : "+v"(l));
      const int32_t r0 = 64 * wn + (int32_t)(l >> 3);
      const uint32_t cb0 = 16u * ((l & 7u) ^ (l >> 4));
      const uint32_t cb1 = 16u * ((l & 7u) ^ ((l >> 4) + 4u));
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int32_t r = r0 + 8 * d;
        const int32_t rr = r < rows ? r : rows - 1;
        dma16(bk, (uint32_t)rr * (uint32_t)K32 + ((d & 1) ? cb1 : cb0), slot + (uint32_t)(d * 1024));
      }
    };
    auto issue_sa = [&](int64_t kb) {
      uint32_t l = (uint32_t)lane;
      asm volatile("" : "+v"(l));
      int32_t sr = 64 * wn + (int32_t)l;
      sr = sr < a_rows ? sr : a_rows - 1;
      const uint32_t o = (uint32_t)(sr * (int32_t)nk + (int32_t)kb) * 4u;
      if constexpr (SC4) {
        const uint32_t l = lds_addr(&s_sa[(kb >> 2) & 1][4 * 64 * wn]);
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(o), "s"(sa_bytes), "{m0}"(l) : "memory");
      } else {
        const uint32_t l = lds_addr(&s_sa[(kb >> 2) & 1][(kb & 3) * BM + 64 * wn]);
        asm volatile("global_load_lds_dword %0, %1" ::"v"(o), "s"(sa_bytes), "{m0}"(l) : "memory");
      }
    };
    auto issue_sb = [&](int64_t kb) {
      const uint32_t o = (uint32_t)(4 * kb);
      if (lane == 0) {
        if constexpr (SC4) {
          const uint32_t l = lds_addr(&s_sb[(kb >> 2) & 1][wn][0]);
          asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(o), "s"(sb_bytes), "{m0}"(l) : "memory");
        } else {
          const uint32_t l = lds_addr(&s_sb[(kb >> 2) & 1][wn][kb & 3]);
          asm volatile("global_load_lds_dword %0, %1" ::"v"(o), "s"(sb_bytes), "{m0}"(l) : "memory");
        }
      }
    };

    auto frag = [&](uint32_t o0, uint32_t o1) {
      const uint4 lo = *reinterpret_cast<const uint4*>(lds + o0);
      const uint4 hi = *reinterpret_cast<const uint4*>(lds + o1);
      return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: K block 0 (both operands) and B of K block 1
    issue_ops(0);
    if (grp == 0) {
      issue_sa(0);
    } else {
      issue_sb(0);
      if (nk > 1) {
        issue_ops(1);
        if (has_scale(1)) issue_sb(1);
      }
    }
    for (int64_t kb = 0; kb < nk; ++kb) {
      // K block kb has landed (each wave waits for its own loads of kb, the
      // barrier for everyone's); every wave is done with kb - 1
      if (grp == 0 || kb + 1 >= nk) {
        wait_vm_lgkm_and_barrier<0>();
      } else if (has_scale(kb + 1)) {
        // B of kb + 1 (issued in the prologue or after the second barrier of
        // kb - 1) may stay in flight
        wait_vm_lgkm_and_barrier<D + 1>();
      } else {
        wait_vm_lgkm_and_barrier<D>();
      }
      if (grp == 0 && kb + 1 < nk) {
        issue_ops(kb + 1);
        if (has_scale(kb + 1)) issue_sa(kb + 1);
      }
      uint32_t so = (uint32_t)((kb & 1) * STAGE);
      asm volatile("" : "+s"(so));
      const int q = (int)(kb & 3);
      const float* ss = &s_sa[(kb >> 2) & 1][0];
      v8i fb[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          fb[j][kh] = frag(so + b_part + fo[kh][0] + 4096 * j, so + b_part + fo[kh][1] + 4096 * j);
      const float sbk = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_sb[(kb >> 2) & 1][wn][q])));
      // A fragments and factor of row block i, double-buffered
      v8i fa[2][2];
      float f[2];
      auto read_a = [&](int i) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          fa[i & 1][kh] = frag(so + a_part + fo[kh][0] + 4096 * i, so + a_part + fo[kh][1] + 4096 * i);
        const int m = grp * TM + 32 * i + lrow;
        f[i & 1] = SC4 ? ss[4 * m + q] : ss[q * BM + m];
      };
      read_a(0);

      // product n = (row block n / 2, column block n % 2): two instructions
      // (K halves) into P[n % 2]; the FMAs of product n - 1 run between them
      const v16f z = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      v16f P[2];
      auto scale_add = [&](int n) {
        const int i = n >> 1, j = n & 1;
        const float fs = f[i & 1] * sbk;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(P[n & 1][e], fs, acc[i][j][e]);
      };
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int i = n >> 1, j = n & 1;
        __builtin_amdgcn_sched_barrier(0);
        P[n & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][0], fa[i & 1][0], z, BE5 ? 1 : 0,
                                                                   AE5 ? 1 : 0, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        if (n > 0) scale_add(n - 1);
        __builtin_amdgcn_sched_barrier(0);
        P[n & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][1], fa[i & 1][1], P[n & 1], BE5 ? 1 : 0,
                                                                   AE5 ? 1 : 0, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        // row block i's A fragments stay live up to its last instruction (no
        // product may take their registers); i + 1's are read while i runs
        if (j == 1) asm volatile("" ::"v"(fa[i & 1][0]), "v"(fa[i & 1][1]));
        if (j == 0 && i + 1 < 4) read_a(i + 1);
        if (n == 1) {
          // every wave holds its B fragments of kb (waited for before the
          // first product): waves 4-7 refill the B half of kb's slot with
          // kb + 2. The products issued so far keep the matrix core busy
          // through the barrier.
          asm volatile("" : "+v"(P[1]), "+v"(acc[0][0]));
          asm volatile("s_barrier" ::: "memory");
          if (grp == 1 && kb + 2 < nk) {
            issue_ops(kb + 2);
            if (has_scale(kb + 2)) issue_sb(kb + 2);
          }
        }
      }
      scale_add(7);
      // the K block's results and B fragments are pinned before the next
      // barrier: the products and FMAs have no side effects and would
      // otherwise be sunk past it
      asm volatile(""
                   : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[2][0]),
                     "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1])
                   : "v"(fb[0][0]), "v"(fb[0][1]), "v"(fb[1][0]), "v"(fb[1][1]));
    }

    // ---- epilogue: element 4 q + u of block (i, j) is row m = 32 i + lrow,
    // column n = 32 j + 8 q + 4 g + u of the wave's part; the four u are
    // adjacent in memory ----
    const int32_t m_lim = (int32_t)(ti.m_end - ti.m0);
    const int32_t n_lim = (int32_t)(N - ti.n0);
    int32_t N32 = (int32_t)N;
    asm volatile("" : "+s"(N32));
    const int64_t corner = ti.m0 * N + ti.n0;
    // lane offsets formed here, per tile: hoisted out of the tile loop they
    // would stay live through the K loop, be spilled, and each reload would
    // wait behind every store issued before it
    int32_t ml0 = grp * TM + lrow, nl0 = wn * TN + 4 * g;
    asm volatile("" : "+v"(ml0), "+v"(nl0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t ml = ml0 + 32 * i;
      if (ml >= m_lim) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t nl = nl0 + 32 * j + 8 * q;
          if (nl >= n_lim) continue;  // n_lim is a multiple of 128: the four are valid together
          const uint32_t o = (uint32_t)(ml * N32 + nl);
          const v16f& a = acc[i][j];
          if constexpr (OF32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + corner + o) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          } else {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(a[4 * q]) | ((uint32_t)f32_to_bf16_rne(a[4 * q + 1]) << 16);
            const uint32_t hi =
                (uint32_t)f32_to_bf16_rne(a[4 * q + 2]) | ((uint32_t)f32_to_bf16_rne(a[4 * q + 3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + corner + o) = make_uint2(lo, hi);
          }
        }
      }
    }
    // every wave is done with the last K block's slot, and the next tile's
    // loads count their own completions: stores complete first
    wait_vm_lgkm_and_barrier<0>();
  }
}

template <bool AE5, bool BE5, int SK, bool OF32, bool EX>
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
    // scales of four K blocks per 16-byte load
    const bool sc4 = (g.K / 128) % 4 == 0 && ((uintptr_t)g.sa % 16) == 0 && ((uintptr_t)g.sb % 16) == 0;
    if (sc4)
      hipLaunchKernelGGL((k_gemm_fp8_block<AE5, BE5, OF32, true>), dim3((unsigned)grid), dim3(512), 0, g.stream, p);
    else
      hipLaunchKernelGGL((k_gemm_fp8_block<AE5, BE5, OF32, false>), dim3((unsigned)grid), dim3(512), 0, g.stream, p);
  } else {
    if (g.offsets && g.b_kpacked)
      hipLaunchKernelGGL((k_gemm_fp8_pp<AE5, BE5, SK, OF32, true, true, EX>), dim3((unsigned)grid), dim3(512), 0,
                         g.stream, p);
    else if (g.offsets)
      hipLaunchKernelGGL((k_gemm_fp8_pp<AE5, BE5, SK, OF32, true, false, EX>), dim3((unsigned)grid), dim3(512), 0,
                         g.stream, p);
    else if (g.b_kpacked)
      hipLaunchKernelGGL((k_gemm_fp8_pp<AE5, BE5, SK, OF32, false, true, EX>), dim3((unsigned)grid), dim3(512), 0,
                         g.stream, p);
    else
      hipLaunchKernelGGL((k_gemm_fp8_pp<AE5, BE5, SK, OF32, false, false, EX>), dim3((unsigned)grid), dim3(512), 0,
                         g.stream, p);
  }
  return hipGetLastError();
}

template <bool AE5, bool BE5>
static hipError_t launch_fast_fmt(const GemmArgs& g) {
  switch (g.scale_kind) {
    case kScaleTensor:
      if (g.exact)
        return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleTensor, true, true>(g)
                         : launch_fast_cfg<AE5, BE5, kScaleTensor, false, true>(g);
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleTensor, true, false>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleTensor, false, false>(g);
    case kScaleRow:
      if (g.exact)
        return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleRow, true, true>(g)
                         : launch_fast_cfg<AE5, BE5, kScaleRow, false, true>(g);
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleRow, true, false>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleRow, false, false>(g);
    case kScaleBlock:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleBlock, true, false>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleBlock, false, false>(g);
    default:
      return g.out_f32 ? launch_fast_cfg<AE5, BE5, kScaleMX, true, false>(g)
                       : launch_fast_cfg<AE5, BE5, kScaleMX, false, false>(g);
  }
}

bool gemm_fp8_fast_eligible(const GemmArgs& g) {
  const auto al = [](const void* q, uintptr_t a) { return ((uintptr_t)q % a) == 0; };
  // full precision: the ping-pong kernel's tensorwise and rowwise forms
  if (g.exact && g.scale_kind != kScaleTensor && g.scale_kind != kScaleRow) return false;
  if (g.N > (1 << 22)) return false;  // 32-bit in-tile output offsets
  if (g.K % 128 != 0 || g.K == 0) return false;
  if (g.K > (1 << 23)) return false;  // 32-bit in-tile offsets: 256 rows * K < 2^31
  if (!al(g.a, 16) || !al(g.b, 16)) return false;
  if ((g.scale_kind == kScaleMX || g.scale_kind == kScaleBlock) && (!al(g.sa, 4) || !al(g.sb, 4))) return false;
  // the blockwise kernel stores 4 adjacent outputs per lane (8 or 16 bytes)
  if (g.scale_kind == kScaleBlock && !al(g.out, 16)) return false;
  return true;
}

hipError_t launch_gemm_fp8_fast(const GemmArgs& g) {
  // B is always the e4m3 variant (the API rejects e5m2 B)
  if (g.b_e5) return hipErrorInvalidValue;
  return g.a_e5 ? launch_fast_fmt<true, false>(g) : launch_fast_fmt<false, false>(g);
}

}  // namespace fp8dyn
