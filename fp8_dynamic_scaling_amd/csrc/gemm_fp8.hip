// gemm_fp8.hip -- scaled FP8 GEMMs on gfx950 matrix cores: dense, and the MoE
// grouped form driven by a device offset tensor, with tensorwise, rowwise
// (per-row A x per-expert-column B), 128-blockwise and MX (E8M0) scales.
//
// Contract ("FP8 Training: Quantization, Autograd, Torchao", section 4
// "_scaled_mm layout requirements"): A is [M][K] row-major, B is the
// column-major K x N operand stored as [N][K]; the fp32 accumulation is
// multiplied by the inverse scales. Grouped form ("FP8 training on AMD GPUs
// with TorchTitan and TorchAO", section "Scaling FP8 to MoE Architectures",
// Figure 3): an offset tensor routes row ranges of A to experts and one
// launch covers all experts.
//
// Design for MI355X:
//  - v_mfma_scale_f32_16x16x128_f8f6f4. Operand layout, measured on MI355X: lane
//    l feeds row l % 16; its low 16 bytes are K [16g, 16g + 16) and its high 16
//    bytes are K [64 + 16g, 64 + 16g + 16) of the 128-deep step, g = l / 16;
//    the E8M0 scale of lane l covers row l % 16 and K [32g, 32g + 32). Loading
//    16-byte chunks g and g + 4 of each 128-byte row therefore keeps the
//    instruction's K order equal to memory order, so each lane's scale is the
//    scale of one 32-element group of the tensor. Operand formats (e4m3 / e5m2)
//    are immediates. For the non-MX scalings the hardware scale is 2^0 and the
//    scales are applied in the epilogue (tensor, row) or per 128-K step
//    (blockwise).
//  - Block tile BM x BN x 128 with a wave grid WM x WN; LDS double buffer,
//    16-byte chunks XOR-swizzled by row so fragment reads avoid bank
//    conflicts; one barrier per K step.
//  - Persistent grid of one workgroup per CU. Tiles are numbered expert by
//    expert, and inside an expert in groups of GM m-tiles with n running
//    fastest, so that the 32 workgroups of one XCD (workgroups are dealt to
//    the 8 XCDs round robin) work on a GM x (32/GM) patch of tiles that
//    shares A rows and B columns in that XCD's L2. Each XCD takes a contiguous
//    eighth of the tile list.
//  - Offsets stay on the device: every workgroup reads them into LDS and
//    builds the per-expert tile prefix itself; empty experts own no tiles.
#include "gemm_common.hpp"

namespace fp8dyn {

// EX: full-precision accumulation. Each 16x16x128 FP8 step becomes four
// v_mfma_f32_16x16x32_bf16 on the codes decoded to bf16: bytes [8 q, 8 q + 8)
// of every lane feed instruction q on both operands. MX scales are powers of
// two and are folded into the decode: a lane's low 16 bytes lie in 32-element
// group g / 2 of the 128-deep step and its high 16 bytes in group 2 + g / 2.
template <int BM, int BN, int WM, int WN, bool AE5, bool BE5, int SK, bool OF32, bool EX = false>
__global__ __launch_bounds__(WM* WN * 64, 1) void k_gemm_fp8(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 128;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MI = TM / 16, NI = TN / 16;
  constexpr int A_LOADS = BM * 8 / NT, B_LOADS = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile / thread mismatch");
  static_assert(SK != kScaleBlock || TN <= 128, "block scaling needs a wave's columns in one 128 block");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * BK];
  __shared__ __attribute__((aligned(16))) float lds_sa[2][SK == kScaleBlock ? BM : 1];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int64_t s_pref[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E;
  const int64_t N = p.N, K = p.K;
  const int64_t nt = (N + BN - 1) / BN;
  const int64_t nk = (K + BK - 1) / BK;

  // ---- tile prefix over experts (offsets live in device memory) ----
  const int64_t total = build_tile_prefix<BM, NT>(p, nt, s_off, s_pref);

  // ---- XCD-aware assignment: XCD x owns tiles [x*total/8, (x+1)*total/8) ----
  const int64_t G = gridDim.x;
  const int64_t per_xcd_blocks = G / kNumXcd;
  const int64_t xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  int64_t t_begin, t_end, t_step;
  if (per_xcd_blocks > 0 && G % kNumXcd == 0) {
    t_begin = xcd * total / kNumXcd + slot;
    t_end = (xcd + 1) * total / kNumXcd;
    t_step = per_xcd_blocks;
  } else {
    t_begin = blockIdx.x;
    t_end = total;
    t_step = G;
  }

  const int lr = lane & 15;        // row within a 16-row fragment
  const int lk = lane >> 4;        // which 32-byte K slice of the 128
  for (int64_t t = t_begin; t < t_end; t += t_step) {
    TileInfo ti;
    tile_of<BM, BN>(t, s_off, s_pref, E, nt, ti);
    const uint8_t* A = p.a;
    const uint8_t* B = p.b + (int64_t)ti.e * N * K;

    v4f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    // global -> register staging for one K step
    uint4 ra[A_LOADS], rb[B_LOADS];
    float rsa = 0.0f;
    auto gload = [&](int64_t kt) {
      const int64_t k0 = kt * BK;
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) {
        const int q = tid + NT * j;
        const int r = q >> 3, c = q & 7;
        const int64_t m = ti.m0 + r, k = k0 + 16 * c;
        ra[j] = (m < ti.m_end && k < K) ? *reinterpret_cast<const uint4*>(A + m * K + k) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < B_LOADS; ++j) {
        const int q = tid + NT * j;
        const int r = q >> 3, c = q & 7;
        const int64_t n = ti.n0 + r, k = k0 + 16 * c;
        rb[j] = (n < N && k < K) ? *reinterpret_cast<const uint4*>(B + n * K + k) : make_uint4(0, 0, 0, 0);
      }
      if constexpr (SK == kScaleBlock) {
        if (tid < BM) {
          const int64_t m = ti.m0 + tid;
          rsa = m < ti.m_end ? reinterpret_cast<const float*>(p.sa)[m * nk + kt] : 0.0f;
        }
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) {
        const int q = tid + NT * j;
        const int r = q >> 3, c = q & 7;
        *reinterpret_cast<uint4*>(&lds_a[buf][r * BK + 16 * (c ^ (r & 7))]) = ra[j];
      }
#pragma unroll
      for (int j = 0; j < B_LOADS; ++j) {
        const int q = tid + NT * j;
        const int r = q >> 3, c = q & 7;
        *reinterpret_cast<uint4*>(&lds_b[buf][r * BK + 16 * (c ^ (r & 7))]) = rb[j];
      }
      if constexpr (SK == kScaleBlock) {
        if (tid < BM) lds_sa[buf][tid] = rsa;
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
      const int buf = (int)(kt & 1);
      if (kt + 1 < nk) gload(kt + 1);

      // per-lane MX scales for this K step
      int sa_w[MI], sb_w[NI];
      float sa_x[MI][2], sb_x[NI][2];  // EX: decode scales of the low and high 16 bytes
      if constexpr (EX && SK == kScaleMX) {
        const int64_t kb32 = K / 32;
        const uint8_t* SA = reinterpret_cast<const uint8_t*>(p.sa);
        const uint8_t* SB = reinterpret_cast<const uint8_t*>(p.sb);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t kg = kt * 4 + 2 * h + (lk >> 1);
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int64_t m = ti.m0 + wm * TM + 16 * i + lr;
            const int e = (m < ti.m_end && kg < kb32) ? (int)SA[m * kb32 + kg] : 127;
            sa_x[i][h] = e8m0_to_f32(e);
          }
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int64_t n = ti.n0 + wn * TN + 16 * j + lr;
            const int e = (n < N && kg < kb32) ? (int)SB[((int64_t)ti.e * N + n) * kb32 + kg] : 127;
            sb_x[j][h] = e8m0_to_f32(e);
          }
        }
      }
      if constexpr (SK == kScaleMX && !EX) {
        const int64_t kb32 = K / 32;
        const int64_t kg = kt * 4 + lk;
        const uint8_t* SA = reinterpret_cast<const uint8_t*>(p.sa);
        const uint8_t* SB = reinterpret_cast<const uint8_t*>(p.sb);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int64_t m = ti.m0 + wm * TM + 16 * i + lr;
          sa_w[i] = (m < ti.m_end && kg < kb32) ? (int)SA[m * kb32 + kg] : 127;
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int64_t n = ti.n0 + wn * TN + 16 * j + lr;
          sb_w[j] = (n < N && kg < kb32) ? (int)SB[((int64_t)ti.e * N + n) * kb32 + kg] : 127;
        }
      } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) sa_w[i] = 127;
#pragma unroll
        for (int j = 0; j < NI; ++j) sb_w[j] = 127;
      }

      // B fragments of this wave for the whole K step
      v8i bf[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = wn * TN + 16 * j + lr;
        const uint8_t* base = &lds_b[buf][r * BK];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * (lk ^ (r & 7)));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * ((lk + 4) ^ (r & 7)));
        bf[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      float sbk = 1.0f;
      if constexpr (SK == kScaleBlock) {
        const int64_t nb = (ti.n0 + wn * TN) / 128;
        const int64_t nbt = N / 128;
        sbk = nb < nbt ? reinterpret_cast<const float*>(p.sb)[((int64_t)ti.e * nbt + nb) * nk + kt] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * TM + 16 * i + lr;
        const uint8_t* base = &lds_a[buf][r * BK];
        const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * (lk ^ (r & 7)));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * ((lk + 4) ^ (r & 7)));
        const v8i af = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if constexpr (EX) {
          // decode, two wait states, four BF16 instructions per (i, j)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            v8bf ab[4], bb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if constexpr (SK == kScaleMX) {
                ab[q] = bf16x8_scaled<AE5>(af, q, sa_x[i][q >> 1]);
                bb[q] = bf16x8_scaled<BE5>(bf[j], q, sb_x[j][q >> 1]);
              } else {
                ab[q] = bf16x8<AE5>(af, q);
                bb[q] = bf16x8<BE5>(bf[j], q);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_nop 1" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            v4f t4 = SK == kScaleBlock ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : acc[i][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) t4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[q], bb[q], t4, 0, 0, 0);
            asm volatile("" ::"v"(ab[0]), "v"(ab[1]), "v"(ab[2]), "v"(ab[3]), "v"(bb[0]), "v"(bb[1]), "v"(bb[2]),
                         "v"(bb[3]));
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (SK == kScaleBlock) {
              const float4 s4 = *reinterpret_cast<const float4*>(&lds_sa[buf][wm * TM + 16 * i + 4 * lk]);
              acc[i][j][0] += t4[0] * (s4.x * sbk);
              acc[i][j][1] += t4[1] * (s4.y * sbk);
              acc[i][j][2] += t4[2] * (s4.z * sbk);
              acc[i][j][3] += t4[3] * (s4.w * sbk);
            } else {
              acc[i][j] = t4;
            }
          }
        } else if constexpr (SK == kScaleBlock) {
          const float4 s4 = *reinterpret_cast<const float4*>(&lds_sa[buf][wm * TM + 16 * i + 4 * lk]);
          const float s0 = s4.x * sbk, s1 = s4.y * sbk, s2 = s4.z * sbk, s3 = s4.w * sbk;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
            const v4f tmp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], z, AE5 ? 1 : 0, BE5 ? 1 : 0,
                                                                             0, 127, 0, 127);
            keep_live(af);
            keep_live(bf[j]);
            acc[i][j][0] += tmp[0] * s0;
            acc[i][j][1] += tmp[1] * s1;
            acc[i][j][2] += tmp[2] * s2;
            acc[i][j][3] += tmp[3] * s3;
          }
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j)
          {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], AE5 ? 1 : 0,
                                                                         BE5 ? 1 : 0, 0, sa_w[i], 0, sb_w[j]);
            keep_live(af);
            keep_live(bf[j]);
          }
        }
      }
      if (kt + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: scales and store ----
    const float* SA = reinterpret_cast<const float*>(p.sa);
    const float* SB = reinterpret_cast<const float*>(p.sb);
    float st = 1.0f;
    if constexpr (SK == kScaleTensor) st = SA[0] * SB[0];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t n = ti.n0 + wn * TN + 16 * j + lr;
      if (n >= N) continue;
      float sbn = 1.0f;
      if constexpr (SK == kScaleRow) sbn = SB[(int64_t)ti.e * N + n];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = ti.m0 + wm * TM + 16 * i + 4 * lk + r;
          if (m >= ti.m_end) continue;
          float v = acc[i][j][r];
          if constexpr (SK == kScaleTensor) v *= st;
          if constexpr (SK == kScaleRow) v = v * SA[m] * sbn;
          if constexpr (OF32)
            reinterpret_cast<float*>(p.out)[m * N + n] = v;
          else
            reinterpret_cast<uint16_t*>(p.out)[m * N + n] = f32_to_bf16_rne(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool AE5, bool BE5, int SK, bool OF32, bool EX>
static hipError_t launch_cfg(const GemmArgs& g) {
  GemmParams p{g.a, g.b, g.sa, g.sb, g.offsets, g.E, g.M, g.N, g.K, g.out};
  const int64_t nt = (g.N + BN - 1) / BN;
  const int64_t tiles_ub = g.offsets ? ((g.M + BM - 1) / BM + g.E) * nt : ((g.M + BM - 1) / BM) * nt;
  // fewer tiles than CUs: one workgroup per tile (the kernel then deals tiles
  // by workgroup index); else a persistent grid, a multiple of the XCD count
  int64_t grid = device_cus();
  if (tiles_ub < grid)
    grid = tiles_ub;
  else if (grid >= kNumXcd)
    grid -= grid % kNumXcd;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_gemm_fp8<BM, BN, WM, WN, AE5, BE5, SK, OF32, EX>), dim3((unsigned)grid),
                     dim3(WM * WN * 64), 0, g.stream, p);
  return hipGetLastError();
}

template <bool AE5, bool BE5, int SK, bool OF32>
static hipError_t launch_sk(const GemmArgs& g) {
  if constexpr (SK == kScaleTensor || SK == kScaleRow) {
    if (g.offsets == nullptr && gemm_fp8_small_dense(g.M, g.N)) {
      if (g.exact) return launch_cfg<64, 64, 2, 2, AE5, BE5, SK, OF32, true>(g);
      return launch_cfg<64, 64, 2, 2, AE5, BE5, SK, OF32, false>(g);
    }
  }
  // 64 x 64 per wave: the accumulators, a blockwise step's partial product
  // and the decoded operands of full precision all fit in registers (with
  // 128 x 128 per wave they spilled)
  if (g.exact) return launch_cfg<128, 128, 2, 2, AE5, BE5, SK, OF32, true>(g);
  return launch_cfg<128, 128, 2, 2, AE5, BE5, SK, OF32, false>(g);
}

template <bool AE5, bool BE5>
static hipError_t launch_fmt(const GemmArgs& g) {
  switch (g.scale_kind) {
    case kScaleTensor:
      return g.out_f32 ? launch_sk<AE5, BE5, kScaleTensor, true>(g) : launch_sk<AE5, BE5, kScaleTensor, false>(g);
    case kScaleRow:
      return g.out_f32 ? launch_sk<AE5, BE5, kScaleRow, true>(g) : launch_sk<AE5, BE5, kScaleRow, false>(g);
    case kScaleBlock:
      return g.out_f32 ? launch_sk<AE5, BE5, kScaleBlock, true>(g) : launch_sk<AE5, BE5, kScaleBlock, false>(g);
    default:
      return g.out_f32 ? launch_sk<AE5, BE5, kScaleMX, true>(g) : launch_sk<AE5, BE5, kScaleMX, false>(g);
  }
}

// Small dense outputs: when the 64 x 64 tiles number at most one per CU, the
// 256 x 256 ping-pong kernel would run on a handful of CUs, each streaming a
// whole 256-row panel of A and B; 64 x 64 tiles of four 32 x 32 waves spread
// the same work over up to a CU each. Measured on MI355X with cold caches
// (tensorwise, fp32 out): 256 x 512 x 512 in 9.5 us instead of 17.8 us,
// 1024 x 1024 x 1024 in 13.4 instead of 23.4, 256 x 4096 x 4096 in 34
// instead of 55; from 512 such tiles on the ping-pong kernel is as fast or
// faster (1024 x 2048 x 2048: 34 us either way).
bool gemm_fp8_small_dense(int64_t M, int64_t N) {
  return ((M + 63) / 64) * ((N + 63) / 64) <= (int64_t)device_cus();
}

hipError_t launch_gemm_fp8(const GemmArgs& g) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const bool small = g.offsets == nullptr && !g.b_kpacked &&
                     (g.scale_kind == kScaleTensor || g.scale_kind == kScaleRow) && gemm_fp8_small_dense(g.M, g.N);
  if (!small && gemm_fp8_fast_eligible(g)) return launch_gemm_fp8_fast(g);
  // B is always the e4m3 variant (the API rejects e5m2 B)
  if (g.b_e5) return hipErrorInvalidValue;
  return g.a_e5 ? launch_fmt<true, false>(g) : launch_fmt<false, false>(g);
}

}  // namespace fp8dyn
