// linear.hip -- one Linear layer, forward and backward, as stream-ordered
// launches of the quantization kernels and GEMMs ("FP8 Training:
// Quantization, Autograd, Torchao", section 6: three GEMMs per layer;
// "FP8 training on AMD GPUs with TorchTitan and TorchAO", Figure 1 caption:
// the rowwise recipe keeps the weight-gradient GEMM in BF16).
//
//   forward   y  = (qx * inv_x) (qw * inv_w)^T    qx, qw: e4m3
//   backward  gx = (qg * inv_g) (qwT * inv_wc)^T  qg: e5m2 of gy, qwT: e4m3 of w
//                                                 written transposed [K][N]
//                                                 (rowwise: per column of w)
//             gw = (qgT * inv_g) (qxT * inv_x)^T  tensorwise: all-FP8, qgT and
//                                                 qxT transposed [N][M], [K][M]
//                                                 from one cast launch with qg
//             gw = gy^T x                         rowwise: bf16 matrix cores
// Every FP8 operand is produced directly in the layout its GEMM reads: no
// transposed copies ("FP8 training on AMD GPUs with TorchTitan and TorchAO",
// Level 1). In the rowwise recipe the weight operands are written k-packed
// (1 KB chunks of 16 rows x 64 K, the layout the GEMM's LDS loads read as
// whole cache lines) when the shapes allow it; the bytes are the same codes.
// Accumulation follows "FP8 Training: Quantization, Autograd, Torchao",
// section 5: both backward GEMMs use full precision; the forward takes the
// caller's choice (the pages' recipe: fast accumulation).
#include <cmath>

#include "../../include/fp8dyn.h"
#include "internal.hpp"

using namespace fp8dyn;

namespace {

struct Bump {
  uint8_t* base;
  size_t off = 0;
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  }
};

struct FwdLayout {
  void *qx, *qw, *sx, *ix, *sw, *iw, *wsx, *wsw, *part;
};
FwdLayout fwd_layout(uint8_t* ws, int64_t M, int64_t N, int64_t K, fp8_recipe r, size_t* total) {
  Bump b{ws};
  FwdLayout L;
  const bool tw = r == FP8_RECIPE_TENSORWISE;
  L.qx = b.take((size_t)(M * K));
  L.qw = b.take((size_t)(N * K));
  L.sx = b.take(4 * (tw ? 1 : (size_t)M));
  L.ix = b.take(4 * (tw ? 1 : (size_t)M));
  L.sw = b.take(4 * (tw ? 1 : (size_t)N));
  L.iw = b.take(4 * (tw ? 1 : (size_t)N));
  L.wsx = b.take(256);
  L.wsw = b.take(256);
  // tensorwise: per-workgroup amax partials of x and w
  L.part = tw ? b.take(4 * 2 * (size_t)kPairMaxAmaxBlocks) : nullptr;
  *total = b.off;
  return L;
}

struct BwdLayout {
  void *qg, *sg, *ig, *qwt, *swc, *iwc, *wsg, *wscol, *qgt, *qxt, *sx, *ix;
};
BwdLayout bwd_layout(uint8_t* ws, int64_t M, int64_t N, int64_t K, fp8_recipe r, size_t* total) {
  Bump b{ws};
  BwdLayout L;
  const bool tw = r == FP8_RECIPE_TENSORWISE;
  L.qg = b.take((size_t)(M * N));
  L.sg = b.take(4 * (tw ? 1 : (size_t)M));
  L.ig = b.take(4 * (tw ? 1 : (size_t)M));
  L.qwt = b.take((size_t)(K * N));
  L.swc = b.take(4 * (tw ? 1 : (size_t)K));
  L.iwc = b.take(4 * (tw ? 1 : (size_t)K));
  L.wsg = b.take(256);
  size_t colws = tw ? 256 : quant_col_ws_bytes(1, N, K);
  L.wscol = b.take(colws > 0 ? colws : 256);
  // tensorwise: transposed gy and x for the FP8 grad-weight GEMM
  L.qgt = tw ? b.take((size_t)(N * M)) : nullptr;
  L.qxt = tw ? b.take((size_t)(K * M)) : nullptr;
  L.sx = tw ? b.take(4) : nullptr;
  L.ix = tw ? b.take(4) : nullptr;
  *total = b.off;
  return L;
}

fp8_status as_status(hipError_t e) {
  if (e == hipSuccess) return FP8_OK;
  return FP8_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shapes whose rowwise weight operands go k-packed: the forward's w [N][K]
// (fp8_quant_row_kpacked + fp8_scaled_mm_kpacked), the backward's w^T [K][N]
// (fp8_quant_col_kpacked + fp8_scaled_mm_kpacked, contraction over N). Outputs
// small enough for the 64 x 64 tile GEMM ([M][N] forward, [M][K] grad-input)
// keep the row-major operands, which that GEMM reads.
bool fwd_kpacked(int64_t M, int64_t N, int64_t K) {
  return K > 0 && N % 16 == 0 && K % 128 == 0 && K <= 16384 && N * K < ((int64_t)1 << 31) &&
         !gemm_fp8_small_dense(M, N);
}
bool bwd_kpacked(int64_t M, int64_t N, int64_t K) {
  return N % 128 == 0 && K % 16 == 0 && N * K < ((int64_t)1 << 30) && !gemm_fp8_small_dense(M, K);
}

bool bad_eps(double eps) { return !(std::isfinite(eps) && eps > 0.0); }

}  // namespace

extern "C" {

size_t fp8_linear_ws_bytes(int64_t M, int64_t N, int64_t K, fp8_recipe recipe) {
  if (M < 0 || N < 0 || K < 0) return 0;
  size_t f = 0, b = 0;
  fwd_layout(nullptr, M, N, K, recipe, &f);
  bwd_layout(nullptr, M, N, K, recipe, &b);
  return f > b ? f : b;
}

fp8_status fp8_linear_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K, fp8_recipe recipe,
                          double eps, fp8_out out_type, int use_fast_accum, void* y, void* ws, size_t ws_bytes,
                          void* stream) {
  if (recipe != FP8_RECIPE_TENSORWISE && recipe != FP8_RECIPE_ROWWISE_BF16_WGRAD) return FP8_ERR_INVALID_ARGUMENT;
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (M == 0 || N == 0) return FP8_OK;
  if (!y || (K > 0 && (!x || !w))) return FP8_ERR_INVALID_ARGUMENT;
  if (K % 16 != 0) return FP8_ERR_ALIGNMENT;
  size_t need = 0;
  fwd_layout(nullptr, M, N, K, recipe, &need);
  if (!ws || ws_bytes < need) return FP8_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return FP8_ERR_ALIGNMENT;
  FwdLayout L = fwd_layout((uint8_t*)ws, M, N, K, recipe, &need);
  const bool tw = recipe == FP8_RECIPE_TENSORWISE;
  fp8_status st;
  if (tw && K > 0) {
    // x and w in one amax launch and one cast launch
    if (bad_eps(eps)) return FP8_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(w, 16)) return FP8_ERR_ALIGNMENT;
    fp8_format e4f, e5f;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_DEVICE;
    if ((st = fp8_probe(dev, &e4f, &e5f)) != FP8_OK) return st;
    const TPairSpec jobs[2] = {{x, M * K, (uint8_t*)L.qx, (float*)L.sx, (float*)L.ix},
                               {w, N * K, (uint8_t*)L.qw, (float*)L.sw, (float*)L.iw}};
    if ((st = as_status(launch_quant_tensor_pair(jobs, false, fp8_format_max(e4f), eps, (float*)L.part,
                                                 (hipStream_t)stream))) != FP8_OK)
      return st;
  } else if (tw) {
    // no contraction terms: empty-tensor scales, then the zero output
    if ((st = fp8_quant_tensor(x, 0, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qx, (float*)L.sx, (float*)L.ix, L.wsx, 256,
                               stream)) != FP8_OK)
      return st;
    if ((st = fp8_quant_tensor(w, 0, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qw, (float*)L.sw, (float*)L.iw, L.wsw, 256,
                               stream)) != FP8_OK)
      return st;
  } else {
    if ((st = fp8_quant_row(x, 1, M, K, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qx, (float*)L.sx, (float*)L.ix, stream)) !=
        FP8_OK)
      return st;
    if (fwd_kpacked(M, N, K)) {
      if ((st = fp8_quant_row_kpacked(w, 1, N, K, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qw, (float*)L.sw, (float*)L.iw,
                                      stream)) != FP8_OK)
        return st;
      return fp8_scaled_mm_kpacked((const uint8_t*)L.qx, FP8_E4M3_NATIVE, (const uint8_t*)L.qw, FP8_E4M3_NATIVE,
                                   FP8_SCALE_ROW, (const float*)L.ix, (const float*)L.iw, M, N, K, out_type, y,
                                   use_fast_accum, stream);
    }
    if ((st = fp8_quant_row(w, 1, N, K, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qw, (float*)L.sw, (float*)L.iw, stream)) !=
        FP8_OK)
      return st;
  }
  return fp8_scaled_mm((const uint8_t*)L.qx, FP8_E4M3_NATIVE, (const uint8_t*)L.qw, FP8_E4M3_NATIVE,
                       tw ? FP8_SCALE_TENSOR : FP8_SCALE_ROW, (const float*)L.ix, (const float*)L.iw, M, N, K, out_type,
                       y, use_fast_accum, stream);
}

fp8_status fp8_linear_bwd(const uint16_t* gy, const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                          fp8_recipe recipe, double eps, uint16_t* gx, uint16_t* gw, void* ws, size_t ws_bytes,
                          void* stream) {
  if (recipe != FP8_RECIPE_TENSORWISE && recipe != FP8_RECIPE_ROWWISE_BF16_WGRAD) return FP8_ERR_INVALID_ARGUMENT;
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (K == 0) return FP8_OK;  // both gradients are empty
  // the empty sums: grad-weight over no rows, grad-input over no outputs
  if (M == 0 || N == 0) {
    uint16_t* z = M == 0 ? gw : gx;
    const int64_t n = (M == 0 ? N : M) * K;
    if (n == 0) return FP8_OK;
    if (!z) return FP8_ERR_INVALID_ARGUMENT;
    if (!aligned(z, 4)) return FP8_ERR_ALIGNMENT;
    return as_status(launch_zero_fill(z, n * 2, (hipStream_t)stream));
  }
  if (!gy || !x || !w || !gx || !gw || bad_eps(eps)) return FP8_ERR_INVALID_ARGUMENT;
  if (N % 16 != 0 || K % 16 != 0) return FP8_ERR_ALIGNMENT;
  size_t need = 0;
  bwd_layout(nullptr, M, N, K, recipe, &need);
  if (!ws || ws_bytes < need) return FP8_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return FP8_ERR_ALIGNMENT;
  BwdLayout L = bwd_layout((uint8_t*)ws, M, N, K, recipe, &need);
  const bool tw = recipe == FP8_RECIPE_TENSORWISE;
  fp8_status st;
  if (tw) {
    // the transposed casts and the grad-weight GEMM contract over m
    if (M % 16 != 0) return FP8_ERR_ALIGNMENT;
    const int64_t lim = (int64_t)1 << 30;
    if (M * N >= lim || M * K >= lim || N * K >= lim) return FP8_ERR_UNSUPPORTED;
    fp8_format e4f, e5f;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_DEVICE;
    if ((st = fp8_probe(dev, &e4f, &e5f)) != FP8_OK) return st;
    // one amax launch and one cast launch for all three tensors: gy in both
    // layouts (e5m2), x transposed [K][M] and w transposed [K][N] (e4m3)
    const TJobSpec jobs[3] = {
        {gy, M, N, true, fp8_format_max(e5f), (uint8_t*)L.qg, (uint8_t*)L.qgt, (float*)L.sg, (float*)L.ig},
        {x, M, K, false, fp8_format_max(e4f), nullptr, (uint8_t*)L.qxt, (float*)L.sx, (float*)L.ix},
        {w, N, K, false, fp8_format_max(e4f), nullptr, (uint8_t*)L.qwt, (float*)L.swc, (float*)L.iwc}};
    if ((st = as_status(launch_quant_tensor_multi_t(jobs, 3, eps, (uint32_t*)L.wsg, (hipStream_t)stream))) != FP8_OK)
      return st;
  } else {
    if ((st = fp8_quant_row(gy, 1, M, N, FP8_E5M2_NATIVE, eps, (uint8_t*)L.qg, (float*)L.sg, (float*)L.ig, stream)) !=
        FP8_OK)
      return st;
    const size_t colws = quant_col_ws_bytes(1, N, K) > 0 ? quant_col_ws_bytes(1, N, K) : 256;
    if (bwd_kpacked(M, N, K)) {
      // w^T k-packed as the grad-input GEMM's B operand
      if ((st = fp8_quant_col_kpacked(w, 1, N, K, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qwt, (float*)L.swc, (float*)L.iwc,
                                      L.wscol, colws, stream)) != FP8_OK)
        return st;
      if ((st = fp8_scaled_mm_kpacked((const uint8_t*)L.qg, FP8_E5M2_NATIVE, (const uint8_t*)L.qwt, FP8_E4M3_NATIVE,
                                      FP8_SCALE_ROW, (const float*)L.ig, (const float*)L.iwc, M, K, N, FP8_OUT_BF16,
                                      gx, 0, stream)) != FP8_OK)
        return st;
      return fp8_wgrad_bf16(gy, x, M, N, K, gw, stream);
    }
    if ((st = fp8_quant_col(w, 1, N, K, FP8_E4M3_NATIVE, eps, (uint8_t*)L.qwt, (float*)L.swc, (float*)L.iwc, L.wscol,
                            colws, stream)) != FP8_OK)
      return st;
  }
  // grad-input: [M][N] x ([K][N])^T -> [M][K]
  if ((st = fp8_scaled_mm((const uint8_t*)L.qg, FP8_E5M2_NATIVE, (const uint8_t*)L.qwt, FP8_E4M3_NATIVE,
                          tw ? FP8_SCALE_TENSOR : FP8_SCALE_ROW, (const float*)L.ig, (const float*)L.iwc, M, K, N,
                          FP8_OUT_BF16, gx, 0, stream)) != FP8_OK)
    return st;
  // grad-weight [N][K]: tensorwise in FP8, ([N][M] x ([K][M])^T), rowwise in BF16 (gy^T x)
  if (tw)
    return fp8_scaled_mm((const uint8_t*)L.qgt, FP8_E5M2_NATIVE, (const uint8_t*)L.qxt, FP8_E4M3_NATIVE,
                         FP8_SCALE_TENSOR, (const float*)L.ig, (const float*)L.ix, N, K, M, FP8_OUT_BF16, gw, 0, stream);
  return fp8_wgrad_bf16(gy, x, M, N, K, gw, stream);
}

}  // extern "C"
