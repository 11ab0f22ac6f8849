// api.hip -- the C ABI (include/fp8dyn.h): host-side validation, format
// resolution through the per-device probe cache, and dispatch to the kernel
// launchers. Nothing is launched when validation fails.
#include <cmath>
#include <mutex>
#include <atomic>
#include <cstring>

#include "../../include/fp8dyn.h"
#include "internal.hpp"

using namespace fp8dyn;

namespace {

std::atomic<int> g_last_error{0};

struct ProbeCache {
  std::mutex mu;
  bool done[64] = {};
  fp8_status status[64] = {};
  fp8_format e4[64] = {};
  fp8_format e5[64] = {};
};
ProbeCache& cache() {
  static ProbeCache c;
  return c;
}

fp8_status dev_err(hipError_t e) {
  if (e == hipSuccess) return FP8_OK;
  g_last_error.store((int)e);
  return FP8_ERR_DEVICE;
}

fp8_status probe_device(int device, fp8_format* e4, fp8_format* e5) {
  if (device < 0 || device >= 64) return FP8_ERR_INVALID_ARGUMENT;
  ProbeCache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  if (!c.done[device]) {
    int cur = 0;
    hipError_t he = hipGetDevice(&cur);
    if (he != hipSuccess) return dev_err(he);
    if (cur != device && (he = hipSetDevice(device)) != hipSuccess) return dev_err(he);
    fp8_status st = FP8_OK;
    hipDeviceProp_t prop;
    he = hipGetDeviceProperties(&prop, device);
    if (he != hipSuccess) {
      st = dev_err(he);
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      st = FP8_ERR_UNSUPPORTED;
    } else {
      float r[6] = {0, 0, 0, 0, 0, 0};
      he = run_probe(r);
      if (he != hipSuccess) {
        st = dev_err(he);
      } else {
        // convert side: code of 1.0; matrix-core side: 128 * value(code)^2
        const bool cvt_e4_ocp = r[0] == 56.0f, cvt_e4_fnuz = r[0] == 64.0f;
        const bool cvt_e5_ocp = r[1] == 60.0f, cvt_e5_fnuz = r[1] == 64.0f;
        const bool mma_e4_ocp = r[4] == 128.0f, mma_e4_fnuz = r[4] == 32.0f;
        const bool mma_e5_ocp = r[5] == 128.0f, mma_e5_fnuz = r[5] == 32.0f;
        if (cvt_e4_ocp && mma_e4_ocp && cvt_e5_ocp && mma_e5_ocp) {
          c.e4[device] = FP8_E4M3FN;
          c.e5[device] = FP8_E5M2;
        } else if (cvt_e4_fnuz && mma_e4_fnuz && cvt_e5_fnuz && mma_e5_fnuz) {
          c.e4[device] = FP8_E4M3FNUZ;
          c.e5[device] = FP8_E5M2FNUZ;
        } else {
          st = FP8_ERR_UNSUPPORTED;  // converts and matrix cores disagree
        }
      }
    }
    if (cur != device) (void)hipSetDevice(cur);
    c.status[device] = st;
    c.done[device] = true;
  }
  if (c.status[device] != FP8_OK) return c.status[device];
  if (e4) *e4 = c.e4[device];
  if (e5) *e5 = c.e5[device];
  return FP8_OK;
}

// Resolves a requested format for the current device. Only the device's
// native variants are produced/consumed by the kernels.
fp8_status resolve(fp8_format f, bool* is_e5, double* fmax) {
  if ((int)f < 0 || (int)f > 5) return FP8_ERR_INVALID_ARGUMENT;
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return dev_err(he);
  fp8_format e4, e5;
  fp8_status st = probe_device(dev, &e4, &e5);
  if (st != FP8_OK) return st;
  if (f == FP8_E4M3_NATIVE) f = e4;
  if (f == FP8_E5M2_NATIVE) f = e5;
  if (f == e4) {
    *is_e5 = false;
  } else if (f == e5) {
    *is_e5 = true;
  } else {
    return FP8_ERR_UNSUPPORTED;
  }
  *fmax = f == FP8_E4M3FN ? 448.0 : (f == FP8_E4M3FNUZ ? 240.0 : 57344.0);
  return FP8_OK;
}

// Quantization outputs that are not consumed by this GPU's matrix cores: the
// fnuz variants on an OCP device, written by the software encoder (MI300
// interop). Anything else resolves as above.
fp8_status resolve_out(fp8_format f, bool* is_e5, double* fmax, bool* fnuz) {
  *fnuz = false;
  fp8_status st = resolve(f, is_e5, fmax);
  if (st != FP8_ERR_UNSUPPORTED || (f != FP8_E4M3FNUZ && f != FP8_E5M2FNUZ)) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_DEVICE;
  fp8_format e4, e5;
  if ((st = probe_device(dev, &e4, &e5)) != FP8_OK) return st;
  if (e4 != FP8_E4M3FN || e5 != FP8_E5M2) return FP8_ERR_UNSUPPORTED;
  *is_e5 = f == FP8_E5M2FNUZ;
  *fmax = f == FP8_E4M3FNUZ ? 240.0 : 57344.0;
  *fnuz = true;
  return FP8_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool bad_eps(double eps) { return !(std::isfinite(eps) && eps > 0.0); }

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status s) {
  switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FP8_ERR_ALIGNMENT: return "alignment or divisibility rule broken";
    case FP8_ERR_UNSUPPORTED: return "unsupported format, device or shape";
    case FP8_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8_ERR_DEVICE: return "HIP error";
  }
  return "unknown status";
}

int fp8_last_device_error(void) { return g_last_error.load(); }

double fp8_format_max(fp8_format f) {
  switch (f) {
    case FP8_E4M3FN: return 448.0;
    case FP8_E4M3FNUZ: return 240.0;
    case FP8_E5M2:
    case FP8_E5M2FNUZ: return 57344.0;
    default: {
      bool e5;
      double fm;
      return resolve(f, &e5, &fm) == FP8_OK ? fm : 0.0;
    }
  }
}

fp8_status fp8_probe(int device, fp8_format* e4m3_native, fp8_format* e5m2_native) {
  return probe_device(device, e4m3_native, e5m2_native);
}

size_t fp8_quant_tensor_ws_bytes(void) { return 256; }

size_t fp8_quant_col_ws_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 0 || cols < 0) return 0;
  return quant_col_ws_bytes(batch, rows, cols);
}

static fp8_status check_quant_common(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, double eps,
                                     const uint8_t* q, const void* scale) {
  if (batch < 0 || rows < 0 || cols < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (bad_eps(eps)) return FP8_ERR_INVALID_ARGUMENT;
  if (batch * rows * cols == 0) return FP8_OK;
  if (!x || !q || !scale) return FP8_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8_ERR_ALIGNMENT;
  return FP8_OK;
}

// Groups with no elements still get their scales: amax 0, so the eps-clamped
// value. Nothing is read; scale (and inv, when given) must hold n floats.
// fnuz: whether the calling quantizer offers the fnuz outputs.
static fp8_status empty_group_scales(fp8_format fmt, bool fnuz, double eps, float* scale, float* inv, int64_t n,
                                     void* stream) {
  if (n == 0) return FP8_OK;
  if (!scale) return FP8_ERR_INVALID_ARGUMENT;
  if (!aligned(scale, 4) || (inv && !aligned(inv, 4))) return FP8_ERR_ALIGNMENT;
  bool e5, nz;
  double fm;
  fp8_status st = fnuz ? resolve_out(fmt, &e5, &fm, &nz) : resolve(fmt, &e5, &fm);
  if (st != FP8_OK) return st;
  return dev_err(launch_empty_group_scales(scale, inv, n, fm, eps, (hipStream_t)stream));
}

fp8_status fp8_quant_tensor(const uint16_t* x, int64_t n, fp8_format fmt, double eps, uint8_t* q, float* scale,
                            float* inv_scale, void* ws, size_t ws_bytes, void* stream) {
  fp8_status st = check_quant_common(x, 1, 1, n, eps, q, scale);
  if (st != FP8_OK) return st;
  if (n == 0) return empty_group_scales(fmt, true, eps, scale, inv_scale, 1, stream);
  if (!ws || ws_bytes < fp8_quant_tensor_ws_bytes()) return FP8_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return FP8_ERR_ALIGNMENT;
  bool e5, nz;
  double fm;
  if ((st = resolve_out(fmt, &e5, &fm, &nz)) != FP8_OK) return st;
  QuantArgs a{x, 1, 1, n, e5, fm, eps, q, scale, inv_scale, (hipStream_t)stream, nz};
  return dev_err(launch_quant_tensor(a, ws));
}

fp8_status fp8_quant_row(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt, double eps,
                         uint8_t* q, float* scale, float* inv_scale, void* stream) {
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, scale);
  if (st != FP8_OK) return st;
  if (cols == 0) return empty_group_scales(fmt, true, eps, scale, inv_scale, batch * rows, stream);
  if (batch * rows == 0) return FP8_OK;
  bool e5, nz;
  double fm;
  if ((st = resolve_out(fmt, &e5, &fm, &nz)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, scale, inv_scale, (hipStream_t)stream, nz};
  return dev_err(launch_quant_row(a));
}

fp8_status fp8_quant_row_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                 double eps, uint8_t* q, float* scale, float* inv_scale, void* stream) {
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, scale);
  if (st != FP8_OK) return st;
  if (rows % 16 != 0 || cols % 64 != 0) return FP8_ERR_ALIGNMENT;
  if (cols > 16384) return FP8_ERR_UNSUPPORTED;
  if (cols == 0) return empty_group_scales(fmt, false, eps, scale, inv_scale, batch * rows, stream);
  if (batch * rows == 0) return FP8_OK;
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, scale, inv_scale, (hipStream_t)stream};
  return dev_err(launch_quant_row_kpacked(a, 16));
}

fp8_status fp8_quant_row_kpaired(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                 double eps, uint8_t* q, float* scale, float* inv_scale, void* stream) {
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, scale);
  if (st != FP8_OK) return st;
  if (rows % 2 != 0 || cols % 64 != 0) return FP8_ERR_ALIGNMENT;
  if (cols > 16384) return FP8_ERR_UNSUPPORTED;
  if (cols == 0) return empty_group_scales(fmt, false, eps, scale, inv_scale, batch * rows, stream);
  if (batch * rows == 0) return FP8_OK;
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, scale, inv_scale, (hipStream_t)stream};
  return dev_err(launch_quant_row_kpacked(a, 2));
}

fp8_status fp8_quant_col(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt, double eps,
                         uint8_t* qT, float* scale, float* inv_scale, void* ws, size_t ws_bytes, void* stream) {
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, qT, scale);
  if (st != FP8_OK) return st;
  if (rows == 0) return empty_group_scales(fmt, false, eps, scale, inv_scale, batch * cols, stream);
  if (batch * cols == 0) return FP8_OK;
  const size_t need = quant_col_ws_bytes(batch, rows, cols);
  const bool vec_path = cols % 8 == 0 && rows % 16 == 0;
  if (need > 0 && vec_path) {
    if (!ws || ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return FP8_ERR_ALIGNMENT;
  }
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, qT, scale, inv_scale, (hipStream_t)stream};
  return dev_err(launch_quant_col(a, ws));
}

fp8_status fp8_quant_col_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                 double eps, uint8_t* qT, float* scale, float* inv_scale, void* ws, size_t ws_bytes,
                                 void* stream) {
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, qT, scale);
  if (st != FP8_OK) return st;
  if (rows % 64 != 0 || cols % 16 != 0) return FP8_ERR_ALIGNMENT;
  if (rows * cols >= ((int64_t)1 << 30)) return FP8_ERR_UNSUPPORTED;  // 32-bit offsets in a batch slice
  if (rows == 0) return empty_group_scales(fmt, false, eps, scale, inv_scale, batch * cols, stream);
  if (batch * cols == 0) return FP8_OK;
  const size_t need = quant_col_ws_bytes(batch, rows, cols);
  if (need > 0) {
    if (!ws || ws_bytes < need) return FP8_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return FP8_ERR_ALIGNMENT;
  }
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, qT, scale, inv_scale, (hipStream_t)stream};
  return dev_err(launch_quant_col_kpacked(a, ws));
}

fp8_status fp8_norm_quant_row(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                              int64_t cols, fp8_norm kind, double norm_eps, fp8_format fmt, double eps, uint16_t* y,
                              uint8_t* q, float* scale, float* inv_scale, void* stream) {
  if (rows < 0 || cols < 0 || bad_eps(eps) || !(std::isfinite(norm_eps) && norm_eps >= 0.0))
    return FP8_ERR_INVALID_ARGUMENT;
  if (kind != FP8_NORM_RMS && kind != FP8_NORM_LAYER) return FP8_ERR_INVALID_ARGUMENT;
  if (kind == FP8_NORM_RMS && beta) return FP8_ERR_INVALID_ARGUMENT;
  if (rows == 0) return FP8_OK;
  // empty rows: nothing to normalize, and the quantization's groups are empty
  if (cols == 0) return empty_group_scales(fmt, false, eps, scale, inv_scale, scale ? rows : 0, stream);
  if (!x || !gamma || (!y && !q) || (q && !scale)) return FP8_ERR_INVALID_ARGUMENT;
  if (cols % 8 != 0) return FP8_ERR_ALIGNMENT;
  if (cols > 16384) return FP8_ERR_UNSUPPORTED;  // the row lives in registers
  if (!aligned(x, 16) || !aligned(gamma, 16) || (beta && !aligned(beta, 16)) || (y && !aligned(y, 16)) ||
      (q && !aligned(q, 8)) || (scale && !aligned(scale, 4)) || (inv_scale && !aligned(inv_scale, 4)))
    return FP8_ERR_ALIGNMENT;
  bool e5;
  double fm;
  fp8_status st;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  NormQuantArgs a{x, gamma, beta, rows, cols, kind == FP8_NORM_LAYER, norm_eps, e5, fm, eps, y, q, scale, inv_scale,
                  (hipStream_t)stream};
  return dev_err(launch_norm_quant_row(a));
}

size_t fp8_quant_dual_ws_bytes(void) { return 256; }

fp8_status fp8_quant_dual(const uint16_t* gy, const uint16_t* x, int64_t M, int64_t N, int64_t K, fp8_format g_fmt,
                          fp8_format x_fmt, double eps, uint8_t* gq, uint8_t* gqT, float* g_scale, float* g_inv,
                          uint8_t* xqT, float* x_scale, float* x_inv, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0 || bad_eps(eps)) return FP8_ERR_INVALID_ARGUMENT;
  bool ge5, xe5;
  double gfm, xfm;
  fp8_status st;
  if ((st = resolve(g_fmt, &ge5, &gfm)) != FP8_OK || (st = resolve(x_fmt, &xe5, &xfm)) != FP8_OK) return st;
  // each tensor has one group and so one scale, even when it is empty
  const bool g_has = M * N > 0, x_has = M * K > 0;
  if (!g_scale || !x_scale) return FP8_ERR_INVALID_ARGUMENT;
  if ((g_has && (!gy || !gqT)) || (x_has && (!x || !xqT))) return FP8_ERR_INVALID_ARGUMENT;
  if ((g_has || x_has) && M % 16 != 0) return FP8_ERR_ALIGNMENT;
  if ((g_has && N % 8 != 0) || (x_has && K % 8 != 0)) return FP8_ERR_ALIGNMENT;
  if (M * N >= ((int64_t)1 << 30) || M * K >= ((int64_t)1 << 30)) return FP8_ERR_UNSUPPORTED;
  if ((gy && !aligned(gy, 16)) || (x && !aligned(x, 16)) || (gqT && !aligned(gqT, 16)) || (xqT && !aligned(xqT, 16)) ||
      (gq && !aligned(gq, 8)) || !aligned(g_scale, 4) || !aligned(x_scale, 4) || (g_inv && !aligned(g_inv, 4)) ||
      (x_inv && !aligned(x_inv, 4)))
    return FP8_ERR_ALIGNMENT;
  TJobSpec jobs[2];
  int nj = 0;
  if (g_has) jobs[nj++] = {gy, M, N, ge5, gfm, gq, gqT, g_scale, g_inv};
  if (x_has) jobs[nj++] = {x, M, K, xe5, xfm, nullptr, xqT, x_scale, x_inv};
  if (nj > 0) {
    if (!ws || ws_bytes < fp8_quant_dual_ws_bytes()) return FP8_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return FP8_ERR_ALIGNMENT;
    if ((st = dev_err(launch_quant_tensor_multi_t(jobs, nj, eps, (uint32_t*)ws, (hipStream_t)stream))) != FP8_OK)
      return st;
  }
  if (!g_has && (st = dev_err(launch_empty_group_scales(g_scale, g_inv, 1, gfm, eps, (hipStream_t)stream))) != FP8_OK)
    return st;
  if (!x_has) return dev_err(launch_empty_group_scales(x_scale, x_inv, 1, xfm, eps, (hipStream_t)stream));
  return FP8_OK;
}

fp8_status fp8_quant_block(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int block_rows,
                           int block_cols, fp8_format fmt, double eps, uint8_t* q, float* scale, float* inv_scale,
                           void* stream) {
  if (!((block_rows == 1 || block_rows == 128) && block_cols == 128)) return FP8_ERR_INVALID_ARGUMENT;
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, scale);
  if (st != FP8_OK || batch * rows * cols == 0) return st;
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, scale, inv_scale, (hipStream_t)stream};
  return dev_err(launch_quant_block(a, block_rows, block_cols));
}

fp8_status fp8_quant_mx(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                        fp8_mx_mode mode, double eps, uint8_t* q, uint8_t* e8m0, void* stream) {
  if (mode != FP8_MX_POW2_FLOOR && mode != FP8_MX_OCP) return FP8_ERR_INVALID_ARGUMENT;
  // the E8M0 range: with eps >= 2^-100 every group's exponent lies in [-120, 115]
  if (!(eps >= 0x1p-100)) return FP8_ERR_INVALID_ARGUMENT;
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, e8m0);
  if (st != FP8_OK || batch * rows * cols == 0) return st;
  if (cols % 32 != 0) return FP8_ERR_ALIGNMENT;
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, nullptr, nullptr, (hipStream_t)stream};
  return dev_err(launch_quant_mx(a, e8m0, (int)mode));
}

// fp8_quant_mx with packed codes (group_rows 16: k-packed, 2: pair-interleaved)
static fp8_status quant_mx_packed(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                  fp8_mx_mode mode, double eps, uint8_t* q, uint8_t* e8m0, void* stream,
                                  int group_rows) {
  if (mode != FP8_MX_POW2_FLOOR && mode != FP8_MX_OCP) return FP8_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0x1p-100)) return FP8_ERR_INVALID_ARGUMENT;
  fp8_status st = check_quant_common(x, batch, rows, cols, eps, q, e8m0);
  if (st != FP8_OK || batch * rows * cols == 0) return st;
  if (rows % group_rows != 0 || cols % 64 != 0) return FP8_ERR_ALIGNMENT;
  if (((uintptr_t)x & 15) != 0 || ((uintptr_t)q & 15) != 0) return FP8_ERR_ALIGNMENT;
  bool e5;
  double fm;
  if ((st = resolve(fmt, &e5, &fm)) != FP8_OK) return st;
  QuantArgs a{x, batch, rows, cols, e5, fm, eps, q, nullptr, nullptr, (hipStream_t)stream};
  return dev_err(launch_quant_mx_packed(a, e8m0, (int)mode, group_rows));
}

fp8_status fp8_quant_mx_kpacked(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                fp8_mx_mode mode, double eps, uint8_t* q, uint8_t* e8m0, void* stream) {
  return quant_mx_packed(x, batch, rows, cols, fmt, mode, eps, q, e8m0, stream, 16);
}

fp8_status fp8_quant_mx_kpaired(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                fp8_mx_mode mode, double eps, uint8_t* q, uint8_t* e8m0, void* stream) {
  return quant_mx_packed(x, batch, rows, cols, fmt, mode, eps, q, e8m0, stream, 2);
}

static fp8_status check_gemm(const void* a, const void* b, const void* sa, const void* sb, int64_t M, int64_t N,
                             int64_t K, fp8_scaling scaling, fp8_out out_type, const void* out) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
  if ((int)scaling < 0 || (int)scaling > 3) return FP8_ERR_INVALID_ARGUMENT;
  if (out_type != FP8_OUT_BF16 && out_type != FP8_OUT_F32) return FP8_ERR_INVALID_ARGUMENT;
  if (M == 0 || N == 0) return FP8_OK;
  if (!out) return FP8_ERR_INVALID_ARGUMENT;
  if (K > 0 && (!a || !b || !sa || !sb)) return FP8_ERR_INVALID_ARGUMENT;
  if (K % 16 != 0) return FP8_ERR_ALIGNMENT;
  if (scaling == FP8_SCALE_BLOCK128 && (K % 128 != 0 || N % 128 != 0)) return FP8_ERR_ALIGNMENT;
  if (scaling == FP8_SCALE_MX32 && K % 32 != 0) return FP8_ERR_ALIGNMENT;
  if ((a && !aligned(a, 16)) || (b && !aligned(b, 16)) || !aligned(out, 4)) return FP8_ERR_ALIGNMENT;
  if (scaling != FP8_SCALE_MX32 && ((sa && !aligned(sa, 4)) || (sb && !aligned(sb, 4)))) return FP8_ERR_ALIGNMENT;
  return FP8_OK;
}

// A in {e4m3, e5m2} (native variants), B the e4m3 native variant.
static fp8_status resolve_ab(fp8_format fa, fp8_format fb, bool* ea) {
  if (fb == FP8_E5M2 || fb == FP8_E5M2FNUZ || fb == FP8_E5M2_NATIVE) return FP8_ERR_UNSUPPORTED;
  bool eb;
  double fm;
  fp8_status st;
  if ((st = resolve(fa, ea, &fm)) != FP8_OK) return st;
  if ((st = resolve(fb, &eb, &fm)) != FP8_OK) return st;
  return eb ? FP8_ERR_UNSUPPORTED : FP8_OK;
}

fp8_status fp8_scaled_mm(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb, fp8_scaling scaling,
                         const float* a_inv, const float* b_inv, int64_t M, int64_t N, int64_t K, fp8_out out_type,
                         void* out, int use_fast_accum, void* stream) {
  if (scaling != FP8_SCALE_TENSOR && scaling != FP8_SCALE_ROW) return FP8_ERR_UNSUPPORTED;
  fp8_status st = check_gemm(a, b, a_inv, b_inv, M, N, K, scaling, out_type, out);
  if (st != FP8_OK || M == 0 || N == 0) return st;
  bool ea;
  if ((st = resolve_ab(fa, fb, &ea)) != FP8_OK) return st;
  // no contraction terms: the empty sum (nothing is read)
  if (K == 0) return dev_err(launch_zero_fill(out, M * N * (out_type == FP8_OUT_F32 ? 4 : 2), (hipStream_t)stream));
  GemmArgs g{a, b, a_inv, b_inv, nullptr, 1, M, N, K, ea, false, (int)scaling, out_type == FP8_OUT_F32, out,
             (hipStream_t)stream};
  g.exact = !use_fast_accum;
  return dev_err(launch_gemm_fp8(g));
}

fp8_status fp8_grouped_mm(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb, fp8_scaling scaling,
                          const void* a_scale, const void* b_scale, const int32_t* offsets, int32_t E, int64_t Mtot,
                          int64_t N, int64_t K, fp8_out out_type, void* out, int use_fast_accum, void* stream) {
  if (scaling == FP8_SCALE_TENSOR) return FP8_ERR_UNSUPPORTED;
  if (E < 1 || E > 1024) return FP8_ERR_INVALID_ARGUMENT;
  fp8_status st = check_gemm(a, b, a_scale, b_scale, Mtot, N, K, scaling, out_type, out);
  if (st != FP8_OK || Mtot == 0 || N == 0) return st;
  if (!offsets) return FP8_ERR_INVALID_ARGUMENT;
  if (!aligned(offsets, 4)) return FP8_ERR_ALIGNMENT;
  bool ea;
  if ((st = resolve_ab(fa, fb, &ea)) != FP8_OK) return st;
  // no contraction terms: every row of every expert is the empty sum
  if (K == 0)
    return dev_err(launch_zero_fill(out, Mtot * N * (out_type == FP8_OUT_F32 ? 4 : 2), (hipStream_t)stream));
  GemmArgs g{a, b, a_scale, b_scale, offsets, E, Mtot, N, K, ea, false, (int)scaling, out_type == FP8_OUT_F32, out,
             (hipStream_t)stream};
  g.exact = !use_fast_accum;
  return dev_err(launch_gemm_fp8(g));
}

fp8_status fp8_scaled_mm_kpacked(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                 fp8_scaling scaling, const float* a_inv, const float* b_inv, int64_t M, int64_t N,
                                 int64_t K, fp8_out out_type, void* out, int use_fast_accum, void* stream) {
  if (scaling != FP8_SCALE_TENSOR && scaling != FP8_SCALE_ROW) return FP8_ERR_UNSUPPORTED;
  fp8_status st = check_gemm(a, b, a_inv, b_inv, M, N, K, scaling, out_type, out);
  if (st != FP8_OK || M == 0 || N == 0) return st;
  if (N % 16 != 0 || K % 128 != 0) return FP8_ERR_ALIGNMENT;
  if (N * K >= ((int64_t)1 << 31)) return FP8_ERR_UNSUPPORTED;  // 32-bit offsets in B
  bool ea;
  if ((st = resolve_ab(fa, fb, &ea)) != FP8_OK) return st;
  GemmArgs g{a, b, a_inv, b_inv, nullptr, 1, M, N, K, ea, false, (int)scaling, out_type == FP8_OUT_F32, out,
             (hipStream_t)stream, true};
  g.exact = !use_fast_accum;
  if (!gemm_fp8_fast_eligible(g)) return FP8_ERR_UNSUPPORTED;
  return dev_err(launch_gemm_fp8_fast(g));
}

fp8_status fp8_grouped_mm_kpacked(const uint8_t* a, fp8_format fa, const uint8_t* b, fp8_format fb,
                                  fp8_scaling scaling, const void* a_scale, const void* b_scale,
                                  const int32_t* offsets, int32_t E, int64_t Mtot, int64_t N, int64_t K,
                                  fp8_out out_type, void* out, int use_fast_accum, void* stream) {
  if (scaling != FP8_SCALE_ROW && scaling != FP8_SCALE_MX32) return FP8_ERR_UNSUPPORTED;
  if (!use_fast_accum && scaling != FP8_SCALE_ROW) return FP8_ERR_UNSUPPORTED;
  if (E < 1 || E > 1024) return FP8_ERR_INVALID_ARGUMENT;
  fp8_status st = check_gemm(a, b, a_scale, b_scale, Mtot, N, K, scaling, out_type, out);
  if (st != FP8_OK || Mtot == 0 || N == 0) return st;
  if (!offsets) return FP8_ERR_INVALID_ARGUMENT;
  if (!aligned(offsets, 4)) return FP8_ERR_ALIGNMENT;
  if (N % 16 != 0 || K % 128 != 0 || Mtot % 2 != 0) return FP8_ERR_ALIGNMENT;
  // 32-bit offsets in an expert's B and in a tile's pairs of A rows
  if (N * K >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 22)) return FP8_ERR_UNSUPPORTED;
  bool ea;
  if ((st = resolve_ab(fa, fb, &ea)) != FP8_OK) return st;
  GemmArgs g{a, b, a_scale, b_scale, offsets, E, Mtot, N, K, ea, false, (int)scaling, out_type == FP8_OUT_F32, out,
             (hipStream_t)stream, true};
  g.exact = !use_fast_accum;
  if (!gemm_fp8_fast_eligible(g)) return FP8_ERR_UNSUPPORTED;
  return dev_err(launch_gemm_fp8_fast(g));
}

fp8_status fp8_wgrad_bf16(const uint16_t* gy, const uint16_t* x, int64_t M, int64_t N, int64_t K, uint16_t* gw,
                          void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (N == 0 || K == 0) return FP8_OK;
  if (!gw || (M > 0 && (!gy || !x))) return FP8_ERR_INVALID_ARGUMENT;
  if (N % 8 != 0 || K % 8 != 0) return FP8_ERR_ALIGNMENT;
  if ((gy && !aligned(gy, 16)) || (x && !aligned(x, 16)) || !aligned(gw, 4)) return FP8_ERR_ALIGNMENT;
  // no rows: the empty sum
  if (M == 0) return dev_err(launch_zero_fill(gw, N * K * 2, (hipStream_t)stream));
  WgradArgs w{gy, x, M, N, K, gw, (hipStream_t)stream};
  return dev_err(launch_wgrad_bf16(w));
}

fp8_status fp8_grouped_wgrad_bf16(const uint16_t* gy, const uint16_t* x, const int32_t* offsets, int32_t E,
                                  int64_t Mtot, int64_t N, int64_t K, uint16_t* gw, void* stream) {
  if (E < 0 || Mtot < 0 || N < 0 || K < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (E == 0 || N == 0 || K == 0) return FP8_OK;
  if (!gw || !offsets || (Mtot > 0 && (!gy || !x))) return FP8_ERR_INVALID_ARGUMENT;
  if (E > 1024) return FP8_ERR_UNSUPPORTED;  // the kernel keeps offsets and costs in LDS
  if (N % 8 != 0 || K % 8 != 0) return FP8_ERR_ALIGNMENT;
  if ((gy && !aligned(gy, 16)) || (x && !aligned(x, 16)) || !aligned(gw, 4) || !aligned(offsets, 4))
    return FP8_ERR_ALIGNMENT;
  // a 32-row stage of either operand addressed with 32-bit offsets
  if (32 * (N > K ? N : K) * 2 >= ((int64_t)1 << 31)) return FP8_ERR_UNSUPPORTED;
  GroupedWgradArgs w{gy, x, offsets, E, Mtot, N, K, gw, (hipStream_t)stream};
  return dev_err(launch_grouped_wgrad_bf16(w));
}

fp8_status fp8_validate_offsets(const int32_t* host_offsets, int32_t E, int64_t Mtot) {
  if (!host_offsets || E < 1 || Mtot < 0) return FP8_ERR_INVALID_ARGUMENT;
  if (host_offsets[0] != 0 || host_offsets[E] != Mtot) return FP8_ERR_INVALID_ARGUMENT;
  for (int32_t e = 0; e < E; ++e)
    if (host_offsets[e + 1] < host_offsets[e]) return FP8_ERR_INVALID_ARGUMENT;
  return FP8_OK;
}

}  // extern "C"
