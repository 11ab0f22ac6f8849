// noalloc.hip -- fp8_quant_col_noalloc: the column quantization of
// fp8_quant_col with its workspace (one amax word per column in the split
// form over row chunks) taken from a buffer the library keeps in device
// memory, for callers that cannot allocate: code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc.
//
// The buffer is one file-scope device array per GPU, held until the process
// ends. Host code never passes the array's name to a kernel: the name is a
// host-side stand-in. The device address comes from hipGetSymbolAddress, once
// per device with that device current, and is cached per device. Every call on
// a GPU shares that GPU's array: the kernels clear the words they use at the
// start of each call (a fill kernel, not a memset), and two calls that overlap
// on one GPU (different streams, no ordering between them) race on it.
#include <mutex>

#include "../../include/fp8dyn.h"
#include "internal.hpp"

constexpr size_t kScratchBytes = 64 * 1024;  // 16384 column-amax words

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array (the current device's).
fp8_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return FP8_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FP8_OK;
}

}  // namespace

extern "C" {

fp8_status fp8_quant_col_noalloc(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, fp8_format fmt,
                                 double eps, uint8_t* qT, float* scale, float* inv_scale, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0) return FP8_ERR_INVALID_ARGUMENT;
  const size_t need = fp8_quant_col_ws_bytes(batch, rows, cols);
  if (need > kScratchBytes) return FP8_ERR_UNSUPPORTED;  // more column-amax words than the scratch holds
  void* ws = nullptr;
  if (need > 0) {
    const fp8_status st = scratch_ptr(&ws);
    if (st != FP8_OK) return st;
  }
  return fp8_quant_col(x, batch, rows, cols, fmt, eps, qT, scale, inv_scale, ws, need > 0 ? kScratchBytes : 0,
                       stream);
}

}  // extern "C"
