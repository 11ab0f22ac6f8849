// fill.hip -- what the degenerate sizes produce.
//
// A group with no elements has amax 0 (the maximum of |x| over an empty set
// of non-negative values), so its scale is the eps-clamped one, the same
// scale_from_amax(0) every quantization kernel computes ("FP8 Training:
// Quantization, Autograd, Torchao", section 2: scale = fp8 max / max(amax,
// eps)). A GEMM with no contraction terms (K = 0), or a weight gradient over
// no rows (M = 0), is the empty sum: all zeros.
#include "common.hpp"
#include "internal.hpp"

namespace fp8dyn {

__global__ void k_empty_group_scales(float* __restrict__ scale, float* __restrict__ inv, int64_t n, double fmax,
                                     double eps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s, iv;
  scale_from_amax(0.0f, fmax, eps, s, iv);
  scale[i] = s;
  if (inv) inv[i] = iv;
}

// p is 2-byte aligned, bytes even: 16-byte stores where aligned, 2-byte at
// the ends
__global__ void k_zero_fill(uint8_t* __restrict__ p, int64_t bytes) {
  const int64_t mis = (int64_t)((16 - ((uintptr_t)p & 15)) & 15);  // bytes before the first 16-byte boundary
  const int64_t head = mis < bytes ? mis : bytes;
  const int64_t nvec = (bytes - head) / 16;
  const int64_t tail0 = head + nvec * 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = t; i < nvec; i += stride) reinterpret_cast<uint4*>(p + head)[i] = make_uint4(0, 0, 0, 0);
  if (t < head / 2) reinterpret_cast<uint16_t*>(p)[t] = 0;
  if (t < (bytes - tail0) / 2) reinterpret_cast<uint16_t*>(p + tail0)[t] = 0;
}

hipError_t launch_empty_group_scales(float* scale, float* inv, int64_t n, double fmax, double eps,
                                     hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_empty_group_scales, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, scale, inv, n,
                     fmax, eps);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0) return hipSuccess;
  const int64_t nvec = bytes / 16 + 1;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<uint8_t*>(p),
                     bytes);
  return hipGetLastError();
}

}  // namespace fp8dyn
