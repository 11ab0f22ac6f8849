// probe.hip -- measures which FP8 variants this GPU's converts and matrix
// cores use. Selecting the right variant and max is a correctness matter:
// quantizing against the wrong max silently clips or mis-scales values
// ("FP8 training on AMD GPUs with TorchTitan and TorchAO", section "AMD FP8
// format in TorchAO"). The answer is measured, never assumed from the
// platform name.
//
// Convert side: the code the hardware produces for 1.0 is 0x38 (e4m3) /
// 0x3C (e5m2) under the OCP encodings (bias 7 / 15) and 0x40 under the fnuz
// encodings (bias 8 / 16). Matrix-core side: a 128-long dot product of the
// code 0x38 with itself is 128 when the code means 1.0 (OCP) and 32 when it
// means 0.5 (fnuz); likewise 0x3C for e5m2.
#include "common.hpp"
#include "internal.hpp"

namespace fp8dyn {

__device__ float g_probe_out[8];

// The matrix-core part is written in assembly with fixed registers and
// explicit wait states: on gfx950 an f8f6f4 MFMA that reads a VGPR written by
// the immediately preceding VALU instruction can see the old value, and the
// compiler does not always separate the two in a kernel this small.
__global__ __launch_bounds__(64) void k_probe(int pat_e4, int pat_e5) {
  const int lane = threadIdx.x;
  if (lane == 0) {
    g_probe_out[0] = (float)(__builtin_amdgcn_cvt_pk_fp8_f32(1.0f, 0.0f, 0, false) & 0xff);
    g_probe_out[1] = (float)(__builtin_amdgcn_cvt_pk_bf8_f32(1.0f, 0.0f, 0, false) & 0xff);
    g_probe_out[2] = (float)(__builtin_amdgcn_cvt_pk_fp8_f32(448.0f, 0.0f, 0, false) & 0xff);
    g_probe_out[3] = (float)(__builtin_amdgcn_cvt_pk_bf8_f32(57344.0f, 0.0f, 0, false) & 0xff);
  }
  float c4, c5;
  // A = B = 128 copies of one code per row; E8M0 scales 127 = 2^0;
  // cbsz / blgp 0: e4m3 operands, 1: e5m2 operands.
  asm volatile(
      "v_mov_b32 v100, %2\n v_mov_b32 v101, %2\n v_mov_b32 v102, %2\n v_mov_b32 v103, %2\n"
      "v_mov_b32 v104, %2\n v_mov_b32 v105, %2\n v_mov_b32 v106, %2\n v_mov_b32 v107, %2\n"
      "v_mov_b32 v108, %3\n v_mov_b32 v109, %3\n v_mov_b32 v110, %3\n v_mov_b32 v111, %3\n"
      "v_mov_b32 v112, %3\n v_mov_b32 v113, %3\n v_mov_b32 v114, %3\n v_mov_b32 v115, %3\n"
      "v_mov_b32 v116, 0x7f\n"
      "s_nop 7\n s_nop 7\n"
      "v_mfma_scale_f32_16x16x128_f8f6f4 v[120:123], v[100:107], v[100:107], 0, v116, v116 op_sel_hi:[0,0,0]\n"
      "s_nop 7\n"
      "v_mfma_scale_f32_16x16x128_f8f6f4 v[124:127], v[108:115], v[108:115], 0, v116, v116 op_sel_hi:[0,0,0] cbsz:1 blgp:1\n"
      "s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n"
      "v_mov_b32 %0, v120\n"
      "v_mov_b32 %1, v124\n"
      : "=v"(c4), "=v"(c5)
      : "v"(pat_e4), "v"(pat_e5)
      : "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108", "v109", "v110", "v111", "v112",
        "v113", "v114", "v115", "v116", "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127");
  if (lane == 0) {
    g_probe_out[4] = c4;
    g_probe_out[5] = c5;
  }
}

hipError_t run_probe(float* host_results) {
  hipLaunchKernelGGL(k_probe, dim3(1), dim3(64), 0, (hipStream_t)0, 0x38383838, 0x3C3C3C3C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  return hipMemcpyFromSymbol(host_results, HIP_SYMBOL(g_probe_out), 6 * sizeof(float), 0, hipMemcpyDeviceToHost);
}

}  // namespace fp8dyn
