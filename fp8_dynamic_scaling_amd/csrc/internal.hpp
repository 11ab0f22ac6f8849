// internal.hpp -- launcher interfaces between the C-ABI layer (api.hip) and
// the kernels. Host-side only declarations; no validation happens below this
// line, so every launcher assumes arguments the API has already checked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace fp8dyn {

struct QuantArgs {
  const uint16_t* x;
  int64_t batch, rows, cols;
  bool e5;      // e5m2 (else e4m3)
  double fmax;  // largest finite value of the output format
  double eps;
  uint8_t* q;
  float* scale;
  float* inv;
  hipStream_t stream;
  bool fnuz = false;  // write the fnuz variant by software encoding (rowwise, tensorwise)
};

hipError_t launch_quant_row(const QuantArgs& a);
// codes k-packed in chunks of group_rows (16 or 2) rows x 64 columns; rows % group_rows == 0,
// cols % 64 == 0, cols <= 16384
hipError_t launch_quant_row_kpacked(const QuantArgs& a, int group_rows);
hipError_t launch_quant_col(const QuantArgs& a, void* ws);
// qT k-packed as the [cols][rows] B operand; rows % 64 == 0, cols % 16 == 0, the vector path's conditions
hipError_t launch_quant_col_kpacked(const QuantArgs& a, void* ws);
size_t quant_col_ws_bytes(int64_t batch, int64_t rows, int64_t cols);
hipError_t launch_quant_tensor(const QuantArgs& a, void* ws);  // ws >= 256 bytes
// tensorwise scale, transposed output qT[b][c][r]; needs cols % 8 == 0, rows % 16 == 0
hipError_t launch_quant_tensor_transposed(const QuantArgs& a, void* ws);
hipError_t launch_quant_block(const QuantArgs& a, int block_rows, int block_cols);
// Row normalization fused with the rowwise quantization of its bf16 output.
struct NormQuantArgs {
  const uint16_t* x;      // [rows][cols], cols % 8 == 0, cols <= 16384, 16-byte aligned
  const uint16_t* gamma;  // [cols]
  const uint16_t* beta;   // [cols] or nullptr (LayerNorm)
  int64_t rows, cols;
  bool layer;             // LayerNorm (else RMSNorm)
  double norm_eps;
  bool e5;
  double fmax, eps;
  uint16_t* y;            // [rows][cols] bf16 or nullptr
  uint8_t* q;             // [rows][cols] or nullptr (then y only)
  float* scale;
  float* inv;
  hipStream_t stream;
};
hipError_t launch_norm_quant_row(const NormQuantArgs& a);

// Tensorwise quantization of up to kMaxTJobs tensors in three launches (clear
// the amax words, amax of every tensor, one cast launch): each tensor gets its
// transposed output qT [cols][rows] and, when q is set, its row-major output
// q [rows][cols] from the same read. rows % 16 == 0, cols % 8 == 0,
// rows * cols < 2^30, 16-byte aligned x and qT, 8-byte aligned q.
// amax_words: kMaxTJobs device words.
constexpr int kMaxTJobs = 3;
struct TJobSpec {
  const uint16_t* x;
  int64_t rows, cols;
  bool e5;
  double fmax;
  uint8_t* q;   // or nullptr
  uint8_t* qT;
  float* scale;
  float* inv;   // or nullptr
};
hipError_t launch_quant_tensor_multi_t(const TJobSpec* specs, int n, double eps, uint32_t* amax_words,
                                       hipStream_t stream);
// Tensorwise quantization of two tensors (row-major codes only) in two
// launches: a per-workgroup amax pass into `partials`, then a cast pass that
// reduces them; no word needs clearing first. n % 8 == 0 for both tensors.
struct TPairSpec {
  const uint16_t* x;
  int64_t n;
  uint8_t* q;
  float* scale;
  float* inv;  // or nullptr
};
constexpr int kPairMaxAmaxBlocks = 2048;  // per tensor
hipError_t launch_quant_tensor_pair(const TPairSpec* specs, bool e5, double fmax, double eps, float* partials,
                                    hipStream_t stream);
hipError_t launch_quant_mx(const QuantArgs& a, uint8_t* e8m0, int mode);
hipError_t launch_quant_mx_packed(const QuantArgs& a, uint8_t* e8m0, int mode, int group_rows);

// Probe kernels: results[0..3] = fp8 codes of 1.0 (e4m3, e5m2) and of the
// formats' maxima; results[4..5] = matrix-core dot products of 128 copies of
// the codes 0x38 (e4m3) and 0x3C (e5m2) with themselves.
hipError_t run_probe(float* host_results);

// GEMMs ------------------------------------------------------------------------
enum ScaleKind : int { kScaleTensor = 0, kScaleRow = 1, kScaleBlock = 2, kScaleMX = 3 };

struct GemmArgs {
  const uint8_t* a;   // [Mtot][K]
  const uint8_t* b;   // [E][N][K]
  const void* sa;     // per ScaleKind
  const void* sb;
  const int32_t* offsets;  // device [E+1], or nullptr for a dense problem (E == 1)
  int32_t E;
  int64_t M, N, K;    // M = Mtot
  bool a_e5, b_e5;
  int scale_kind;
  bool out_f32;
  void* out;          // [M][N]
  hipStream_t stream;
  bool b_kpacked = false;  // B in 1 KB chunks of 16 rows x 64 K (fast kernel, ROW/TENSOR/MX scales)
  bool exact = false;      // full-precision accumulation (codes decoded to bf16, BF16 matrix cores)
};
hipError_t launch_gemm_fp8(const GemmArgs& g);
// the direct-to-LDS kernel (K % 128 == 0, aligned operands); launch_gemm_fp8 picks it
bool gemm_fp8_fast_eligible(const GemmArgs& g);
// dense tensorwise / rowwise outputs small enough for the 64 x 64 tile form
// of the generic kernel (at most one tile per CU)
bool gemm_fp8_small_dense(int64_t M, int64_t N);
hipError_t launch_gemm_fp8_fast(const GemmArgs& g);

struct WgradArgs {
  const uint16_t* gy;  // [M][N]
  const uint16_t* x;   // [M][K]
  int64_t M, N, K;
  uint16_t* gw;        // [N][K]
  hipStream_t stream;
};
hipError_t launch_wgrad_bf16(const WgradArgs& w);

struct GroupedWgradArgs {
  const uint16_t* gy;       // [Mtot][N]
  const uint16_t* x;        // [Mtot][K]
  const int32_t* offsets;   // device [E+1]
  int32_t E;
  int64_t Mtot, N, K;       // N % 8 == 0, K % 8 == 0, 32 * max(N, K) * 2 < 2^31
  uint16_t* gw;             // [E][N][K]
  hipStream_t stream;
};
hipError_t launch_grouped_wgrad_bf16(const GroupedWgradArgs& w);

// Degenerate sizes (fill.hip): the eps-clamped scale of an empty group into
// scale[0..n) (and inv), and zeros over bytes (2-byte aligned, even count).
hipError_t launch_empty_group_scales(float* scale, float* inv, int64_t n, double fmax, double eps,
                                     hipStream_t stream);
hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream);

}  // namespace fp8dyn
