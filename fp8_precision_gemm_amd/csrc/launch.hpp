// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loka {

// ---- quantization --------------------------------------------------------
struct QuantLaunch {
  const void* src;
  int64_t rows, cols, ld;
  int src_dtype;  // 0 bf16, 1 fp32
  int fmt;        // 0 e4m3, 1 e5m2
  int mode;       // loka_scaling
  int transpose_out;
  uint8_t* codes;
  void* scales;
  float* amax_out;
  void* workspace;
};
struct QuantPlan {
  int64_t np = 0;         // number of partial maxima (tensor/col) or rows (row)
  int64_t rpc = 0;        // rows per chunk (col)
  int64_t ws_floats = 0;  // workspace floats
};
QuantPlan quant_plan(int64_t rows, int64_t cols, int mode);
// One column-scaled quantization whose column maxima are already reduced to
// row-chunk partials: codes to the fragment-interleaved transposed layout
// (rows padded to 128 with zero codes), scales and multipliers per column.
struct ColQuantJob {
  const void* src;
  int src_dtype, fmt;
  int64_t rows, cols, ld;
  const float* partials;
  int64_t np;
  uint8_t* codes_t;
  float* scales;
  float* mult;  // cols floats of scratch
};
hipError_t launch_col_amax_partials(const void* src, int src_dtype, int64_t rows, int64_t cols, int64_t ld,
                                   float* partials, int64_t* np, hipStream_t s);
hipError_t launch_col_quant_pair(const ColQuantJob& a, const ColQuantJob& b, hipStream_t s);
hipError_t launch_quant(const QuantLaunch& a, hipStream_t s);

// ---- forward -------------------------------------------------------------
struct FwdLaunch {
  int64_t M, N, K;
  int x_mode;  // 0 tensor, 1 row, 3 mx32, 5 mx32 square blocks (X given as codes)
  float eps;
  const void* x;
  const uint8_t* qw;
  const void* sw;
  const void* bias;
  const void* gamma;
  const void* beta;
  void* y;
  float* z;
  float* mean;
  float* rstd;
  uint8_t* qx_out;
  void* sx_out;
  void* workspace;
  const uint8_t* x_scales;  // square-block recipe: X's E8M0 scales [M/32][K/32] (x holds its codes)
  uint8_t* y_codes;         // optional: Y quantized in 32 x 32 blocks, e4m3 [M][N]
  uint8_t* y_scales;        //   and its E8M0 scales [M/32][N/32]
  bool w_packed;   // qw already in the fragment-interleaved layout
  bool blocknorm;  // BlockNorm(256) + Hard Swish epilogue instead of LayerNorm
};
// Workspace of one forward: the tensor recipe's amax partials, then (for
// the weight-resident kernel with a row-major weight) the weight rearranged
// into the fragment-interleaved layout.
size_t fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int x_mode, bool w_packed, bool blocknorm);
// BlockNorm + Hard Swish: can the column-slab resident kernel take (N, K)?
bool fwd_blocknorm_fits(int64_t N, int64_t K);
// Bytes of a [R][C] code array in the fragment-interleaved layout (C padded
// to a multiple of 128).
inline size_t ilv_bytes(int64_t R, int64_t C) { return (size_t)R * (size_t)((C + 127) / 128 * 128); }
// [R][C] row-major codes (R % 16 == 0, C % 16 == 0) -> fragment-interleaved.
hipError_t launch_relayout(const uint8_t* src, int64_t R, int64_t C, uint8_t* dst, hipStream_t s);
// Two such rearrangements in one launch (src1 may be NULL to skip the first).
hipError_t launch_relayout2(const uint8_t* src1, int64_t R1, int64_t C1, uint8_t* dst1, const uint8_t* src2,
                            int64_t R2, int64_t C2, uint8_t* dst2, hipStream_t s);
hipError_t launch_fwd(const FwdLaunch& a, hipStream_t s);
// the allocation-free forward's device scratch (fwd_noalloc.hip)
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

// ---- backward ------------------------------------------------------------
struct BwdLaunch {
  int64_t M, N, K;
  int no_ln;
  bool sq;  // square-block recipe: sx, sw, dz_scales are E8M0 grids of 32 x 32 blocks
  const void* dy;
  const uint8_t* qx;
  const void* sx;
  const float* mean;
  const float* rstd;
  const uint8_t* qw;
  const void* sw;
  const void* bias;
  const void* gamma;
  const void* x;
  const uint8_t* qw_row;
  const float* sw_row;
  void* dx;
  float* dw;
  float* dgamma;
  float* dbeta;
  float* dbias;
  float* dz;
  uint8_t* dz_codes;
  void* dz_scales;
  void* workspace;
  bool w_packed;       // qw, qw_row already fragment-interleaved
  uint8_t* xc_codes;   // optional: the wgrad operands (else in the workspace)
  float* xc_scales;
  uint8_t* dzc_codes;
  float* dzc_scales;
};
size_t bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sq);
hipError_t launch_bwd(const BwdLaunch& a, hipStream_t s);

// ---- MERE against the fp32 reference of the linear layer ----------------
struct MereLaunch {
  int64_t M, N, K, S;
  const void* x;       // bf16 [M][K]
  const void* w;       // bf16 [K][N]
  const void* bias;    // bf16 [N] or null
  const float* z;      // the candidate's Z, fp32 [M][N]
  const int64_t* rows; // device [S]
  double* out;         // device [3]
  void* workspace;
};
size_t mere_workspace_bytes(int64_t S);
int mere_max_k();
hipError_t launch_mere(const MereLaunch& a, hipStream_t s);

// ---- Probe statistics ------------------------------------------------------
struct ProbeInputLaunch {
  int64_t B, K, n_old;
  const void* T;  // bf16 [B][K]
  float* mu;      // [K], updated
  float* S;       // [K][K] scatter, updated
  void* workspace;
};
struct ProbeWeightLaunch {
  int64_t R, C;
  float m;
  bool first;
  const void* W;  // bf16 [R][C]
  float *M, *U, *V;
  int* info;      // device [2]: Cholesky status of V, U
  void* workspace;
};
struct ProbeSampleInputLaunch {
  int64_t B, K, n;
  const float* mu;
  const float* S;
  uint64_t seed;
  void* out;  // bf16 [B][K]
  int* info;
  void* workspace;
};
struct ProbeSampleWeightLaunch {
  int64_t R, C;
  const float *M, *U, *V;
  uint64_t seed;
  void* out;  // bf16 [R][C]
  int* info;  // device [2]
  void* workspace;
};
size_t probe_input_ws(int64_t B, int64_t K);
size_t probe_weight_ws(int64_t R, int64_t C);
size_t probe_sample_input_ws(int64_t B, int64_t K);
size_t probe_sample_weight_ws(int64_t R, int64_t C);
hipError_t probe_input_update(const ProbeInputLaunch& a, hipStream_t s);
hipError_t probe_weight_update(const ProbeWeightLaunch& a, hipStream_t s);
hipError_t probe_sample_input(const ProbeSampleInputLaunch& a, hipStream_t s);
hipError_t probe_sample_weight(const ProbeSampleWeightLaunch& a, hipStream_t s);

// ---- grouped -------------------------------------------------------------
struct GroupDev {  // one group as the device sees it (copied into the workspace)
  int64_t M, N, K;
  const void* x;
  const uint8_t* qw;
  const float* sw;
  const void* bias;
  const void* gamma;
  const void* beta;
  void* y;
  float* z;
};
struct GroupedLaunch {
  int num_groups;
  float eps;
  const GroupDev* groups;  // host array
  void* workspace;         // device
  bool w_packed;           // every group's qw already fragment-interleaved
};
size_t grouped_workspace_bytes(int num_groups, const GroupDev* groups, bool w_packed);
int grouped_max_groups();
// Does a forward of this shape fit the weight-resident kernel (K*N <= 256 KiB
// of codes held in registers, N <= 512)?  Every group of a grouped launch must.
bool fwd_weight_resident(int64_t N, int64_t K);
hipError_t launch_grouped(const GroupedLaunch& a, hipStream_t s);

}  // namespace loka
