// loka_gemm_fp8_ln host dispatch: the tensor recipe's amax pass, then the
// fused kernel of the requested recipe (fwd_tensor.hip, fwd_row.hip,
// fwd_mx.hip hold the kernels; fwd_block.hpp the shared block body).
#include "fwd_block.hpp"
#include "fwd_resident.hpp"

namespace loka {

QuantPlan quant_plan(int64_t rows, int64_t cols, int mode);
hipError_t launch_amax_tensor_partials(const void* src, int64_t rows, int64_t cols, int64_t ld, float* partials,
                                       hipStream_t s);
namespace fwd {
hipError_t launch_tensor(const FwdBlock& p, const float* partials, int np, hipStream_t s);
hipError_t launch_row(const FwdBlock& p, const float* partials, int np, hipStream_t s);
hipError_t launch_mx(const FwdBlock& p, const float* partials, int np, hipStream_t s);
hipError_t launch_mx_square(const FwdBlock& p, hipStream_t s);
hipError_t launch_row_blocknorm(const FwdBlock& p, hipStream_t s);
}  // namespace fwd

bool fwd_weight_resident(int64_t N, int64_t K) { return N <= 512 && K <= 2048 && fwd::res_fits((int)K, (int)N); }

namespace {

// [R][C] row-major bytes -> fragment-interleaved (C padded to 128 with zeros).
// One thread per 16-byte piece of the destination, in destination order.
__global__ __launch_bounds__(256) void k_relayout(const uint8_t* src, int64_t R, int64_t C, uint8_t* dst) {
  const int64_t nch = (C + 127) / 128, pieces = nch * 8;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= R * pieces) return;
  const int64_t row = u / pieces, col = (u - row * pieces) * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (col < C) v = *reinterpret_cast<const uint4*>(src + row * C + col);
  *reinterpret_cast<uint4*>(dst + ilv_offset(row, col, nch)) = v;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t partial_bytes(int64_t M, int64_t K, int x_mode) {
  return x_mode == 0 ? align256((size_t)quant_plan(M, K, 0).np * sizeof(float)) : 0;
}

}  // namespace

hipError_t launch_relayout(const uint8_t* src, int64_t R, int64_t C, uint8_t* dst, hipStream_t s) {
  const int64_t n = R * ((C + 127) / 128) * 8;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_relayout, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, R, C, dst);
  return hipGetLastError();
}

namespace {
// Two [R][C] -> fragment-interleaved rearrangements: blocks [0, n1) the first.
__global__ __launch_bounds__(256) void k_relayout2(const uint8_t* src1, int64_t R1, int64_t C1, uint8_t* dst1,
                                                   int64_t n1, const uint8_t* src2, int64_t R2, int64_t C2,
                                                   uint8_t* dst2) {
  const bool first = (int64_t)blockIdx.x < n1;
  const uint8_t* src = first ? src1 : src2;
  const int64_t R = first ? R1 : R2, C = first ? C1 : C2;
  uint8_t* dst = first ? dst1 : dst2;
  const int64_t nch = (C + 127) / 128, pieces = nch * 8;
  const int64_t u = ((int64_t)blockIdx.x - (first ? 0 : n1)) * 256 + threadIdx.x;
  if (u >= R * pieces) return;
  const int64_t row = u / pieces, col = (u - row * pieces) * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (col < C) v = *reinterpret_cast<const uint4*>(src + row * C + col);
  *reinterpret_cast<uint4*>(dst + ilv_offset(row, col, nch)) = v;
}
}  // namespace

hipError_t launch_relayout2(const uint8_t* src1, int64_t R1, int64_t C1, uint8_t* dst1, const uint8_t* src2,
                            int64_t R2, int64_t C2, uint8_t* dst2, hipStream_t s) {
  const int64_t b1 = src1 ? (R1 * ((C1 + 127) / 128) * 8 + 255) / 256 : 0;
  const int64_t b2 = (R2 * ((C2 + 127) / 128) * 8 + 255) / 256;
  if (b1 + b2 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_relayout2, dim3((unsigned)(b1 + b2)), dim3(256), 0, s, src1, R1, C1, dst1, b1, src2, R2, C2,
                     dst2);
  return hipGetLastError();
}

// N a multiple of 256 up to 8192; slabs of 512 columns need K <= 512, slabs
// of 256 columns K <= 1024
bool fwd_blocknorm_fits(int64_t N, int64_t K) {
  return N >= 256 && N <= 8192 && N % 256 == 0 && K >= 16 && K % 16 == 0 && K <= 1024;
}

size_t fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int x_mode, bool w_packed, bool blocknorm) {
  size_t b = partial_bytes(M, K, x_mode);
  if (!w_packed && (blocknorm || fwd_weight_resident(N, K))) b += ilv_bytes(N, K);
  return b;
}

hipError_t launch_fwd(const FwdLaunch& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  fwd::FwdBlock p{};
  p.M = a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.x = static_cast<const uint16_t*>(a.x);
  p.qw = a.qw; p.sw = a.sw;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.gamma = static_cast<const uint16_t*>(a.gamma);
  p.beta = static_cast<const uint16_t*>(a.beta);
  p.y = static_cast<uint16_t*>(a.y);
  p.z = a.z; p.mean = a.mean; p.rstd = a.rstd; p.qx_out = a.qx_out; p.sx_out = a.sx_out;
  p.eps = a.eps; p.x_r = 1.0f; p.x_s = 1.0f;
  p.ldy = (int)a.N;
  p.xq = nullptr; p.xs = nullptr;
  p.y_codes = a.y_codes; p.y_scales = a.y_scales;
  if (a.x_mode == 5) {
    p.xq = static_cast<const uint8_t*>(a.x);
    p.xs = a.x_scales;
    p.x = nullptr;
  }
  if (!a.w_packed && (a.blocknorm || fwd_weight_resident(a.N, a.K))) {
    // the resident kernel reads the weight fragment-interleaved
    uint8_t* wi = static_cast<uint8_t*>(a.workspace) + partial_bytes(a.M, a.K, a.x_mode);
    hipError_t e = launch_relayout(a.qw, a.N, a.K, wi, s);
    if (e != hipSuccess) return e;
    p.qw = wi;
  }
  if (a.blocknorm) return fwd::launch_row_blocknorm(p, s);
  if (a.x_mode == 0) {
    // small X on the resident kernel: no partials pass, each workgroup reads
    // all of X (elements x workgroups <= 2^22, 8 MiB of cached reads)
    const int64_t tiles = (a.M + 15) / 16;
    if (fwd::res_fits((int)a.K, (int)a.N) && a.M * a.K * (tiles < 256 ? tiles : 256) <= ((int64_t)1 << 22))
      return fwd::launch_tensor(p, nullptr, -1, s);
    float* partials = static_cast<float*>(a.workspace);
    const int np = (int)quant_plan(a.M, a.K, 0).np;
    hipError_t e = launch_amax_tensor_partials(a.x, a.M, a.K, a.K, partials, s);
    if (e != hipSuccess) return e;
    return fwd::launch_tensor(p, partials, np, s);
  }
  if (a.x_mode == 1) return fwd::launch_row(p, nullptr, 0, s);
  if (a.x_mode == 5) return fwd::launch_mx_square(p, s);
  return fwd::launch_mx(p, nullptr, 0, s);
}

}  // namespace loka
