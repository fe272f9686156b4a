// Error of a candidate recipe against a high-precision reference, the
// quantity the Dispatch runtime filters on ([LoKA] section II-C "Error
// Analysis": the mean element-wise relative error of a low-precision linear
// layer's output; section III-C "Library and Recipe Selection": candidates
// with MERE below a threshold).  The reference is the linear layer on the
// unquantized bf16 inputs, z_ref = X W + b, in fp32 (every bf16 x bf16
// product is exact in fp32; the sum runs in k order).
#include "common.hpp"
#include "launch.hpp"

namespace loka {
namespace {

constexpr int kMereThreads = 256;
constexpr int kMereMaxK = 2048;

// Fixed-order tree sum of one value per thread (deterministic).
__device__ __forceinline__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kMereThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

// One workgroup per sampled row s (row rows[s] of X and z): the row's
// reference over every column, then its sum of |z - z_ref| / |z_ref| over
// z_ref != 0 and the count of those entries.  A row index outside [0, M)
// reads row 0, contributes nothing and is counted in part[3 s + 2].
__global__ __launch_bounds__(kMereThreads) void k_mere_rows(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                                                           const float* z, const int64_t* rows, int64_t M, int N,
                                                           int K, double* part) {
  __shared__ float xs[kMereMaxK];
  __shared__ double red[kMereThreads];
  const int64_t s = blockIdx.x;
  const int64_t m0 = rows[s];
  const bool ok = m0 >= 0 && m0 < M;
  const int64_t m = ok ? m0 : 0;
  for (int k = threadIdx.x; k < K; k += kMereThreads) xs[k] = bf16_lo(x[m * K + k]);
  __syncthreads();
  double se = 0.0, cnt = 0.0;
  for (int n = threadIdx.x; n < N; n += kMereThreads) {
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) acc = fmaf(xs[k], bf16_lo(w[(int64_t)k * N + n]), acc);
    if (bias != nullptr) acc += bf16_lo(bias[n]);
    if (ok && acc != 0.0f) {
      se += fabs((double)z[m * N + n] - (double)acc) / fabs((double)acc);
      cnt += 1.0;
    }
  }
  se = block_sum(se, red);
  cnt = block_sum(cnt, red);
  if (threadIdx.x == 0) {
    part[3 * s] = se;
    part[3 * s + 1] = cnt;
    part[3 * s + 2] = ok ? 0.0 : 1.0;
  }
}

// out = {MERE, count, rows out of range}: the rows' partials summed in a
// fixed order by one workgroup.
__global__ __launch_bounds__(kMereThreads) void k_mere_sum(const double* part, int64_t S, double* out) {
  __shared__ double red[kMereThreads];
  double a = 0.0, b = 0.0, c = 0.0;
  for (int64_t i = threadIdx.x; i < S; i += kMereThreads) {
    a += part[3 * i];
    b += part[3 * i + 1];
    c += part[3 * i + 2];
  }
  a = block_sum(a, red);
  b = block_sum(b, red);
  c = block_sum(c, red);
  if (threadIdx.x == 0) {
    out[0] = b > 0.0 ? a / b : 0.0;
    out[1] = b;
    out[2] = c;
  }
}

}  // namespace

size_t mere_workspace_bytes(int64_t S) { return (size_t)S * 3 * sizeof(double); }
int mere_max_k() { return kMereMaxK; }

hipError_t launch_mere(const MereLaunch& a, hipStream_t s) {
  double* part = static_cast<double*>(a.workspace);
  hipLaunchKernelGGL(k_mere_rows, dim3((unsigned)a.S), dim3(kMereThreads), 0, s, static_cast<const uint16_t*>(a.x),
                     static_cast<const uint16_t*>(a.w), static_cast<const uint16_t*>(a.bias), a.z, a.rows, a.M,
                     (int)a.N, (int)a.K, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mere_sum, dim3(1), dim3(kMereThreads), 0, s, part, a.S, a.out);
  return hipGetLastError();
}

}  // namespace loka
