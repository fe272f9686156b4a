#define LOKA_FWD_MODE 0
#define LOKA_FWD_LAUNCHER launch_tensor
// loka_gemm_fp8_ln kernels for one scaling recipe (LOKA_FWD_MODE), all column counts.
#include "fwd_block.hpp"

namespace loka {
namespace fwd {
namespace {

template <int MODE, int NTW, bool ALLV>
__global__ __launch_bounds__(kThreads) void k_fwd(FwdBlock p, const float* partials, int np) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (MODE == 0) {
    __shared__ float red8[kWaves];
    ScalePair sp = reduce_tensor_scale<0>(partials, np, red8);
    p.x_r = sp.r;
    p.x_s = sp.s;
  }
  fwd_block<MODE, NTW, Shape<NTW>::MT, ALLV>(p, (int64_t)blockIdx.x * (16 * Shape<NTW>::MT), smem);
}

template <int NTW, bool ALLV>
hipError_t launch_t(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  constexpr int BM = 16 * Shape<NTW>::MT;
  const unsigned grid = (unsigned)((p.M + BM - 1) / BM);
  const size_t lds = fwd_lds_bytes(BM, p.K, p.N);
  auto kern = k_fwd<LOKA_FWD_MODE, NTW, ALLV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, p, partials, np);
  return hipGetLastError();
}

}  // namespace

hipError_t LOKA_FWD_LAUNCHER(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  switch ((p.N + 127) / 128) {  // column tiles per wavefront
#define LOKA_CASE(V) \
  case V:            \
    return p.N % 128 == 0 ? launch_t<V, true>(p, partials, np, s) : launch_t<V, false>(p, partials, np, s);
    LOKA_CASE(1) LOKA_CASE(2) LOKA_CASE(3) LOKA_CASE(4) LOKA_CASE(5) LOKA_CASE(6) LOKA_CASE(7) LOKA_CASE(8)
#undef LOKA_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fwd
}  // namespace loka
