// loka_gemm_fp8_ln kernels for the MX32 block recipe (one translation unit per
// recipe keeps the compile parallel).
#include "fwd_kernels.hpp"

namespace loka {
namespace fwd {

hipError_t launch_mx(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  return launch_mode<3>(p, partials, np, s);
}

}  // namespace fwd
}  // namespace loka
