// loka_gemm_fp8_ln kernels for the rowwise recipe (one translation unit per
// recipe keeps the compile parallel).
#include "fwd_kernels.hpp"

namespace loka {
namespace fwd {

hipError_t launch_row(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  return launch_mode<1>(p, partials, np, s);
}

}  // namespace fwd
}  // namespace loka
