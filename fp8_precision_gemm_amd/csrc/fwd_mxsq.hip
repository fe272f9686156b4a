// loka_gemm_fp8_ln kernels for the square-block MX32 recipe: X given as e4m3
// codes with one E8M0 scale per 32 x 32 block, the weight likewise (GEM "Low
// Precision Flash Attention", Block-wise Quantization; activation
// quantization fused into the producer, GEM "Mixed Ultra-Low-Precision
// Training").  One translation unit per recipe keeps the compile parallel.
#include "fwd_kernels.hpp"

namespace loka {
namespace fwd {

hipError_t launch_mx_square(const FwdBlock& p, hipStream_t s) { return launch_mode<4>(p, nullptr, 0, s); }

}  // namespace fwd
}  // namespace loka
