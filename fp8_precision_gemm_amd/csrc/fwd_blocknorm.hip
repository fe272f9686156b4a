// loka_gemm_fp8_ln with the BlockNorm + Hard Swish epilogue
// (LOKA_FWD_BLOCKNORM_HSWISH), rowwise recipe.
//
// Source: LoKA section III-B2 (Block-wise Normalization, Fig. 7d): the
// statistics are taken over fixed blocks of 256 output features instead of
// the whole row, so no reduction crosses a block and a large output
// dimension needs no cross-block synchronization (Case 2); section III-B3
// (Hard Swish, fused in the same epilogue); section III-B1 (No Bias).
//
// Column slabs.  N is cut into slabs of 512 columns (when N % 512 == 0 and
// K <= 512) or else 256 columns, each a whole number of 256-blocks.  Slab s
// is an independent weight-resident forward over its columns (the resident
// block of fwd_resident.hpp with EPI = 1 and NT = 4 or 2): its weight
// rows are one contiguous run of the packed weight, its outputs a column
// range of Y with the full row stride.  The workgroups of one row group's
// slabs run side by side on one XCD (see slab_of), so the row group's X
// comes into that XCD's L2 once and the other slabs read it from there.
#include "fwd_resident.hpp"

namespace loka {
namespace fwd {
namespace {

// This workgroup's slab s, its row group b and the number G of row groups
// of slab s.  Workgroups go to the eight XCDs round-robin (w % 8).  When the
// grid is a multiple of 8 x slabs, workgroup w = x + 8 j (XCD x) serves slab
// j % slabs of row group x n/(8 slabs) + j / slabs: the slabs of a row group
// share an XCD and its L2, and each XCD streams a contiguous eighth of the
// rows.  Otherwise slab w % slabs of row group w / slabs.
__device__ __forceinline__ void slab_of(int slabs, int& s, int64_t& b, int64_t& G) {
  const unsigned w = blockIdx.x, n = gridDim.x, S = (unsigned)slabs;
  if (n % (8u * S) == 0) {
    const unsigned j = w >> 3;
    s = (int)(j % S);
    b = (int64_t)(w & 7u) * (n / (8u * S)) + (int64_t)(j / S);
    G = n / S;
  } else {
    s = (int)(w % S);
    b = w / S;
    G = (n - (unsigned)s + S - 1) / S;
  }
}

// the block arguments of slab s: the slab's weight rows, scales, bias and
// its column range of Y and Z
template <int NT>
__device__ __forceinline__ void slab_block(FwdBlock& p, int s) {
  constexpr int WS = 128 * NT;
  p.qw += (int64_t)s * (WS / 16) * ((p.K + 127) / 128) * 2048;
  p.sw = static_cast<const float*>(p.sw) + (int64_t)s * WS;
  if (p.bias != nullptr) p.bias += (int64_t)s * WS;
  p.y += (int64_t)s * WS;
  if (p.z != nullptr) p.z += (int64_t)s * WS;
  if (s != 0) {  // the X codes and scales are the same for every slab: slab 0 writes them
    p.qx_out = nullptr;
    p.sx_out = nullptr;
  }
}

template <int NT, int KC, bool OPT, bool FULL>
__global__ __launch_bounds__(kThreads) void k_fwd_bn(FwdBlock p, int slabs) {
  extern __shared__ __align__(16) uint8_t smem[];
  int s;
  int64_t b, G;
  slab_of(slabs, s, b, G);
  slab_block<NT>(p, s);
  const int64_t T = (p.M + kResRows - 1) / kResRows;
  ResBlock<1, NT, KC, OPT, FULL, 1> blk(p, b * T / G, (b + 1) * T / G, smem);
  blk.run();
}

// The staged run (ResBlock::run_xl, as the LayerNorm forward's k_fwd_xl)
// when every workgroup has at most kXlTiles tiles of its slab: the whole
// batch quantized, multiplied and normalized together.  Each tile's
// arithmetic is the same as k_fwd_bn's.
template <int NT, int KC, bool OPT, bool EXACT>
__global__ __launch_bounds__(kThreads) void k_fwd_bn_xl(FwdBlock p, int slabs) {
  extern __shared__ __align__(16) uint8_t smem[];
  int s;
  int64_t b, G;
  slab_of(slabs, s, b, G);
  slab_block<NT>(p, s);
  const int64_t T = (p.M + kResRows - 1) / kResRows;
  ResBlock<1, NT, KC, OPT, true, 1, true> blk(p, b * T / G, (b + 1) * T / G, smem);
  blk.xl_layout(smem);
  blk.template run_xl<EXACT>();
}

template <int NT, int KC>
hipError_t launch_bn_t(const FwdBlock& p, int slabs, int grid, hipStream_t s) {
  const bool opt = p.z != nullptr || p.qx_out != nullptr || p.sx_out != nullptr;
  const bool full = res_full(p.M, p.N, p.K, NT, KC);
  // staged: guard-free shapes with at most kXlTiles tiles for every workgroup
  // of every slab (the slab with the fewest workgroups has grid / slabs)
  const int64_t T = (p.M + kResRows - 1) / kResRows;
  const int64_t gmin = grid / slabs;
  if constexpr (KC <= 4) {
    if (full && gmin > 0 && (T + gmin - 1) / gmin <= kXlTiles && xl_lds(NT, KC, p.N, p.K).total <= 160 * 1024) {
      const size_t lds = (size_t)xl_lds(NT, KC, p.N, p.K).total;
      const bool exact = grid % slabs == 0 && T == gmin * kXlTiles;
      auto kern = opt ? (exact ? k_fwd_bn_xl<NT, KC, true, true> : k_fwd_bn_xl<NT, KC, true, false>)
                      : (exact ? k_fwd_bn_xl<NT, KC, false, true> : k_fwd_bn_xl<NT, KC, false, false>);
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p, slabs);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)res_lds(NT, KC, p.N).total;
  auto kern = opt ? (full ? k_fwd_bn<NT, KC, true, true> : k_fwd_bn<NT, KC, true, false>)
                  : (full ? k_fwd_bn<NT, KC, false, true> : k_fwd_bn<NT, KC, false, false>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p, slabs);
  return hipGetLastError();
}

}  // namespace

// slab width for BlockNorm: 512 columns when N % 512 == 0 and K <= 512, else 256
int blocknorm_slab_nt(int64_t N, int64_t K) { return (N % 512 == 0 && K <= 512) ? 4 : 2; }

hipError_t launch_row_blocknorm(const FwdBlock& p0, hipStream_t s) {
  FwdBlock p = p0;
  const int nt = blocknorm_slab_nt(p0.N, p0.K);
  const int slabs = p0.N / (128 * nt);
  p.ldy = p0.N;
  p.N = 128 * nt;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t T = (p.M + kResRows - 1) / kResRows;
  const int64_t want = T * slabs;
  const int grid = (int)(want < cus ? want : (cus < slabs ? slabs : cus));
  const int kc = res_kc(nt, p.K);
  if (nt == 4) {
    if (kc == 2) return launch_bn_t<4, 2>(p, slabs, grid, s);
    if (kc == 4) return launch_bn_t<4, 4>(p, slabs, grid, s);
  } else {
    if (kc == 2) return launch_bn_t<2, 2>(p, slabs, grid, s);
    if (kc == 4) return launch_bn_t<2, 4>(p, slabs, grid, s);
    if (kc == 8) return launch_bn_t<2, 8>(p, slabs, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fwd
}  // namespace loka
