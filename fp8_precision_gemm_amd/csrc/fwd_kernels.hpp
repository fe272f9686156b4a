// Kernels and launch logic of loka_gemm_fp8_ln for one scaling recipe, all
// column counts: the weight-resident persistent kernel (fwd_resident.hpp)
// when the FP8 weight fits in the workgroup's registers (K*N <= 256 KiB,
// N <= 512), otherwise one workgroup per 64-row (32 for N > 512) tile of
// the general block (fwd_block.hpp).  Each recipe's translation unit
// (fwd_tensor.hip, fwd_row.hip, fwd_mx.hip) instantiates launch_mode<MODE>.
#pragma once

#include "fwd_block.hpp"
#include "fwd_resident.hpp"

namespace loka {
namespace fwd {
namespace {

template <int MODE, int NTW, bool ALLV>
__global__ __launch_bounds__(kThreads) void k_fwd(FwdBlock p, const float* partials, int np) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (MODE == 0) {
    __shared__ float red8[kWaves];
    ScalePair sp = np < 0 ? tensor_scale_self(p, red8) : reduce_tensor_scale<0>(partials, np, red8);
    p.x_r = sp.r;
    p.x_s = sp.s;
  }
  fwd_block<MODE, NTW, Shape<NTW>::MT, ALLV>(p, (int64_t)blockIdx.x * (16 * Shape<NTW>::MT), smem);
}

template <int MODE, int NTW, bool ALLV>
hipError_t launch_t(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  constexpr int BM = 16 * Shape<NTW>::MT;
  const unsigned grid = (unsigned)((p.M + BM - 1) / BM);
  const size_t lds = fwd_lds_bytes(BM, p.K, p.N);
  auto kern = k_fwd<MODE, NTW, ALLV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, p, partials, np);
  return hipGetLastError();
}


template <int MODE, int NT, int KC, bool OPT, bool FULL>
__global__ __launch_bounds__(kThreads) void k_fwd_res(FwdBlock p, const float* partials, int np) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (MODE == 0) {
    // np < 0: X is small and every workgroup takes its max itself
    __shared__ float red8[kWaves];
    ScalePair sp = np < 0 ? tensor_scale_self(p, red8) : reduce_tensor_scale<0>(partials, np, red8);
    p.x_r = sp.r;
    p.x_s = sp.s;
  }
  // a contiguous, balanced range of 16-row tiles per workgroup (of tile
  // pairs when Y also leaves in 32 x 32 blocks: a block is two tiles); the
  // ranges in XCD order as in k_fwd_xl
  const int64_t T = (p.M + kResRows - 1) / kResRows, G = gridDim.x;
  const int64_t b = (G & 7) == 0 ? (int64_t)(blockIdx.x & 7u) * (G >> 3) + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
  const bool pairs = OPT && p.y_codes != nullptr;
  const int64_t tb = pairs ? 2 * (b * (T / 2) / G) : b * T / G, te = pairs ? 2 * ((b + 1) * (T / 2) / G) : (b + 1) * T / G;
  ResBlock<MODE, NT, KC, OPT, FULL> blk(p, tb, te, smem);
  blk.run();
}

// The staged weight-resident forward: the workgroup's whole tile range (at
// most kXlTiles tiles) in one batch (ResBlock::run_xl).
template <int MODE, int NT, int KC, bool OPT, bool EXACT>
__global__ __launch_bounds__(kThreads) void k_fwd_xl(FwdBlock p, const float* partials, int np) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (MODE == 0) {
    __shared__ float red8[kWaves];
    ScalePair sp = np < 0 ? tensor_scale_self(p, red8) : reduce_tensor_scale<0>(partials, np, red8);
    p.x_r = sp.r;
    p.x_s = sp.s;
  }
  // Workgroups go to the eight XCDs round-robin (w % 8); with G % 8 == 0
  // workgroup x + 8 j takes row group x G/8 + j, so each XCD streams one
  // contiguous eighth of X and Y (11.9 us against 12.0-12.1 at
  // 16384 x 512 x 512 with row group w)
  const int64_t T = (p.M + kResRows - 1) / kResRows, G = gridDim.x;
  const int64_t b = (G & 7) == 0 ? (int64_t)(blockIdx.x & 7u) * (G >> 3) + (blockIdx.x >> 3) : (int64_t)blockIdx.x;
  ResBlock<MODE, NT, KC, OPT, true, 0, true> blk(p, b * T / G, (b + 1) * T / G, smem);
  blk.xl_layout(smem);
  blk.template run_xl<EXACT>();
}

// Does the staged variant take this call?  Guard-free shapes (N = 128 NT,
// K = 256 KQ, M % 16 == 0) of the row-quantizing recipes with K <= 512, at
// most kXlTiles tiles per workgroup, no square-block Y output, and its LDS
// layout within the compute unit's 160 KiB.
inline bool xl_takes(const FwdBlock& p, int mode, int nt, int kc, int grid) {
  if (kc > 4 || p.y_codes != nullptr || !res_full(p.M, p.N, p.K, nt, kc)) return false;
  if (mode == 4 && p.K != 512) return false;  // code input: two rows are one 1 KiB load
  const int64_t T = (p.M + kResRows - 1) / kResRows;
  if ((T + grid - 1) / grid > kXlTiles) return false;
  return xl_lds(nt, kc, p.N, p.K).total <= 160 * 1024;
}

template <int MODE, int NT, int KC>
hipError_t launch_res_t(const FwdBlock& p, const float* partials, int np, int grid, hipStream_t s) {
  const bool opt = p.z != nullptr || p.mean != nullptr || p.rstd != nullptr || p.qx_out != nullptr ||
                   p.sx_out != nullptr || p.y_codes != nullptr;
  if constexpr (KC == 4 || (MODE != 4 && KC <= 4)) {
    if (xl_takes(p, MODE, NT, KC, grid)) {
      const size_t lds = (size_t)xl_lds(NT, KC, p.N, p.K).total;
      const bool exact = ((p.M + kResRows - 1) / kResRows) == (int64_t)grid * kXlTiles;
      auto kern = opt ? (exact ? k_fwd_xl<MODE, NT, KC, true, true> : k_fwd_xl<MODE, NT, KC, true, false>)
                      : (exact ? k_fwd_xl<MODE, NT, KC, false, true> : k_fwd_xl<MODE, NT, KC, false, false>);
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p, partials, np);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)res_lds(NT, KC, p.N).total;
  const bool full = res_full(p.M, p.N, p.K, NT, KC);
  auto kern = opt ? (full ? k_fwd_res<MODE, NT, KC, true, true> : k_fwd_res<MODE, NT, KC, true, false>)
                  : (full ? k_fwd_res<MODE, NT, KC, false, true> : k_fwd_res<MODE, NT, KC, false, false>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p, partials, np);
  return hipGetLastError();
}

}  // namespace

// Workgroups for the weight-resident kernel: one per compute unit (each
// holds a full copy of the weight), fewer when there are fewer tiles.
inline hipError_t res_grid(int64_t M, int* grid) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t T = (M + kResRows - 1) / kResRows;
  *grid = (int)(T < cus ? T : cus);
  return hipSuccess;
}

template <int MODE>
hipError_t launch_mode(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  if (res_fits(p.K, p.N)) {
    int grid = 0;
    hipError_t e = res_grid(p.M, &grid);
    if (e != hipSuccess) return e;
    const int nt = res_nt(p.N);
    switch (res_shape(nt, res_kc(nt, p.K))) {
      case 0: return launch_res_t<MODE, 1, 2>(p, partials, np, grid, s);
      case 1: return launch_res_t<MODE, 1, 4>(p, partials, np, grid, s);
      case 2: return launch_res_t<MODE, 1, 8>(p, partials, np, grid, s);
      case 3: return launch_res_t<MODE, 2, 2>(p, partials, np, grid, s);
      case 4: return launch_res_t<MODE, 2, 4>(p, partials, np, grid, s);
      case 5: return launch_res_t<MODE, 2, 8>(p, partials, np, grid, s);
      case 6: return launch_res_t<MODE, 3, 2>(p, partials, np, grid, s);
      case 7: return launch_res_t<MODE, 3, 4>(p, partials, np, grid, s);
      case 8: return launch_res_t<MODE, 3, 5>(p, partials, np, grid, s);
      case 9: return launch_res_t<MODE, 4, 2>(p, partials, np, grid, s);
      case 10: return launch_res_t<MODE, 4, 4>(p, partials, np, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  if constexpr (MODE == 4) {
    return hipErrorInvalidValue;  // the square-block recipe runs on the resident shapes only
  } else {
  switch ((p.N + 127) / 128) {  // column tiles per wavefront
#define LOKA_CASE(V) \
  case V:            \
    return p.N % 128 == 0 ? launch_t<MODE, V, true>(p, partials, np, s) : launch_t<MODE, V, false>(p, partials, np, s);
    LOKA_CASE(1) LOKA_CASE(2) LOKA_CASE(3) LOKA_CASE(4) LOKA_CASE(5) LOKA_CASE(6) LOKA_CASE(7) LOKA_CASE(8)
#undef LOKA_CASE
    default: return hipErrorInvalidValue;
  }
  }
}

}  // namespace fwd
}  // namespace loka
