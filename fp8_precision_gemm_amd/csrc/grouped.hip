// loka_grouped_gemm_fp8_ln: many independent rowwise forwards in one launch.
//
// Source: LoKA section I (wide ensembles of small layers); GEM "Generalized
// Dot-Product Attention" (tile lists precomputed on the CPU, empty tiles
// skipped) and "Expert Parallelism" (one expert per rank).  Each workgroup
// finds its group by binary search in the host-built tile table and runs
// the same block body as the single forward, so every group's output is
// bit-identical to a single loka_gemm_fp8_ln call.
#include "fwd_block.hpp"

namespace loka {
namespace fwd {
namespace {

constexpr int kMT = 4;  // 64-row tiles (groups have N <= 512: at most 4 column tiles per wavefront)

// tile_start[g] = first workgroup of group g (prefix sums of ceil(M_g / 64)),
// tile_start[num_groups] = grid size.
__global__ __launch_bounds__(kThreads) void k_grouped(const GroupDev* groups, const int* tile_start, int num_groups,
                                                 float eps) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  int lo = 0, hi = num_groups - 1;  // last group with tile_start <= b (skips empty groups)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const GroupDev gd = groups[lo];
  FwdBlock p;
  p.M = gd.M; p.N = (int)gd.N; p.K = (int)gd.K;
  p.x = static_cast<const uint16_t*>(gd.x);
  p.qw = gd.qw; p.sw = gd.sw;
  p.bias = static_cast<const uint16_t*>(gd.bias);
  p.gamma = static_cast<const uint16_t*>(gd.gamma);
  p.beta = static_cast<const uint16_t*>(gd.beta);
  p.y = static_cast<uint16_t*>(gd.y);
  p.z = gd.z;
  p.mean = nullptr; p.rstd = nullptr; p.qx_out = nullptr; p.sx_out = nullptr;
  p.eps = eps; p.x_r = 1.0f; p.x_s = 1.0f;
  const int64_t m0 = (int64_t)(b - tile_start[lo]) * (16 * kMT);
  switch ((p.N + 127) / 128) {  // column tiles per wavefront
    case 1: fwd_block<1, 1, kMT, false>(p, m0, smem); break;
    case 2: fwd_block<1, 2, kMT, false>(p, m0, smem); break;
    case 3: fwd_block<1, 3, kMT, false>(p, m0, smem); break;
    case 4: fwd_block<1, 4, kMT, false>(p, m0, smem); break;
    default: break;
  }
}

}  // namespace
}  // namespace fwd

size_t grouped_workspace_bytes(int num_groups, const GroupDev* groups) {
  (void)groups;
  size_t b = (size_t)num_groups * sizeof(GroupDev);
  b = (b + 255) / 256 * 256;
  b += (size_t)(num_groups + 1) * sizeof(int);
  return b;
}

hipError_t launch_grouped(const GroupedLaunch& a, hipStream_t s) {
  constexpr int BM = 16 * fwd::kMT;
  // host-built tile table: prefix sums of ceil(M_g / BM); empty groups get no tiles
  int* starts = new int[a.num_groups + 1];
  int total = 0;
  size_t lds = 0;
  for (int gi = 0; gi < a.num_groups; ++gi) {
    starts[gi] = total;
    total += (int)((a.groups[gi].M + BM - 1) / BM);
    const size_t l = fwd::fwd_lds_bytes(BM, (int)a.groups[gi].K, (int)a.groups[gi].N);
    if (l > lds) lds = l;
  }
  starts[a.num_groups] = total;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const size_t gbytes = ((size_t)a.num_groups * sizeof(GroupDev) + 255) / 256 * 256;
  GroupDev* dgroups = reinterpret_cast<GroupDev*>(ws);
  int* dstarts = reinterpret_cast<int*>(ws + gbytes);
  // pageable host sources: the runtime stages them before these calls return
  hipError_t e = hipMemcpyAsync(dgroups, a.groups, (size_t)a.num_groups * sizeof(GroupDev), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dstarts, starts, (size_t)(a.num_groups + 1) * sizeof(int), hipMemcpyHostToDevice, s);
  delete[] starts;
  if (e != hipSuccess) return e;
  if (total == 0) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(fwd::k_grouped), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd::k_grouped, dim3((unsigned)total), dim3(fwd::kThreads), lds, s, dgroups, dstarts, a.num_groups, a.eps);
  return hipGetLastError();
}

}  // namespace loka
