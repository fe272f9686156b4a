// loka_grouped_gemm_fp8_ln: many independent rowwise forwards in one call: one
// persistent launch when every group has N <= 384, K <= 512 and a guarded
// shape (k_grouped_mixed), else one persistent launch per register shape
// class of the groups.
//
// Source: LoKA section I (wide ensembles of small layers); GEM "Generalized
// Dot-Product Attention" (tile lists precomputed instead of discovered by
// every block, empty tiles skipped) and "Expert Parallelism" (one expert per
// rank).
//
// Launches on the caller's stream:
//  1. The plan: normally computed on the host and passed by value to each
//     class launch (GroupPlan, at most 256 groups per class and 256
//     workgroups); for larger problems k_grouped_plan (one workgroup) reads
//     the group descriptors and writes
//     the plan into the workspace, per shape class (column tiles per
//     wavefront NT = ceil(N/128), and whether the shape is the guard-free
//     FULL case): the first global 16-row tile of every group of the class
//     (exclusive prefix sums of ceil(M_g/16), other classes counting as
//     empty) and the first tile of every persistent workgroup, chosen so
//     that each workgroup gets an equal share of the estimated cost (bytes
//     moved per tile, 32(K_g+N_g), plus a fixed per-tile term, tile_cost).
//  2. without packed weights, k_relayout_groups rearranges every group's
//     row-major weight into the fragment-interleaved layout the resident
//     block reads (group g at g * stride in the workspace);
//  3. per class present, k_grouped_res<NT, FULL> (one persistent workgroup
//     per compute unit) walks its contiguous range of the class's tiles
//     group by group; for each group it loads that group's weight into
//     registers and runs exactly the weight-resident block of the single
//     forward (fwd_resident.hpp) over its tiles of that group.  The per-tile
//     arithmetic is the same as a single loka_gemm_fp8_ln call's, so every
//     group's output is bit-identical to one.  (One kernel per class keeps
//     each kernel's registers to one block variant.)
#include "fwd_resident.hpp"

namespace loka {
namespace fwd {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kMaxGroups = 2048;

// Where the groups' fragment-interleaved weights are: the descriptors' own
// qw (base == nullptr) or the workspace copy of group g at base + g*stride.
struct WeightSrc {
  const uint8_t* base;
  int64_t stride;
};
__device__ __forceinline__ const uint8_t* group_weight(const WeightSrc& w, const GroupDev& gd, int g) {
  return w.base != nullptr ? w.base + (int64_t)g * w.stride : gd.qw;
}

// Every group's [N][K] weight codes -> fragment-interleaved at dst + g*stride
// (grid.y = group, one thread per 16-byte destination piece).
__global__ __launch_bounds__(256) void k_relayout_groups(const GroupDev* groups, uint8_t* dst, int64_t stride) {
  const GroupDev gd = groups[blockIdx.y];
  const int64_t nch = (gd.K + 127) / 128, pieces = nch * 8;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= gd.N * pieces) return;
  const int64_t row = u / pieces, col = (u - row * pieces) * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (col < gd.K) v = *reinterpret_cast<const uint4*>(gd.qw + row * gd.K + col);
  *reinterpret_cast<uint4*>(dst + (int64_t)blockIdx.y * stride + ilv_offset(row, col, nch)) = v;
}

// estimated cost of one 16-row tile: bytes of X read and Y written, plus a
// fixed term for the per-tile reductions, synchronization and latencies.  The
// fixed term was fitted on the 64-group workload (K and N in 128..384): its
// steps cost about 1.1 us at K = N = 128 and 2 us at K = N = 384, so most of a
// small tile's cost is fixed.  With 12288 the launch took 183 us, with 2048
// 209 us (the workgroups holding small groups finished last), and with
// 20480 or 32768, 189 and 197 us.
__host__ __device__ inline int64_t tile_cost(int64_t K, int64_t N) { return 32 * (K + N) + 12288; }

constexpr int kClasses = 2 * kResShapes;  // (NT, KC) shape x FULL or not
constexpr int kMaxGrid = 1024;    // workgroups per class launch

// Resident chunk count of a group: 4 for K <= 512, else the maximum.  Fewer
// classes mean fewer launches (each pays a weight prologue and a drain);
// the chunk count only sizes the registers, the per-tile arithmetic over
// ceil(K/128) chunks is the single forward's whatever it is.
__host__ __device__ inline int group_kc(int nt, int K) { return (K + 127) / 128 <= 4 ? 4 : res_kc_max(nt); }
// shape class of a group: 2 res_shape(NT, KC) + FULL
__host__ __device__ inline int group_class(int64_t M, int64_t N, int64_t K) {
  const int nt = res_nt((int)N), kc = group_kc(nt, (int)K);
  return 2 * res_shape(nt, kc) + (res_full(M, (int)N, (int)K, nt, kc) ? 1 : 0);
}

// The plan's tile range a workgroup walks.  Workgroups go to the eight XCDs
// round-robin (w % 8); with n % 8 == 0, workgroup w takes range
// (w % 8) n/8 + w / 8, so consecutive ranges (mostly tiles of the same
// groups) run on one XCD and each group's weight is fetched into one L2.
__device__ __forceinline__ int plan_range(int w, int n) { return (n & 7) == 0 ? (w & 7) * (n >> 3) + (w >> 3) : w; }

// The plan of one class as a kernel argument (by value, so a captured graph
// replays it without any host copy): the class's groups, their exclusive
// prefix of 16-row tiles, and each workgroup's first tile.
constexpr int kPlanGroups = 256;
struct GroupPlan {
  int ngroups;
  int grid;
  int gid[kPlanGroups];
  int tile_pre[kPlanGroups + 1];
  int wg_start[kPlanGroups + 1];
};

// plan of class c: tile_pre[c][G+1], wg_start[c][kMaxGrid+1]; grid[c] workgroups
__global__ __launch_bounds__(kPlanThreads) void k_grouped_plan(const GroupDev* groups, int G, int cus,
                                                                 int* tile_pre, int* wg_start) {
  __shared__ int64_t cpre[kMaxGroups + 1];   // exclusive prefix of group costs
  __shared__ int tpre[kMaxGroups + 1];       // exclusive prefix of group tiles
  __shared__ int64_t ccost[kMaxGroups];      // per-tile cost of each group
  __shared__ int64_t sc[kPlanThreads];
  __shared__ int st[kPlanThreads];
  const int tid = threadIdx.x;
  for (int cls = 0; cls < kClasses; ++cls) {
    int64_t carry_c = 0;
    int carry_t = 0;
    for (int base = 0; base < G; base += kPlanThreads) {
      const int i = base + tid;
      int tiles = 0;
      int64_t cost = 0;
      if (i < G) {
        const GroupDev& gd = groups[i];
        ccost[i] = tile_cost(gd.K, gd.N);
        if (group_class(gd.M, gd.N, gd.K) == cls) {
          tiles = (int)((gd.M + kResRows - 1) / kResRows);
          cost = (int64_t)tiles * ccost[i];
        }
      }
      sc[tid] = cost;
      st[tid] = tiles;
      __syncthreads();
      for (int o = 1; o < kPlanThreads; o <<= 1) {  // inclusive scan (Hillis-Steele)
        const int64_t a = tid >= o ? sc[tid - o] : 0;
        const int b = tid >= o ? st[tid - o] : 0;
        __syncthreads();
        sc[tid] += a;
        st[tid] += b;
        __syncthreads();
      }
      if (i < G) {
        cpre[i] = carry_c + sc[tid] - cost;
        tpre[i] = carry_t + st[tid] - tiles;
      }
      carry_c += sc[kPlanThreads - 1];
      carry_t += st[kPlanThreads - 1];
      __syncthreads();
    }
    if (tid == 0) {
      cpre[G] = carry_c;
      tpre[G] = carry_t;
    }
    __syncthreads();
    int* tp = tile_pre + cls * (G + 1);
    int* ws = wg_start + cls * (kMaxGrid + 1);
    for (int i = tid; i <= G; i += kPlanThreads) tp[i] = tpre[i];
    // workgroup b starts at the first tile whose starting cost is >= b*C/grid
    const int64_t C = cpre[G];
    const int grid = (int)(tpre[G] < cus ? tpre[G] : cus);
    for (int b = tid; b <= grid; b += kPlanThreads) {
      int start;
      if (b == grid) {
        start = tpre[G];
      } else {
        const int64_t x = (C / grid) * b + ((C % grid) * b) / grid;
        int lo = 0, hi = G - 1;  // last group with cpre[g] <= x
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (cpre[mid] <= x) lo = mid;
          else hi = mid - 1;
        }
        const int tiles_g = tpre[lo + 1] - tpre[lo];
        int64_t j = tiles_g == 0 ? 0 : (x - cpre[lo] + ccost[lo] - 1) / ccost[lo];
        if (j > tiles_g) j = tiles_g;
        start = tpre[lo] + (int)j;
      }
      ws[b] = start;
    }
    __syncthreads();  // cpre/tpre are rebuilt for the next class
  }
}

// the resident block's arguments for one group (rowwise X, no optional
// statistics or context outputs)
__device__ __forceinline__ FwdBlock group_block(const GroupDev& gd, const uint8_t* qw, float eps) {
  FwdBlock p{};
  p.M = gd.M; p.N = (int)gd.N; p.K = (int)gd.K;
  p.x = static_cast<const uint16_t*>(gd.x);
  p.qw = qw; p.sw = gd.sw;
  p.ldy = (int)gd.N;
  p.bias = static_cast<const uint16_t*>(gd.bias);
  p.gamma = static_cast<const uint16_t*>(gd.gamma);
  p.beta = static_cast<const uint16_t*>(gd.beta);
  p.y = static_cast<uint16_t*>(gd.y);
  p.z = gd.z;
  p.eps = eps; p.x_r = 1.0f; p.x_s = 1.0f;
  return p;
}

template <bool OPT, int NT, int KC, bool FULL>
__global__ __launch_bounds__(kThreads) void k_grouped_res(const GroupDev* groups, const int* tile_pre,
                                                          const int* wg_start, int G, float eps, WeightSrc wsrc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wr = plan_range((int)blockIdx.x, (int)gridDim.x);
  int t = wg_start[wr];
  const int tend = wg_start[wr + 1];
  int lo = 0, hi = G - 1;  // last group with tile_pre[g] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  int g = lo;
  while (t < tend) {
    while (tile_pre[g + 1] <= t) ++g;  // past finished groups and those of other classes
    const int seg_end = min(tend, tile_pre[g + 1]);
    const FwdBlock p = group_block(groups[g], group_weight(wsrc, groups[g], g), eps);
    ResBlock<1, NT, KC, OPT, FULL> blk(p, t - tile_pre[g], seg_end - tile_pre[g], smem);
    blk.run();
    __syncthreads();  // the next group's set-up rewrites the LDS
    t = seg_end;
  }
}

// the same walk, with the plan as an argument (group index through gid)
template <bool OPT, int NT, int KC, bool FULL>
__global__ __launch_bounds__(kThreads) void k_grouped_res_arg(const GroupDev* groups, GroupPlan plan, float eps,
                                                              WeightSrc wsrc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wr = plan_range((int)blockIdx.x, (int)gridDim.x);
  int t = plan.wg_start[wr];
  const int tend = plan.wg_start[wr + 1];
  int lo = 0, hi = plan.ngroups - 1;  // last class group with tile_pre <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan.tile_pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  int q = lo;
  while (t < tend) {
    while (plan.tile_pre[q + 1] <= t) ++q;  // past finished and empty groups
    const int seg_end = min(tend, plan.tile_pre[q + 1]);
    const FwdBlock p = group_block(groups[plan.gid[q]], group_weight(wsrc, groups[plan.gid[q]], plan.gid[q]), eps);
    ResBlock<1, NT, KC, OPT, FULL> blk(p, t - plan.tile_pre[q], seg_end - plan.tile_pre[q], smem);
    blk.run();
    __syncthreads();  // the next group's set-up rewrites the LDS
    t = seg_end;
  }
}

// Every group in one launch when all have N <= 384, K <= 512 and guarded
// (not FULL) shapes: the same walk over one plan of all the groups, and each
// group's segment runs the block variant of its column-tile count
// (N <= 128 NT).  The variants share the 4-chunk weight footprint, so the
// kernel's registers are those of the widest (with N = 512 they would
// spill).
template <int NT, bool OPT>
__device__ __forceinline__ void run_group(const FwdBlock& p, int64_t tb, int64_t te, uint8_t* smem) {
  // K <= 256: the block of two K chunks (one 16-byte X load per lane per
  // tile, so eight tiles in flight), two tiles per step (its four-buffer LDS
  // layout is part of the launch's size)
  if (p.K <= 256) {
    ResBlock<1, NT, 2, OPT, false, 0, false, true> blk(p, tb, te, smem);
    blk.run();
  } else {
    // four K chunks: two tiles per step too where the registers allow
    ResBlock<1, NT, 4, OPT, false, 0, false, (NT <= 2)> blk(p, tb, te, smem);
    blk.run();
  }
}
template <bool OPT>
__global__ __launch_bounds__(kThreads) void k_grouped_mixed(const GroupDev* groups, GroupPlan plan, float eps,
                                                            WeightSrc wsrc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wr = plan_range((int)blockIdx.x, (int)gridDim.x);
  int t = plan.wg_start[wr];
  const int tend = plan.wg_start[wr + 1];
  int lo = 0, hi = plan.ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan.tile_pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  int q = lo;
  while (t < tend) {
    while (plan.tile_pre[q + 1] <= t) ++q;
    const int seg_end = min(tend, plan.tile_pre[q + 1]);
    const int gi = plan.gid[q];
    const FwdBlock p = group_block(groups[gi], group_weight(wsrc, groups[gi], gi), eps);
    const int64_t tb = t - plan.tile_pre[q], te = seg_end - plan.tile_pre[q];
    switch (res_nt(p.N)) {
      case 1: run_group<1, OPT>(p, tb, te, smem); break;
      case 2: run_group<2, OPT>(p, tb, te, smem); break;
      default: run_group<3, OPT>(p, tb, te, smem); break;
    }
    __syncthreads();  // the next group's set-up rewrites the LDS
    t = seg_end;
  }
}

template <bool OPT>
hipError_t launch_mixed(const GroupDev* dg, const GroupPlan& plan, size_t lds, float eps, WeightSrc w,
                        hipStream_t s) {
  auto kern = k_grouped_mixed<OPT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.grid), dim3(kThreads), lds, s, dg, plan, eps, w);
  return hipGetLastError();
}

template <bool OPT, int NT, int KC, bool FULL>
hipError_t launch_class_arg(const GroupDev* dg, const GroupPlan& plan, size_t lds, float eps, WeightSrc w,
                            hipStream_t s) {
  auto kern = k_grouped_res_arg<OPT, NT, KC, FULL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.grid), dim3(kThreads), lds, s, dg, plan, eps, w);
  return hipGetLastError();
}

template <bool OPT, int NT, int KC, bool FULL>
hipError_t launch_class(const GroupDev* dg, const int* tp, const int* ws, int G, int grid, size_t lds, float eps,
                        WeightSrc w, hipStream_t s) {
  auto kern = k_grouped_res<OPT, NT, KC, FULL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, dg, tp, ws, G, eps, w);
  return hipGetLastError();
}

}  // namespace
}  // namespace fwd

int grouped_max_groups() { return fwd::kMaxGroups; }

namespace {
// stride of the packed weight copies: the largest group's, 256-byte aligned
size_t packed_stride(int num_groups, const GroupDev* groups) {
  size_t m = 0;
  for (int i = 0; i < num_groups; ++i) {
    const size_t b = ilv_bytes(groups[i].N, groups[i].K);
    if (b > m) m = b;
  }
  return (m + 255) / 256 * 256;
}
size_t plan_bytes(int num_groups) {
  size_t b = ((size_t)num_groups * sizeof(GroupDev) + 255) / 256 * 256;
  b += ((size_t)fwd::kClasses * (num_groups + 1) * sizeof(int) + 255) / 256 * 256;
  b += ((size_t)fwd::kClasses * (fwd::kMaxGrid + 1) * sizeof(int) + 255) / 256 * 256;
  return b;
}
// the plan of the groups `take` selects, in descriptor order: each one's
// first 16-row tile, and for each of min(tiles, cus) workgroups the first
// tile whose starting cost reaches its equal share of the total
template <class Take>
void host_plan_of(const GroupDev* groups, int G, int cus, Take take, fwd::GroupPlan& plan) {
  plan.ngroups = 0;
  int64_t cost_pre[fwd::kPlanGroups + 1];
  int64_t ccost[fwd::kPlanGroups];
  int64_t tp = 0, cp = 0;
  for (int gi = 0; gi < G; ++gi) {
    const GroupDev& gd = groups[gi];
    if (!take(gd)) continue;
    const int q = plan.ngroups++;
    plan.gid[q] = gi;
    plan.tile_pre[q] = (int)tp;
    cost_pre[q] = cp;
    ccost[q] = fwd::tile_cost(gd.K, gd.N);
    const int64_t tl = (gd.M + fwd::kResRows - 1) / fwd::kResRows;
    tp += tl;
    cp += tl * ccost[q];
  }
  const int ng = plan.ngroups;
  plan.tile_pre[ng] = (int)tp;
  cost_pre[ng] = cp;
  const int grid = (int)(tp < cus ? tp : cus);
  plan.grid = grid;
  for (int b = 0; b <= grid; ++b) {
    if (b == grid) {
      plan.wg_start[b] = (int)tp;
      continue;
    }
    const int64_t x = (cp / grid) * b + ((cp % grid) * b) / grid;
    int q = 0;
    while (q + 1 < ng && cost_pre[q + 1] <= x) ++q;
    const int64_t tq = plan.tile_pre[q + 1] - plan.tile_pre[q];
    int64_t j = tq == 0 ? 0 : (x - cost_pre[q] + ccost[q] - 1) / ccost[q];
    if (j > tq) j = tq;
    plan.wg_start[b] = plan.tile_pre[q] + (int)j;
  }
}
}  // namespace

// workspace: [ descriptors | tile_pre [classes][G+1] | wg_start [classes][kMaxGrid+1] |
//              packed weights [G][stride] (without LOKA_FWD_W_PACKED) ]
size_t grouped_workspace_bytes(int num_groups, const GroupDev* groups, bool w_packed) {
  size_t b = plan_bytes(num_groups);
  if (!w_packed) b += (size_t)num_groups * packed_stride(num_groups, groups);
  return b;
}

hipError_t launch_grouped(const GroupedLaunch& a, hipStream_t s) {
  const int G = a.num_groups;
  int64_t tiles[fwd::kClasses] = {0};
  size_t lds[fwd::kClasses] = {0};
  bool opt = false;
  for (int gi = 0; gi < G; ++gi) {
    const GroupDev& gd = a.groups[gi];
    const int c = fwd::group_class(gd.M, gd.N, gd.K);
    tiles[c] += (gd.M + fwd::kResRows - 1) / fwd::kResRows;
    const int nt = fwd::res_nt((int)gd.N);
    const size_t l = (size_t)fwd::res_lds(nt, fwd::group_kc(nt, (int)gd.K), (int)gd.N).total;
    if (l > lds[c]) lds[c] = l;
    if (gd.z != nullptr) opt = true;
  }
  int64_t total = 0;
  for (int c = 0; c < fwd::kClasses; ++c) total += tiles[c];
  if (total == 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const size_t gbytes = ((size_t)G * sizeof(GroupDev) + 255) / 256 * 256;
  const size_t tbytes = ((size_t)fwd::kClasses * (G + 1) * sizeof(int) + 255) / 256 * 256;
  GroupDev* dgroups = reinterpret_cast<GroupDev*>(ws);
  int* tile_pre = reinterpret_cast<int*>(ws + gbytes);
  int* wg_start = reinterpret_cast<int*>(ws + gbytes + tbytes);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus > fwd::kMaxGrid) cus = fwd::kMaxGrid;
  // the caller's descriptor array is the copy's source (it must stay valid
  // until the copy has run)
  e = hipMemcpyAsync(dgroups, a.groups, (size_t)G * sizeof(GroupDev), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  fwd::WeightSrc wsrc{nullptr, 0};
  if (!a.w_packed) {
    const size_t stride = packed_stride(G, a.groups);
    int64_t pieces = 0;
    for (int gi = 0; gi < G; ++gi) {
      const int64_t pc = a.groups[gi].N * ((a.groups[gi].K + 127) / 128) * 8;
      if (pc > pieces) pieces = pc;
    }
    uint8_t* wpk = ws + plan_bytes(G);
    hipLaunchKernelGGL(fwd::k_relayout_groups, dim3((unsigned)((pieces + 255) / 256), (unsigned)G), dim3(256), 0, s,
                       dgroups, wpk, (int64_t)stride);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    wsrc = fwd::WeightSrc{wpk, (int64_t)stride};
  }
  // host plans (passed by value) when every class fits GroupPlan
  int ngc[fwd::kClasses] = {0};
  for (int gi = 0; gi < G; ++gi) {
    const GroupDev& gd = a.groups[gi];
    ++ngc[fwd::group_class(gd.M, gd.N, gd.K)];
  }
  bool host_plan = cus <= fwd::kPlanGroups;
  for (int c = 0; c < fwd::kClasses; ++c) host_plan = host_plan && ngc[c] <= fwd::kPlanGroups;
  if (host_plan) {
    // one launch for every group when all groups with rows have N <= 384,
    // K <= 512 and guarded shapes
    bool mixed = true;
    int nrows = 0;
    size_t lmax = 0;
    for (int gi = 0; gi < G; ++gi) {
      const GroupDev& gd = a.groups[gi];
      if (gd.M == 0) continue;
      ++nrows;
      const int nt = fwd::res_nt((int)gd.N);
      if (nt > 3 || fwd::group_kc(nt, (int)gd.K) != 4 || (fwd::group_class(gd.M, gd.N, gd.K) & 1)) mixed = false;
      // the layout run_group uses: two K chunks and four buffers for K <= 256
      const size_t l =
          (size_t)(gd.K <= 256 ? fwd::res_lds(nt, 2, (int)gd.N, 4) : fwd::res_lds(nt, 4, (int)gd.N, nt <= 2 ? 4 : 2)).total;
      if (l > lmax) lmax = l;
    }
    if (mixed && nrows <= fwd::kPlanGroups) {
      fwd::GroupPlan plan;
      host_plan_of(a.groups, G, cus, [](const GroupDev& gd) { return gd.M > 0; }, plan);
      return opt ? fwd::launch_mixed<true>(dgroups, plan, lmax, a.eps, wsrc, s)
                 : fwd::launch_mixed<false>(dgroups, plan, lmax, a.eps, wsrc, s);
    }
    for (int c = 0; c < fwd::kClasses && e == hipSuccess; ++c) {
      if (tiles[c] == 0) continue;
      fwd::GroupPlan plan;
      host_plan_of(a.groups, G, cus,
                   [c](const GroupDev& gd) { return fwd::group_class(gd.M, gd.N, gd.K) == c; }, plan);
#define LOKA_CLASS(S, NT, KC)                                                                     \
  case 2 * S:                                                                                    \
    e = opt ? fwd::launch_class_arg<true, NT, KC, false>(dgroups, plan, lds[c], a.eps, wsrc, s)        \
            : fwd::launch_class_arg<false, NT, KC, false>(dgroups, plan, lds[c], a.eps, wsrc, s);      \
    break;                                                                                       \
  case 2 * S + 1:                                                                                \
    e = opt ? fwd::launch_class_arg<true, NT, KC, true>(dgroups, plan, lds[c], a.eps, wsrc, s)         \
            : fwd::launch_class_arg<false, NT, KC, true>(dgroups, plan, lds[c], a.eps, wsrc, s);       \
    break;
      switch (c) {
        LOKA_CLASS(1, 1, 4) LOKA_CLASS(2, 1, 8) LOKA_CLASS(4, 2, 4) LOKA_CLASS(5, 2, 8) LOKA_CLASS(7, 3, 4)
        LOKA_CLASS(8, 3, 5) LOKA_CLASS(10, 4, 4)
        default: break;
      }
#undef LOKA_CLASS
    }
    return e;
  }
  hipLaunchKernelGGL(fwd::k_grouped_plan, dim3(1), dim3(fwd::kPlanThreads), 0, s, dgroups, G, cus, tile_pre,
                     wg_start);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int c = 0; c < fwd::kClasses && e == hipSuccess; ++c) {
    if (tiles[c] == 0) continue;
    const int grid = (int)(tiles[c] < cus ? tiles[c] : cus);
    const int* tp = tile_pre + c * (G + 1);
    const int* wsc = wg_start + c * (fwd::kMaxGrid + 1);
#define LOKA_CLASS(S, NT, KC)                                                                                \
  case 2 * S:                                                                                               \
    e = opt ? fwd::launch_class<true, NT, KC, false>(dgroups, tp, wsc, G, grid, lds[c], a.eps, wsrc, s)           \
            : fwd::launch_class<false, NT, KC, false>(dgroups, tp, wsc, G, grid, lds[c], a.eps, wsrc, s);         \
    break;                                                                                                  \
  case 2 * S + 1:                                                                                           \
    e = opt ? fwd::launch_class<true, NT, KC, true>(dgroups, tp, wsc, G, grid, lds[c], a.eps, wsrc, s)            \
            : fwd::launch_class<false, NT, KC, true>(dgroups, tp, wsc, G, grid, lds[c], a.eps, wsrc, s);          \
    break;
    switch (c) {
      LOKA_CLASS(1, 1, 4) LOKA_CLASS(2, 1, 8) LOKA_CLASS(4, 2, 4) LOKA_CLASS(5, 2, 8) LOKA_CLASS(7, 3, 4)
      LOKA_CLASS(8, 3, 5) LOKA_CLASS(10, 4, 4)
      default: break;
    }
#undef LOKA_CLASS
  }
  return e;
}

}  // namespace loka
