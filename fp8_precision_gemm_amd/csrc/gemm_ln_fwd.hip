// Fused FP8 GEMM + LayerNorm forward (loka_gemm_fp8_ln) and its grouped
// form (loka_grouped_gemm_fp8_ln) for gfx950.
//
// Source: LoKA section III-B2 (Block-wise Normalization): the normalization
// runs in the GEMM epilogue while the output tile is still on chip, and in
// Case 1 (large batch, small output dimension) a whole output row lives in
// one block, so the result is the standard normalization; section III-B:
// the GEMM output is dequantized and the LayerNorm runs in high precision;
// section III-B1 (No Bias).  GEM "Mixed Ultra-Low-Precision Training":
// activation quantization fused into the neighbouring kernel instead of an
// extra pass over HBM; "Low Precision Flash Attention": MX block scales
// along K.  GEM "Generalized Dot-Product Attention": the grouped launch
// walks a tile list built on the host.
//
// One workgroup (4 wavefronts) owns BM = 16*MT rows and all N columns:
//  1. each wavefront loads 4*MT rows of X (bf16, 16 B per lane), takes the
//     row (or 32-block) max-abs by a wavefront reduction, and writes the
//     FP8 codes to LDS (rows padded by 16 B against bank conflicts);
//  2. wavefront w computes columns [w*N/4, (w+1)*N/4) for all BM rows with
//     v_mfma_scale_f32_16x16x128_f8f6f4: A = W^T rows (streamed from
//     L2/HBM, each byte used by one wavefront only), B = the X codes in LDS;
//  3. the epilogue keeps the accumulators in registers: dequant + bias,
//     row mean (and row max-abs), then the centred sum of squares (two
//     passes over registers, one LDS exchange each), then gamma/beta and one
//     bf16 store.
// X is read from HBM once and Y written once; nothing else reaches HBM
// unless the optional outputs are requested.
#include "common.hpp"
#include "launch.hpp"

namespace loka {
namespace {

struct FwdBlock {
  int64_t M;
  int N, K;
  const uint16_t* x;
  const uint8_t* qw;
  const void* sw;
  const uint16_t* bias;
  const uint16_t* gamma;
  const uint16_t* beta;
  uint16_t* y;
  float* z;
  float* mean;
  float* rstd;
  uint8_t* qx_out;
  void* sx_out;
  float eps;
  float x_r, x_s;  // tensor mode: X multiplier and dequantization scale
};

constexpr int kMaxKChunks = 4;  // K <= 2048 (512 bf16 per wavefront load)

__host__ __device__ constexpr int lds_stride(int K) { return K + 16; }
__host__ __device__ inline size_t fwd_lds_bytes(int BM, int K) {
  size_t b = (size_t)BM * lds_stride(K);       // X codes
  b += (size_t)BM * 4;                         // row scales
  b += ((size_t)BM * (K / 32) + 15) / 16 * 16; // MX scales
  b += (size_t)2 * 4 * BM * 4;                 // two reduction buffers
  return b;
}

// Power-of-two factor c <= 1 for a row whose largest magnitude is 2^e or
// more: with e >= 55, N * (z - mean)^2 could overflow fp32 (N <= 1024), so
// the deviations are scaled by c = 2^(40 - e) (exact) before squaring.
// Ordinary rows get c = 1 and exactly the unscaled arithmetic.
__device__ __forceinline__ float row_rescale(float maxabs) {
  const int e = (int)((__float_as_uint(maxabs) >> 23) & 0xFF) - 127;  // floor(log2) for normal values
  return e >= 55 ? __uint_as_float((uint32_t)(167 - e) << 23) : 1.0f;
}

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float def, float o[4]) {
  if (p == nullptr) {
    o[0] = o[1] = o[2] = o[3] = def;
    return;
  }
  uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
}

// MODE: 0 tensor, 1 row, 3 mx32.  NTMAX: max 16-column tiles per wavefront
// (N / 64 <= NTMAX).  MT: 16-row tiles per workgroup.
template <int MODE, int NTMAX, int MT>
__device__ __forceinline__ void fwd_block(const FwdBlock& p, int64_t m0, uint8_t* smem) {
  constexpr int BM = 16 * MT;
  constexpr int RPW = BM / 4;  // rows quantized per wavefront
  const int K = p.K, N = p.N;
  const int ldk = lds_stride(K);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kb = K / 32;  // MX blocks per row

  uint8_t* xs = smem;
  float* rs = reinterpret_cast<float*>(smem + (size_t)BM * ldk);
  uint8_t* xe8 = reinterpret_cast<uint8_t*>(rs + BM);
  float* red0 = reinterpret_cast<float*>(xe8 + ((size_t)BM * kb + 15) / 16 * 16);
  float* red1 = red0 + 4 * BM;

  // ---- 1. quantize this block's rows of X into LDS ------------------------
  const int nch = (K + 511) / 512;
#pragma unroll 2
  for (int rr = 0; rr < RPW; ++rr) {
    const int lr = wave * RPW + rr;
    const int64_t m = m0 + lr;
    float v[kMaxKChunks][8];
#pragma unroll
    for (int c = 0; c < kMaxKChunks; ++c) {
      const int k = c * 512 + lane * 8;
      if (c < nch && k < K && m < p.M) {
        uint4 u = *reinterpret_cast<const uint4*>(p.x + m * K + k);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[c][2 * i] = bf16_lo(w[i]);
          v[c][2 * i + 1] = bf16_hi(w[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = 0.0f;
      }
    }
    if (MODE == 3) {
#pragma unroll
      for (int c = 0; c < kMaxKChunks; ++c) {
        if (c >= nch) break;
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[c][i]));
        a = fmaxf(a, __shfl_xor(a, 1, 64));  // 4 lanes hold one 32-element block
        a = fmaxf(a, __shfl_xor(a, 2, 64));
        const int e8 = e8m0_from_amax<0>(a);
        const float mu = e8m0_inv_multiplier(e8);
        const int k = c * 512 + lane * 8;
        if (k < K) {
          if ((lane & 3) == 0) xe8[lr * kb + k / 32] = (uint8_t)e8;
          uint32_t lo = cvt4<0>(v[c][0] * mu, v[c][1] * mu, v[c][2] * mu, v[c][3] * mu);
          uint32_t hi = cvt4<0>(v[c][4] * mu, v[c][5] * mu, v[c][6] * mu, v[c][7] * mu);
          *reinterpret_cast<uint2*>(xs + lr * ldk + k) = make_uint2(lo, hi);
        }
      }
    } else {
      float r;
      if (MODE == 1) {
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxKChunks; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[c][i]));
        a = wave_max(a);
        ScalePair sp = scales_from_amax<0>(a);
        if (lane == 0) rs[lr] = sp.s;
        r = sp.r;
      } else {
        r = p.x_r;
      }
#pragma unroll
      for (int c = 0; c < kMaxKChunks; ++c) {
        const int k = c * 512 + lane * 8;
        if (c < nch && k < K) {
          uint32_t lo = cvt4<0>(v[c][0] * r, v[c][1] * r, v[c][2] * r, v[c][3] * r);
          uint32_t hi = cvt4<0>(v[c][4] * r, v[c][5] * r, v[c][6] * r, v[c][7] * r);
          *reinterpret_cast<uint2*>(xs + lr * ldk + k) = make_uint2(lo, hi);
        }
      }
    }
  }
  __syncthreads();

  // optional: the quantized X (bit-identical to loka_quant_fp8) for the backward
  if (p.qx_out != nullptr) {
    const int k16 = K / 16;
    for (int u = tid; u < BM * k16; u += 256) {
      const int lr = u / k16, c = (u - lr * k16) * 16;
      if (m0 + lr < p.M)
        *reinterpret_cast<uint4*>(p.qx_out + (m0 + lr) * K + c) = *reinterpret_cast<const uint4*>(xs + lr * ldk + c);
    }
  }
  if (p.sx_out != nullptr) {
    if (MODE == 1) {
      if (tid < BM && m0 + tid < p.M) static_cast<float*>(p.sx_out)[m0 + tid] = rs[tid];
    } else if (MODE == 3) {
      for (int u = tid; u < BM * kb; u += 256) {
        const int lr = u / kb;
        if (m0 + lr < p.M) static_cast<uint8_t*>(p.sx_out)[(m0 + lr) * kb + (u - lr * kb)] = xe8[u];
      }
    } else if (m0 == 0 && tid == 0) {
      static_cast<float*>(p.sx_out)[0] = p.x_s;
    }
  }

  // ---- 2. GEMM: D[n][m] = sum_k W^T[n][k] X[m][k] ---------------------------
  const int nt = N / 64;
  const int r = lane & 15, g = lane >> 4;
  const int nb = wave * nt * 16;
  v4f acc[NTMAX][MT];
#pragma unroll
  for (int t = 0; t < NTMAX; ++t)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[t][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* sw8 = static_cast<const uint8_t*>(p.sw);
  for (int kc = 0; kc < K; kc += 128) {
    v8i xf[MT];
    int xsc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      xf[i] = load_frag(xs + (16 * i + r) * ldk, g, kc, K);
      if (MODE == 3) {
        const int blk = kc / 32 + g;
        xsc[i] = blk < kb ? (int)xe8[(16 * i + r) * kb + blk] : 127;
      }
    }
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
      if (t < nt) {
        const int n = nb + 16 * t + r;
        const v8i wf = load_frag(p.qw + (int64_t)n * K, g, kc, K);
        if (MODE == 3) {
          const int blk = kc / 32 + g;
          const int wsc = blk < kb ? (int)sw8[(int64_t)n * kb + blk] : 127;
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[t][i] = mfma_mx_e4m3(wf, xf[i], acc[t][i], wsc, xsc[i]);
        } else {
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[t][i] = mfma_fp8<0, 0>(wf, xf[i], acc[t][i]);
        }
      }
    }
  }

  // ---- 3. epilogue: dequant + bias, LayerNorm, bf16 store -------------------
  // lane (r, g) holds, for tile t and row tile i: n = nb + 16t + 4g + j, m = 16i + r
  float sxv[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) sxv[i] = MODE == 1 ? rs[16 * i + r] : (MODE == 0 ? p.x_s : 1.0f);
  float psum[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) psum[i] = 0.0f;
#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    if (t < nt) {
      const int n0 = nb + 16 * t + 4 * g;
      float swv[4], bv[4];
      if (MODE == 1) {
        float4 s4 = *reinterpret_cast<const float4*>(static_cast<const float*>(p.sw) + n0);
        swv[0] = s4.x; swv[1] = s4.y; swv[2] = s4.z; swv[3] = s4.w;
      } else {
        const float s0 = MODE == 0 ? static_cast<const float*>(p.sw)[0] : 1.0f;
        swv[0] = swv[1] = swv[2] = swv[3] = s0;
      }
      load4_bf16(p.bias ? p.bias + n0 : nullptr, 0.0f, bv);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float zz = MODE == 3 ? acc[t][i][j] + bv[j] : acc[t][i][j] * sxv[i] * swv[j] + bv[j];
          acc[t][i][j] = zz;
          psum[i] += zz;
        }
      }
    }
  }
  // row sums and row max-abs in one exchange; rows whose values are so large
  // that their squares would overflow fp32 are rescaled by a power of two
  // (exact) for the variance, so every finite row normalizes correctly
  float pmax[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) pmax[i] = 0.0f;
#pragma unroll
  for (int t = 0; t < NTMAX; ++t)
    if (t < nt)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) pmax[i] = fmaxf(pmax[i], fabsf(acc[t][i][j]));
  const float invn = 1.0f / (float)N;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    psum[i] = group4_sum(psum[i]);
    pmax[i] = fmaxf(pmax[i], __shfl_xor(pmax[i], 16, 64));
    pmax[i] = fmaxf(pmax[i], __shfl_xor(pmax[i], 32, 64));
    if (g == 0) {
      red0[wave * BM + 16 * i + r] = psum[i];
      red1[wave * BM + 16 * i + r] = pmax[i];
    }
  }
  __syncthreads();
  float mu[MT], cs[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int rr = 16 * i + r;
    mu[i] = (red0[rr] + red0[BM + rr] + red0[2 * BM + rr] + red0[3 * BM + rr]) * invn;
    const float mx = fmaxf(fmaxf(red1[rr], red1[BM + rr]), fmaxf(red1[2 * BM + rr], red1[3 * BM + rr]));
    cs[i] = row_rescale(mx);
  }
  __syncthreads();  // red0/red1 are reused below
  float psq[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) psq[i] = 0.0f;
#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    if (t < nt) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = (acc[t][i][j] - mu[i]) * cs[i];
          psq[i] += d * d;
        }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    psq[i] = group4_sum(psq[i]);
    if (g == 0) red0[wave * BM + 16 * i + r] = psq[i];
  }
  __syncthreads();
  float rsd[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int rr = 16 * i + r;
    const float var_s = (red0[rr] + red0[BM + rr] + red0[2 * BM + rr] + red0[3 * BM + rr]) * invn;
    // rstd = 1/sqrt(var + eps) with var = var_s / cs^2
    rsd[i] = cs[i] / sqrtf(var_s + p.eps * cs[i] * cs[i]);
  }
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int64_t m = m0 + 16 * i + r;
      if (m < p.M) {
        if (p.mean) p.mean[m] = mu[i];
        if (p.rstd) p.rstd[m] = rsd[i];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    if (t < nt) {
      const int n0 = nb + 16 * t + 4 * g;
      float gv[4], bv[4];
      load4_bf16(p.gamma ? p.gamma + n0 : nullptr, 1.0f, gv);
      load4_bf16(p.beta ? p.beta + n0 : nullptr, 0.0f, bv);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int64_t m = m0 + 16 * i + r;
        if (m < p.M) {
          float o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = (acc[t][i][j] - mu[i]) * rsd[i] * gv[j] + bv[j];
          *reinterpret_cast<uint2*>(p.y + m * N + n0) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          if (p.z)
            *reinterpret_cast<float4*>(p.z + m * N + n0) =
                make_float4(acc[t][i][0], acc[t][i][1], acc[t][i][2], acc[t][i][3]);
        }
      }
    }
  }
}

// Tensor mode: every workgroup reduces the X amax partials itself.
template <int FMT>
__device__ __forceinline__ ScalePair reduce_tensor_scale(const float* partials, int np, float* red4) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += 256) m = fmaxf(m, partials[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
  return scales_from_amax<FMT>(m);
}

template <int MODE, int NTMAX, int MT>
__global__ __launch_bounds__(256) void k_fwd(FwdBlock p, const float* partials, int np) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (MODE == 0) {
    __shared__ float red4[4];
    ScalePair sp = reduce_tensor_scale<0>(partials, np, red4);
    p.x_r = sp.r;
    p.x_s = sp.s;
  }
  fwd_block<MODE, NTMAX, MT>(p, (int64_t)blockIdx.x * (16 * MT), smem);
}

// Grouped: tile_start[g] = first workgroup of group g (prefix sums of
// ceil(M_g / BM)), tile_start[num_groups] = grid size.
template <int NTMAX, int MT>
__global__ __launch_bounds__(256) void k_grouped(const GroupDev* groups, const int* tile_start, int num_groups,
                                                 float eps) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  int lo = 0, hi = num_groups - 1;  // last group with tile_start <= b
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
  fwd_block<1, NTMAX, MT>(p, (int64_t)(b - tile_start[lo]) * (16 * MT), smem);
}

constexpr int kMT = 4;  // 64 rows per workgroup

template <int MODE, int NTMAX>
hipError_t launch_fwd_t(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  const unsigned grid = (unsigned)((p.M + 16 * kMT - 1) / (16 * kMT));
  const size_t lds = fwd_lds_bytes(16 * kMT, p.K);
  auto kern = k_fwd<MODE, NTMAX, kMT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, s, p, partials, np);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_fwd_mode(const FwdBlock& p, const float* partials, int np, hipStream_t s) {
  if (p.N <= 256) return launch_fwd_t<MODE, 4>(p, partials, np, s);
  if (p.N <= 512) return launch_fwd_t<MODE, 8>(p, partials, np, s);
  return launch_fwd_t<MODE, 16>(p, partials, np, s);
}

}  // namespace

hipError_t launch_amax_tensor_partials(const void* src, int64_t rows, int64_t cols, int64_t ld, float* partials,
                                       hipStream_t s);

size_t fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int x_mode) {
  (void)N;
  if (x_mode != 0) return 0;
  return (size_t)quant_plan(M, K, 0).np * sizeof(float);
}

hipError_t launch_fwd(const FwdLaunch& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  FwdBlock p;
  p.M = a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.x = static_cast<const uint16_t*>(a.x);
  p.qw = a.qw; p.sw = a.sw;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.gamma = static_cast<const uint16_t*>(a.gamma);
  p.beta = static_cast<const uint16_t*>(a.beta);
  p.y = static_cast<uint16_t*>(a.y);
  p.z = a.z; p.mean = a.mean; p.rstd = a.rstd; p.qx_out = a.qx_out; p.sx_out = a.sx_out;
  p.eps = a.eps; p.x_r = 1.0f; p.x_s = 1.0f;
  if (a.x_mode == 0) {
    float* partials = static_cast<float*>(a.workspace);
    const int np = (int)quant_plan(a.M, a.K, 0).np;
    hipError_t e = launch_amax_tensor_partials(a.x, a.M, a.K, a.K, partials, s);
    if (e != hipSuccess) return e;
    return launch_fwd_mode<0>(p, partials, np, s);
  }
  if (a.x_mode == 1) return launch_fwd_mode<1>(p, nullptr, 0, s);
  return launch_fwd_mode<3>(p, nullptr, 0, s);
}

size_t grouped_workspace_bytes(int num_groups, const GroupDev* groups) {
  (void)groups;
  size_t b = (size_t)num_groups * sizeof(GroupDev);
  b = (b + 255) / 256 * 256;
  b += (size_t)(num_groups + 1) * sizeof(int);
  return b;
}

hipError_t launch_grouped(const GroupedLaunch& a, hipStream_t s) {
  constexpr int BM = 16 * kMT;
  // host-built tile table: prefix sums of ceil(M_g / BM); empty groups get no tiles
  int* starts = new int[a.num_groups + 1];
  int total = 0, kmax = 16, nmax = 64;
  for (int gi = 0; gi < a.num_groups; ++gi) {
    starts[gi] = total;
    total += (int)((a.groups[gi].M + BM - 1) / BM);
    if (a.groups[gi].K > kmax) kmax = (int)a.groups[gi].K;
    if (a.groups[gi].N > nmax) nmax = (int)a.groups[gi].N;
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
  const size_t lds = fwd_lds_bytes(BM, kmax);
  if (nmax <= 512) {
    auto kern = k_grouped<8, kMT>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(256), lds, s, dgroups, dstarts, a.num_groups, a.eps);
  } else {
    auto kern = k_grouped<16, kMT>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(256), lds, s, dgroups, dstarts, a.num_groups, a.eps);
  }
  return hipGetLastError();
}

}  // namespace loka
