// The fused forward block shared by loka_gemm_fp8_ln and the grouped launch.
//
// Source: LoKA section III-B2 (Block-wise Normalization): the normalization
// runs in the GEMM epilogue while the output tile is still on chip, and in
// Case 1 (large batch, small output dimension) a whole output row lives in
// one block, so the result is the standard normalization; section III-B:
// the GEMM output is dequantized and the LayerNorm runs in high precision;
// section III-B1 (No Bias).  GEM "Mixed Ultra-Low-Precision Training":
// activation quantization fused into the neighbouring kernel instead of an
// extra pass over HBM; "Low Precision Flash Attention": MX block scales
// along K.
//
// One workgroup of 8 wavefronts owns BM = 16*MT rows and all N columns.
// The N/16 column tiles are dealt to the wavefronts round-robin (wavefront
// w owns tiles w, w+8, ...; NTW = ceil(N/128) per wavefront, the missing
// ones of a short wavefront computed on a clamped tile and discarded):
//  1. each wavefront requests its first K-chunk of weight fragments, then
//     loads BM/8 rows of X (bf16, 16 B per lane, every load of a batch in
//     flight before the first is used), takes the row (or 32-block) max-abs
//     with DPP reductions and writes the FP8 codes to LDS (rows padded by
//     16 B against bank conflicts);
//  2. each wavefront runs v_mfma_scale_f32_16x16x128_f8f6f4 over K for its
//     tiles and all BM rows: A = W^T rows streamed from L2 (the next chunk
//     in flight while the current one feeds the MFMAs), B = the X codes in
//     LDS.  W is read once per workgroup: the wavefronts own disjoint columns;
//  3. the epilogue keeps the accumulators in registers: dequant + bias, row
//     mean, centred sum of squares (two passes, one LDS exchange each), then
//     gamma/beta, hardware bf16 rounding, and the rows staged in LDS so the
//     global stores are whole, coalesced rows.
// X is read from HBM once and Y written once; nothing else reaches HBM
// unless the optional outputs are requested.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace loka {
namespace fwd {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

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
  int ldy;         // row stride of y and z in elements (0: N); a column slab's is the full width
  // square-block recipe (MODE 4): X arrives quantized, e4m3 codes [M][K]
  // and E8M0 scales [M/32][K/32]
  const uint8_t* xq;
  const uint8_t* xs;
  // optional: Y quantized in 32 x 32 blocks (e4m3 [M][N], E8M0 [M/32][N/32])
  uint8_t* y_codes;
  uint8_t* y_scales;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16_hw(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__host__ __device__ constexpr int lds_stride(int K) { return K + 16; }
__host__ __device__ constexpr int ystage_stride(int N) { return 2 * N + 16; }  // bytes per staged Y row

// LDS: [ X codes (BM x (K+16)) | Y staging (BM x (2N+16)) ] share one region
// (X is dead once the GEMM is done), then row scales, MX scales, reductions.
__host__ __device__ inline size_t fwd_lds_bytes(int BM, int K, int N) {
  size_t xb = (size_t)BM * lds_stride(K);
  size_t yb = (size_t)BM * ystage_stride(N);
  size_t b = (xb > yb ? xb : yb);
  b = (b + 15) / 16 * 16;
  b += (size_t)BM * 4;                          // row scales
  b += ((size_t)BM * (K / 32) + 15) / 16 * 16;  // MX scales
  b += (size_t)2 * kWaves * BM * 4;             // two reduction buffers
  b += 128;                                     // workgroup scalars
  return b;
}

// Power-of-two factor c <= 1 for a row whose magnitudes may reach 2^e or
// more: with e >= 55, N * (z - mean)^2 could overflow fp32 (N <= 1024), so
// the deviations are scaled by c = 2^(40 - e) (exact) before squaring.
// Ordinary rows get c = 1 and exactly the unscaled arithmetic.
__device__ __forceinline__ float row_rescale(float bound) {
  const int e = (int)((__float_as_uint(bound) >> 23) & 0xFF) - 127;  // floor(log2) for normal values
  return e >= 55 ? __uint_as_float((uint32_t)(167 - e) << 23) : 1.0f;
}

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float def, float o[4]) {
  if (p == nullptr) {
    o[0] = o[1] = o[2] = o[3] = def;
    return;
  }
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
}

// ---- 1. quantize this workgroup's rows of X into LDS ------------------------
// Wavefront w quantizes rows [w*RPW, (w+1)*RPW), RPW = BM/8.  All loads of a
// batch of rows are issued before any is used (addresses past M or K are
// clamped to valid ones instead of branched around; those values are never
// stored).  KCH: 512-element chunks per row (K <= 512 * KCH).
template <int MODE, int KCH, int MT>
__device__ __forceinline__ void quantize_rows(const FwdBlock& p, int64_t m0, int wave, int lane, uint8_t* xs,
                                              float* rs, uint8_t* xe8) {
  constexpr int RPW = 16 * MT / kWaves;
  constexpr int RB = (16 / KCH) < RPW ? (16 / KCH) : RPW;  // rows per load batch (<= 16 loads in flight)
  const int K = p.K, ldk = lds_stride(K), kb = K / 32;
#pragma unroll
  for (int b0 = 0; b0 < RPW; b0 += RB) {
    uint4 raw[RB][KCH];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      int64_t m = m0 + wave * RPW + b0 + rr;
      m = m < p.M ? m : p.M - 1;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        int k = c * 512 + lane * 8;
        k = k < K ? k : K - 8;
        raw[rr][c] = *reinterpret_cast<const uint4*>(p.x + m * K + k);
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int lr = wave * RPW + b0 + rr;
      float v[KCH][8];
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const uint32_t w[4] = {raw[rr][c].x, raw[rr][c].y, raw[rr][c].z, raw[rr][c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[c][2 * i] = bf16_lo(w[i]);
          v[c][2 * i + 1] = bf16_hi(w[i]);
        }
      }
      if (MODE == 3) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          float a = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[c][i]));
          a = quad_max(a);  // a 32-element block is held by 4 consecutive lanes
          const int e8 = e8m0_from_amax<0>(a);
          const float mu = e8m0_inv_multiplier(e8);
          const int k = c * 512 + lane * 8;
          if (k < K) {
            if ((lane & 3) == 0) xe8[lr * kb + k / 32] = (uint8_t)e8;
            const uint32_t lo = cvt4<0>(v[c][0] * mu, v[c][1] * mu, v[c][2] * mu, v[c][3] * mu);
            const uint32_t hi = cvt4<0>(v[c][4] * mu, v[c][5] * mu, v[c][6] * mu, v[c][7] * mu);
            *reinterpret_cast<uint2*>(xs + lr * ldk + k) = make_uint2(lo, hi);
          }
        }
      } else {
        float r;
        if (MODE == 1) {
          float a = 0.0f;
#pragma unroll
          for (int c = 0; c < KCH; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[c][i]));
          a = wave_max_dpp(a);
          const ScalePair sp = scales_from_amax<0>(a);
          if (lane == 0) rs[lr] = sp.s;
          r = sp.r;
        } else {
          r = p.x_r;
        }
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const int k = c * 512 + lane * 8;
          if (k < K) {
            const uint32_t lo = cvt4<0>(v[c][0] * r, v[c][1] * r, v[c][2] * r, v[c][3] * r);
            const uint32_t hi = cvt4<0>(v[c][4] * r, v[c][5] * r, v[c][6] * r, v[c][7] * r);
            *reinterpret_cast<uint2*>(xs + lr * ldk + k) = make_uint2(lo, hi);
          }
        }
      }
    }
  }
}

// Full-chunk fragment load (the chunk lies inside K).
__device__ __forceinline__ v8i load_frag_full(const uint8_t* p, int g, int kc) {
  const uint4 a = *reinterpret_cast<const uint4*>(p + kc + 16 * g);
  const uint4 b = *reinterpret_cast<const uint4*>(p + kc + 64 + 16 * g);
  v8i f;
  f[0] = (int)a.x; f[1] = (int)a.y; f[2] = (int)a.z; f[3] = (int)a.w;
  f[4] = (int)b.x; f[5] = (int)b.y; f[6] = (int)b.z; f[7] = (int)b.w;
  return f;
}

template <int MODE, int NT, bool FULL>
__device__ __forceinline__ void load_w(v8i (&wf)[NT], int (&wsc)[NT], const uint8_t* const (&wrow)[NT],
                                       const uint8_t* const (&srow)[NT], int g, int kc, int K, int kb) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wf[t] = FULL ? load_frag_full(wrow[t], g, kc) : load_frag(wrow[t], g, kc, K);
    if (MODE == 3) {
      const int blk = kc / 32 + g;
      wsc[t] = (FULL || blk < kb) ? (int)srow[t][blk] : 127;
    }
  }
}

// One 128-deep step of the GEMM for all NT x MT tiles of this wavefront.
template <int MODE, int NT, int MT>
__device__ __forceinline__ void mma_step(v4f (&acc)[NT][MT], const v8i (&wf)[NT], const int (&wsc)[NT],
                                         const uint8_t* xs, const uint8_t* xe8, int ldk, int kb, int r, int g,
                                         int kc, int limit) {
  v8i xf[MT];
  int xsc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    xf[i] = load_frag(xs + (16 * i + r) * ldk, g, kc, limit);
    if (MODE == 3) {
      const int blk = kc / 32 + g;
      xsc[i] = blk < kb ? (int)xe8[(16 * i + r) * kb + blk] : 127;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < MT; ++i)
      acc[t][i] = MODE == 3 ? mfma_mx_e4m3(wf[t], xf[i], acc[t][i], wsc[t], xsc[i])
                            : mfma_fp8<0, 0>(wf[t], xf[i], acc[t][i]);
}

// Per-column vectors of one 16-column tile for this lane's 4 columns,
// requested at kernel start: dequantization scales, bias, gamma, beta.
struct ColVec {
  float4 sw;
  uint2 b, ga, be;
};

__device__ __forceinline__ void unpack4(uint2 u, float o[4]) {
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
}

// One workgroup (8 wavefronts): BM = 16*MT rows, all N columns (N <= 128*NTW).
// MODE: 0 tensor, 1 row, 3 mx32.  ALLV: N is a multiple of 128, so every
// wavefront's NTW tiles are real (no clamped duplicates to mask out).
template <int MODE, int NTW, int MT, bool ALLV>
__device__ __forceinline__ void fwd_block(const FwdBlock& p, int64_t m0, uint8_t* smem) {
  constexpr int BM = 16 * MT;
  const int K = p.K, N = p.N;
  const int T = N >> 4;  // 16-column tiles
  const int ldk = lds_stride(K), ldy = ystage_stride(N);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kb = K / 32;  // MX blocks per row

  size_t xb = (size_t)BM * ldk, yb = (size_t)BM * ldy;
  uint8_t* xs = smem;  // X codes, later the staged Y rows
  float* rs = reinterpret_cast<float*>(smem + ((xb > yb ? xb : yb) + 15) / 16 * 16);
  uint8_t* xe8 = reinterpret_cast<uint8_t*>(rs + BM);
  float* red0 = reinterpret_cast<float*>(xe8 + ((size_t)BM * kb + 15) / 16 * 16);
  float* red1 = red0 + kWaves * BM;
  float* wgs = red1 + kWaves * BM;  // workgroup scalars: [8+w], [16+w] per-wavefront column maxima

  // this wavefront's column tiles: w, w+8, ... (clamped beyond T, discarded)
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* wrow[NTW];
  const uint8_t* srow[NTW];
  int tile[NTW];
  bool tvalid[NTW];
  const uint8_t* sw8 = static_cast<const uint8_t*>(p.sw);
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int t = wave + kWaves * j;
    tvalid[j] = ALLV || t < T;
    tile[j] = (ALLV || t < T) ? t : T - 1;
    wrow[j] = p.qw + (int64_t)(16 * tile[j] + r) * K;
    srow[j] = MODE == 3 ? sw8 + (int64_t)(16 * tile[j] + r) * kb : nullptr;
  }
  // the first two weight chunks and every per-column vector are requested
  // before the activations are touched
  const int nfull = K >> 7;
  v8i wa[NTW], wb[NTW];
  int sa[NTW], sb[NTW];
  if (nfull > 0) load_w<MODE, NTW, true>(wa, sa, wrow, srow, g, 0, K, kb);
  if (nfull > 1) load_w<MODE, NTW, true>(wb, sb, wrow, srow, g, 128, K, kb);
  ColVec cv[NTW];
  const uint2 ones = make_uint2(0x3F803F80u, 0x3F803F80u), zeros = make_uint2(0u, 0u);
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n0 = 16 * tile[j] + 4 * g;
    if (MODE == 1) cv[j].sw = *reinterpret_cast<const float4*>(static_cast<const float*>(p.sw) + n0);
    cv[j].b = p.bias ? *reinterpret_cast<const uint2*>(p.bias + n0) : zeros;
    cv[j].ga = p.gamma ? *reinterpret_cast<const uint2*>(p.gamma + n0) : ones;
    cv[j].be = p.beta ? *reinterpret_cast<const uint2*>(p.beta + n0) : zeros;
  }

  // ---- 1. quantize ----------------------------------------------------------
  if (K <= 512) quantize_rows<MODE, 1, MT>(p, m0, wave, lane, xs, rs, xe8);
  else if (K <= 1024) quantize_rows<MODE, 2, MT>(p, m0, wave, lane, xs, rs, xe8);
  else quantize_rows<MODE, 4, MT>(p, m0, wave, lane, xs, rs, xe8);
  __syncthreads();

  // optional: the quantized X (bit-identical to loka_quant_fp8) for the backward
  if (p.qx_out != nullptr) {
    const int k16 = K / 16;
    for (int u = tid; u < BM * k16; u += kThreads) {
      const int lr = u / k16, c = (u - lr * k16) * 16;
      if (m0 + lr < p.M)
        *reinterpret_cast<uint4*>(p.qx_out + (m0 + lr) * K + c) = *reinterpret_cast<const uint4*>(xs + lr * ldk + c);
    }
  }
  if (p.sx_out != nullptr) {
    if (MODE == 1) {
      if (tid < BM && m0 + tid < p.M) static_cast<float*>(p.sx_out)[m0 + tid] = rs[tid];
    } else if (MODE == 3) {
      for (int u = tid; u < BM * kb; u += kThreads) {
        const int lr = u / kb;
        if (m0 + lr < p.M) static_cast<uint8_t*>(p.sx_out)[(m0 + lr) * kb + (u - lr * kb)] = xe8[u];
      }
    } else if (m0 == 0 && tid == 0) {
      static_cast<float*>(p.sx_out)[0] = p.x_s;
    }
  }

  // ---- 2. GEMM: D[n][m] = sum_k W^T[n][k] X[m][k] ---------------------------
  v4f acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // full 128-deep chunks from two alternating register sets; a set is
  // refilled with the chunk after next as soon as its MFMAs are issued
  for (int c = 0; c < nfull; c += 2) {
    mma_step<MODE, NTW, MT>(acc, wa, sa, xs, xe8, ldk, kb, r, g, c << 7, K);
    if (c + 2 < nfull) load_w<MODE, NTW, true>(wa, sa, wrow, srow, g, (c + 2) << 7, K, kb);
    if (c + 1 >= nfull) break;
    mma_step<MODE, NTW, MT>(acc, wb, sb, xs, xe8, ldk, kb, r, g, (c + 1) << 7, K);
    if (c + 3 < nfull) load_w<MODE, NTW, true>(wb, sb, wrow, srow, g, (c + 3) << 7, K, kb);
  }
  if (K & 127) {  // tail chunk: fragments past K read as zero
    const int kc = nfull << 7;
    load_w<MODE, NTW, false>(wa, sa, wrow, srow, g, kc, K, kb);
    mma_step<MODE, NTW, MT>(acc, wa, sa, xs, xe8, ldk, kb, r, g, kc, K);
  }

  // ---- 3. epilogue: dequant + bias, LayerNorm, bf16 --------------------------
  // lane (r, g) holds, for tile j and row tile i: n = 16 tile[j] + 4g + q, m = 16i + r
  float sxv[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) sxv[i] = MODE == 1 ? rs[16 * i + r] : (MODE == 0 ? p.x_s : 1.0f);
  float psum[MT], pmax[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) psum[i] = pmax[i] = 0.0f;
  float swm = 0.0f, bm = 0.0f;  // this lane's column maxima of s_w and |b| (variance-rescale bound)
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    float swv[4], bv[4];
    if (MODE == 1) {
      swv[0] = cv[j].sw.x; swv[1] = cv[j].sw.y; swv[2] = cv[j].sw.z; swv[3] = cv[j].sw.w;
    } else {
      const float s0 = MODE == 0 ? static_cast<const float*>(p.sw)[0] : 1.0f;
      swv[0] = swv[1] = swv[2] = swv[3] = s0;
    }
    unpack4(cv[j].b, bv);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      swm = fmaxf(swm, swv[q]);
      bm = fmaxf(bm, fabsf(bv[q]));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float zz = MODE == 3 ? acc[j][i][q] + bv[q] : fmaf(acc[j][i][q], sxv[i] * swv[q], bv[q]);
        acc[j][i][q] = zz;
        if (ALLV) {
          psum[i] += zz;
          if (MODE == 3) pmax[i] = fmaxf(pmax[i], fabsf(zz));
        } else {
          const float vm = tvalid[j] ? 1.0f : 0.0f;
          psum[i] = fmaf(zz, vm, psum[i]);
          if (MODE == 3) pmax[i] = fmaxf(pmax[i], fabsf(zz) * vm);
        }
      }
    }
  }
  if (MODE != 3) {
    swm = wave_max_dpp(swm);
    bm = wave_max_dpp(bm);
    if (lane == 0) {
      wgs[8 + wave] = swm;
      wgs[16 + wave] = bm;
    }
  }
  const float invn = 1.0f / (float)N;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    psum[i] = group4_sum(psum[i]);
    if (MODE == 3) {
      pmax[i] = fmaxf(pmax[i], __shfl_xor(pmax[i], 16, 64));
      pmax[i] = fmaxf(pmax[i], __shfl_xor(pmax[i], 32, 64));
    }
    if (g == 0) {
      red0[wave * BM + 16 * i + r] = psum[i];
      if (MODE == 3) red1[wave * BM + 16 * i + r] = pmax[i];
    }
  }
  __syncthreads();
  // |z| <= s_x * 448^2 K max_n s_w + max_n |b| bounds a row's values (tensor/row
  // recipes); MX rows use their actual maximum
  float bound_w = 0.0f, bound_b = 0.0f;
  if (MODE != 3) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      bound_w = fmaxf(bound_w, wgs[8 + w]);
      bound_b = fmaxf(bound_b, wgs[16 + w]);
    }
    bound_w *= (448.0f * 448.0f) * (float)K;
  }
  float mu[MT], cs[MT];
  bool scaled = false;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int rr = 16 * i + r;
    float s = 0.0f, mx = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s += red0[w * BM + rr];
      if (MODE == 3) mx = fmaxf(mx, red1[w * BM + rr]);
    }
    mu[i] = s * invn;
    cs[i] = row_rescale(MODE == 3 ? mx : sxv[i] * bound_w + bound_b);
    scaled |= cs[i] != 1.0f;
  }
  __syncthreads();  // red0/red1 are reused below
  float psq[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) psq[i] = 0.0f;
  if (__any(scaled)) {  // rows too large to square in fp32 (rare)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const float vm = (ALLV || tvalid[j]) ? 1.0f : 0.0f;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float d = (acc[j][i][q] - mu[i]) * cs[i] * vm;
          psq[i] = fmaf(d, d, psq[i]);
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float d = acc[j][i][q] - mu[i];
          if (!ALLV) d *= tvalid[j] ? 1.0f : 0.0f;
          psq[i] = fmaf(d, d, psq[i]);
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
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red0[w * BM + rr];
    // rstd = 1/sqrt(var + eps) with var = (s/N) / cs^2
    rsd[i] = cs[i] / sqrtf(s * invn + p.eps * cs[i] * cs[i]);
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
  // y = (z - mean) * rstd * gamma + beta -> bf16 -> staged rows in LDS
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n0 = 16 * tile[j] + 4 * g;
    float gv[4], bv[4];
    unpack4(cv[j].ga, gv);
    unpack4(cv[j].be, bv);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = fmaf((acc[j][i][q] - mu[i]) * rsd[i], gv[q], bv[q]);
      if (ALLV || tvalid[j])
        *reinterpret_cast<uint2*>(xs + (16 * i + r) * ldy + 2 * n0) = make_uint2(pack_bf16_hw(o[0], o[1]),
                                                                              pack_bf16_hw(o[2], o[3]));
    }
  }
  if (p.z != nullptr) {  // optional fp32 pre-norm output
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n0 = 16 * tile[j] + 4 * g;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int64_t m = m0 + 16 * i + r;
        if ((ALLV || tvalid[j]) && m < p.M)
          *reinterpret_cast<float4*>(p.z + m * N + n0) =
              make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
      }
    }
  }
  __syncthreads();
  // whole rows out: 16 B per thread, consecutive threads along a row
  const int n8 = N >> 3;
  for (int u = tid; u < BM * n8; u += kThreads) {
    const int lr = u / n8, c = u - lr * n8;
    if (m0 + lr < p.M)
      *reinterpret_cast<uint4*>(p.y + (m0 + lr) * N + 8 * c) = *reinterpret_cast<const uint4*>(xs + lr * ldy + 16 * c);
  }
}

// Tensor mode: every workgroup reduces the X amax partials itself.
template <int FMT>
__device__ __forceinline__ ScalePair reduce_tensor_scale(const float* partials, int np, float* red8) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += kThreads) m = fmaxf(m, partials[i]);
  m = wave_max_dpp(m);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red8[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red8[w]);
  return scales_from_amax<FMT>(m);
}

// The tensor scale straight from a small X (bf16 [M][K] contiguous, 16-byte
// aligned, M K a multiple of 8): each thread's max-abs over 16-byte pieces,
// then the workgroup's.  The max of exact values does not depend on the
// order, so the scale equals the one from the partials pass bit for bit.
// X is read through a bounds-checked buffer, so pieces past its end read as
// zeros (which never raise a max) and a round's 16 loads per thread go out
// with no branch before its first wait: two round trips for 512 x 256 where
// four loads in flight took eight.  The caller keeps M K 2 below 2^31 bytes.
__device__ __forceinline__ ScalePair tensor_scale_self(const FwdBlock& p, float* red8) {
  const int64_t n8 = p.M * (int64_t)p.K / 8;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x), (short)0,
                                                                        (int)(n8 * 16), kBufferWord3);
  constexpr int R = 16;
  float m = 0.0f;
  for (int64_t base = threadIdx.x; base < n8; base += (int64_t)R * kThreads) {
    uint4 v[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
      v[q] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)((base + q * kThreads) * 16), 0, 0));
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
      }
    }
  }
  m = wave_max_dpp(m);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red8[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red8[w]);
  return scales_from_amax<0>(m);
}

// Workgroup shape per column count: 64-row tiles up to N = 512 (4 column
// tiles per wavefront), 32-row tiles above (up to 8 per wavefront).
template <int NTW>
struct Shape {
  static constexpr int MT = NTW <= 4 ? 4 : 2;
};

}  // namespace fwd
}  // namespace loka
