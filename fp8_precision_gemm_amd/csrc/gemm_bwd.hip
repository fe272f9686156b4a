// Backward of the fused FP8 GEMM + LayerNorm (loka_gemm_fp8_bwd) on gfx950.
//
// Source: LoKA section III-C (Trainer Integration): the FP8 linear is a
// drop-in for a standard Linear whose own autograd function routes the
// backward separately, so this is the exact gradient of the forward's
// definition with rowwise recipes (Table VI's RW recipe); GEM "Mixed
// Ultra-Low-Precision Training": gradients in the e5m2 range, scale factors
// along each GEMM's own contraction dimension.
//
// Launches (all on the caller's stream):
//  1. k_bwd_main, one workgroup per 64 rows:
//       recompute Z = dequant(qX . qW) + b from the forward's codes (MFMA),
//       LayerNorm backward in fp32 registers (two row reductions),
//       dZ -> e5m2 row codes in LDS (+ optional dz / codes / scales out),
//       dgrad MFMA  dX = q(dZ) . q_row(W)^T  -> bf16,
//       per-workgroup column partials of dgamma, dbeta, dbias and max|dZ|.
//  2. column amax + cast of X (e4m3, transposed to [K, M]);
//     cast of dZ (e5m2, transposed to [N, M]) with the maxima from step 1.
//  3. k_wgrad: split-M FP8 MFMA, fp32 partials per M slice.
//  4. k_finalize: fixed-order sums of the partials (deterministic), scales;
//     k_col_vectors: dgamma, dbeta, dbias from the column partials.
// Every FP8 operand the kernels read as MFMA fragments straight from memory
// (both weights, the transposed X and dZ codes) is first laid out in the
// fragment-interleaved order of ilv_offset(), so each 16-lane fragment load
// reads 256 contiguous bytes (launch_relayout does it for the weights; the
// transposing casts write it directly).
#include "common.hpp"
#include "launch.hpp"

namespace loka {


namespace {

constexpr int kMT = 4;           // 64 rows per workgroup
constexpr int kBM = 16 * kMT;
constexpr int kWgSplitRows = 1024;  // M rows per wgrad slice

struct BwdBlock {
  int64_t M;
  int N, K;
  const uint16_t* dy;
  const uint8_t* qx;
  const float* sx;
  const float* mean;
  const float* rstd;
  const uint8_t* qw;
  const float* sw;
  const uint16_t* bias;
  const uint16_t* gamma;
  const uint8_t* qw_row;
  const float* sw_row;
  const uint8_t* qwi;     // qw [N][K] interleaved (K padded to 128)
  const uint8_t* qwri;    // qw_row [K][N] interleaved (N padded to 128)
  uint16_t* dx;
  float* dz;  // fp32 [M, N] (user buffer or workspace): always written
  uint8_t* dz_codes;
  float* dz_scales;
  float* part;  // [4][nblocks][N]: dgamma, dbeta, dbias, max|dZ|
  int nblocks;
  // square-block recipe: X's and W's E8M0 scales ([M/32][K/32], [K/32][N/32]),
  // dZ's scales out ([M/32][N/32]) and its codes out transposed for the wgrad
  // (fragment-interleaved [N][M padded to 128], nchm 128-row chunks)
  const uint8_t* sx8;
  const uint8_t* sw8;
  uint8_t* sdz;
  uint8_t* dzt;
  int64_t nchm;
  // square-block recipe with the LayerNorm (X's codes staged for Z): X's
  // codes out transposed too, in the same layout as dzt ([K][M padded])
  uint8_t* xt;
  // optional, eight-wavefront kernel only: bf16 X [M][K] and the per-block
  // column maxima of |X| out ([nblocks][K]), the first pass of the wgrad
  // operand's column scales
  const uint16_t* xb;
  float* xpart;
};

// MFMA with both operands' E8M0 scale bytes (the bytes this lane supplies)
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_fp8_scaled(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

__device__ __forceinline__ void ld4_bf16(const uint16_t* p, float def, float o[4]) {
  if (p == nullptr) {
    o[0] = o[1] = o[2] = o[3] = def;
    return;
  }
  uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
}

// Sum / max over the 16 lanes sharing l / 16 (lanes with the same 4
// columns): one DPP row.
__device__ __forceinline__ float col16_sum(float v) { return row16_sum(v); }
__device__ __forceinline__ float col16_max(float v) { return row16_max(v); }

// dY rows staged in LDS for N <= 512 and K <= 512 (the staging area and the
// X and dZ code rows then fit the LDS together)
__host__ __device__ constexpr bool bwd_stage_dy(int ntmax, int ktmax, int waves) {
  return ntmax * waves <= 32 && ktmax * waves <= 32;
}

// The 16-column tiles [t0, t0 + n) of T that wavefront w of WAVES owns (T
// split as evenly as the wavefronts allow)
template <int WAVES>
__device__ __forceinline__ void wave_tiles(int T, int w, int& t0, int& n) {
  t0 = (w * T) / WAVES;
  n = ((w + 1) * T) / WAVES - t0;
}

// FULLM: M is a multiple of the 64-row block, so every row exists (no row
// guards).  WAVES wavefronts split the columns: eight (two per SIMD) where a
// wavefront's accumulators and weight fragments fit half the register file
// (N, K <= 512), else four.
// SQ: the square-block recipe (X, W and dZ with one E8M0 scale per 32 x 32
// block; the MFMAs apply the scales, dZ is quantized by blocks and its codes
// also leave transposed for the wgrad, as do X's staged codes).
template <int NTMAX, int KTMAX, int NO_LN, bool FULLM, int WAVES, bool SQ = false>
__global__ __launch_bounds__(64 * WAVES) void k_bwd_main(BwdBlock p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = p.K, N = p.N;
  const int ldk = K + 16, ldn = N + 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;

  uint8_t* xs = smem;                                  // qX rows [BM][K+16]
  uint8_t* ds = xs + (size_t)kBM * ldk;                // dZ codes [BM][N+16]
  float* red0 = reinterpret_cast<float*>(ds + (size_t)kBM * ldn);
  float* red1 = red0 + WAVES * kBM;
  float* rsc = red1 + WAVES * kBM;                 // dZ row scales [BM]
  // SDY: the block's dY rows staged in LDS [BM][2N+16] (when the LDS has room)
  constexpr bool SDY = bwd_stage_dy(NTMAX, KTMAX, WAVES);
  const int ldy = 2 * N + 16;
  uint8_t* dys = reinterpret_cast<uint8_t*>(rsc + kBM);

  int nt, nb;
  wave_tiles<WAVES>(N / 16, wave, nb, nt);
  nb *= 16;
  int kt, kb0;
  wave_tiles<WAVES>(K / 16, wave, kb0, kt);
  kb0 *= 16;
  v4f acc[NTMAX][kMT];  // holds Z, then dZ

  // Weight fragments of both GEMMs stream from L2 through three rotating
  // buffers, two 128-deep chunks ahead of the MFMAs: the Z recompute's first
  // two chunks are requested before the staging below, the dgrad's right
  // after the Z recompute, so each arrives during the phase before its GEMM.
  const int nchk = (K + 127) >> 7, nchn = (N + 127) >> 7;
  constexpr int WB = NTMAX > KTMAX ? NTMAX : KTMAX;
  v8i w0[WB], w1[WB], w2[WB];
  auto wload = [&](int c, v8i (&w)[WB]) {
#pragma unroll
    for (int t = 0; t < NTMAX; ++t)
      if (t < nt) w[t] = load_frag_ilv(p.qwi, nb / 16 + t, c, nchk, r, g);
  };
  auto rload = [&](int c, v8i (&w)[WB]) {
#pragma unroll
    for (int t = 0; t < KTMAX; ++t)
      if (t < kt) w[t] = load_frag_ilv(p.qwri, kb0 / 16 + t, c, nchn, r, g);
  };
  if (!NO_LN) {
    wload(0, w0);
    if (nchk > 1) wload(1, w1);
  }

  // per-row constants of this lane's rows m = m0 + 16 i + r, requested first
  bool rowok[kMT];
  float mu[kMT], rs[kMT], sxv[kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    const int64_t m = m0 + 16 * i + r;
    rowok[i] = FULLM || m < p.M;
    mu[i] = (!NO_LN && rowok[i]) ? p.mean[m] : 0.0f;
    rs[i] = (!NO_LN && rowok[i]) ? p.rstd[m] : 0.0f;
    sxv[i] = (!NO_LN && !SQ && rowok[i]) ? p.sx[m] : 0.0f;
  }

  if (!NO_LN) {
    // stage the forward's X codes in LDS, and with SDY the block's dY rows
    // too: all requests go out before the first wait, so one HBM latency
    // covers both, and the two LayerNorm passes read dY from LDS
    const int k16 = K / 16, n8 = SDY ? N / 8 : 0, n8d = SDY ? n8 : 1;
    if constexpr (SDY) {
      // N, K <= 512: at most 32 / WAVES pieces of X codes and 64 / WAVES of
      // dY per thread; every load is issued before the first wait, so the
      // staging costs one memory round trip instead of one per piece
      constexpr int XP = 32 / WAVES, YP = 64 / WAVES;
      uint4 xv[XP], yv[YP];
#pragma unroll
      for (int q = 0; q < XP; ++q) {
        const int u = tid + q * 64 * WAVES, lr = u / k16, c = (u - lr * k16) * 16;
        xv[q] = make_uint4(0, 0, 0, 0);
        if (u < kBM * k16 && (FULLM || m0 + lr < p.M)) xv[q] = *reinterpret_cast<const uint4*>(p.qx + (m0 + lr) * K + c);
      }
#pragma unroll
      for (int q = 0; q < YP; ++q) {
        const int u = tid + q * 64 * WAVES, lr = u / n8d, c = (u - lr * n8d) * 8;
        yv[q] = make_uint4(0, 0, 0, 0);
        if (u < kBM * n8 && (FULLM || m0 + lr < p.M)) yv[q] = *reinterpret_cast<const uint4*>(p.dy + (m0 + lr) * N + c);
      }
#pragma unroll
      for (int q = 0; q < XP; ++q) {
        const int u = tid + q * 64 * WAVES, lr = u / k16, c = (u - lr * k16) * 16;
        if (u < kBM * k16) *reinterpret_cast<uint4*>(xs + lr * ldk + c) = xv[q];
      }
#pragma unroll
      for (int q = 0; q < YP; ++q) {
        const int u = tid + q * 64 * WAVES, lr = u / n8d, c = (u - lr * n8d) * 8;
        if (u < kBM * n8) *reinterpret_cast<uint4*>(dys + lr * ldy + 2 * c) = yv[q];
      }
    } else {
      for (int u = tid; u < kBM * (k16 + n8); u += 64 * WAVES) {
        if (u < kBM * k16) {
          const int lr = u / k16, c = (u - lr * k16) * 16;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (FULLM || m0 + lr < p.M) v = *reinterpret_cast<const uint4*>(p.qx + (m0 + lr) * K + c);
          *reinterpret_cast<uint4*>(xs + lr * ldk + c) = v;
        } else {
          const int v8 = u - kBM * k16, lr = v8 / n8d, c = (v8 - lr * n8d) * 8;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (FULLM || m0 + lr < p.M) v = *reinterpret_cast<const uint4*>(p.dy + (m0 + lr) * N + c);
          *reinterpret_cast<uint4*>(dys + lr * ldy + 2 * c) = v;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTMAX; ++t)
#pragma unroll
      for (int i = 0; i < kMT; ++i) acc[t][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // one 128-deep chunk: request chunk c + 2 into the free buffer, then the
    // MFMAs of chunk c
    auto zstep = [&](int c, const v8i (&wc)[WB], v8i (&wn)[WB]) {
      if (c + 2 < nchk) wload(c + 2, wn);
      v8i xf[kMT];
#pragma unroll
      for (int i = 0; i < kMT; ++i) xf[i] = load_frag(xs + (16 * i + r) * ldk, g, 128 * c, K);
      if constexpr (SQ) {
        // lane group g supplies the scales of K block 4c + g (clamped past K,
        // where the codes are zero): W's for its column, X's for its row
        const int kbk = min(4 * c + g, (K >> 5) - 1);
        int sa[NTMAX], sb[kMT];
#pragma unroll
        for (int t = 0; t < NTMAX; ++t) sa[t] = t < nt ? p.sw8[kbk * (N >> 5) + ((nb + 16 * t + r) >> 5)] : 127;
#pragma unroll
        for (int i = 0; i < kMT; ++i) sb[i] = p.sx8[(min(m0 + 16 * i + r, p.M - 1) >> 5) * (K >> 5) + kbk];
#pragma unroll
        for (int t = 0; t < NTMAX; ++t)
          if (t < nt)
#pragma unroll
            for (int i = 0; i < kMT; ++i) acc[t][i] = mfma_fp8_scaled<0, 0>(wc[t], xf[i], acc[t][i], sa[t], sb[i]);
      } else {
#pragma unroll
        for (int t = 0; t < NTMAX; ++t)
          if (t < nt)
#pragma unroll
            for (int i = 0; i < kMT; ++i) acc[t][i] = mfma_fp8<0, 0>(wc[t], xf[i], acc[t][i]);
      }
    };
    for (int c = 0; c < nchk; c += 3) {
      zstep(c, w0, w2);
      if (c + 1 < nchk) zstep(c + 1, w1, w0);
      if (c + 2 < nchk) zstep(c + 2, w2, w1);
    }
  }
  // the dgrad's first weight chunk, into a buffer the Z recompute no longer
  // reads (the second follows once the LayerNorm backward is done)
  rload(0, w0);

  // g = dY * gamma, yhat; row sums of g and g * yhat.  acc <- yhat, dyg[] <- g
  // (the dY values are re-read below; they stay in L1/L2)
  float s1[kMT], s2[kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i) s1[i] = s2[i] = 0.0f;
  float colg[NTMAX][4], colb[NTMAX][4];  // dgamma, dbeta partials (over this lane's rows)
#pragma unroll
  for (int t = 0; t < NTMAX; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) colg[t][j] = colb[t][j] = 0.0f;

#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    if (t < nt) {
      const int n0 = nb + 16 * t + 4 * g;
      float swv[4] = {1.0f, 1.0f, 1.0f, 1.0f}, bv[4], gm[4];
      if (!NO_LN) {
        if (!SQ) {
          float4 s4 = *reinterpret_cast<const float4*>(p.sw + n0);
          swv[0] = s4.x; swv[1] = s4.y; swv[2] = s4.z; swv[3] = s4.w;
        }
        ld4_bf16(p.bias ? p.bias + n0 : nullptr, 0.0f, bv);
        ld4_bf16(p.gamma ? p.gamma + n0 : nullptr, 1.0f, gm);
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        const int64_t m = m0 + 16 * i + r;
        float dyv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (SDY && !NO_LN) ld4_bf16(reinterpret_cast<const uint16_t*>(dys + (16 * i + r) * ldy) + n0, 0.0f, dyv);
        else if (rowok[i]) ld4_bf16(p.dy + m * N + n0, 0.0f, dyv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (NO_LN) {
            acc[t][i][j] = dyv[j];  // dZ = dY
          } else {
            const float z = SQ ? acc[t][i][j] + bv[j] : acc[t][i][j] * sxv[i] * swv[j] + bv[j];
            const float yh = (z - mu[i]) * rs[i];
            const float gg = dyv[j] * gm[j];
            acc[t][i][j] = yh;
            s1[i] += gg;
            s2[i] += gg * yh;
            colg[t][j] += dyv[j] * yh;
            colb[t][j] += dyv[j];
          }
        }
      }
    }
  }

  if (!NO_LN) {
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      s1[i] = rows4_sum(s1[i]);
      s2[i] = rows4_sum(s2[i]);
      if (g == 0) {
        red0[wave * kBM + 16 * i + r] = s1[i];
        red1[wave * kBM + 16 * i + r] = s2[i];
      }
    }
    __syncthreads();
    const float invn = 1.0f / (float)N;
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const int rr = 16 * i + r;
      float a = 0.0f, b = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        a += red0[w * kBM + rr];
        b += red1[w * kBM + rr];
      }
      s1[i] = a * invn;  // mean g
      s2[i] = b * invn;  // mean g*yhat
    }
    // dZ = rstd * (g - mean g - yhat * mean(g yhat))
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
      if (t < nt) {
        const int n0 = nb + 16 * t + 4 * g;
        float gm[4];
        ld4_bf16(p.gamma ? p.gamma + n0 : nullptr, 1.0f, gm);
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
          const int64_t m = m0 + 16 * i + r;
          float dyv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (SDY) ld4_bf16(reinterpret_cast<const uint16_t*>(dys + (16 * i + r) * ldy) + n0, 0.0f, dyv);
          else if (rowok[i]) ld4_bf16(p.dy + m * N + n0, 0.0f, dyv);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gg = dyv[j] * gm[j];
            acc[t][i][j] = rowok[i] ? rs[i] * (gg - s1[i] - acc[t][i][j] * s2[i]) : 0.0f;
          }
        }
      }
    }
  }

  // row amax of dZ -> e5m2 scales; column partials; dZ out; codes -> LDS
  float am[kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i) am[i] = 0.0f;
#pragma unroll
  for (int t = 0; t < NTMAX; ++t)
    if (t < nt)
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) am[i] = fmaxf(am[i], fabsf(acc[t][i][j]));
  float rq[kMT];
  float mq[NTMAX][2];  // SQ: multiplier of the 32 x 32 block of tile t, row band i / 2
  int* be8 = reinterpret_cast<int*>(rsc);  // SQ: the block's E8M0 codes [2][N/32]
  if constexpr (SQ) {
    // 32 x 32 block maxima of |dZ|: per 16 x 16 tile a DPP max over its rows
    // and a permlane max over its column groups, two tiles per 32-row band;
    // the bands' tile maxima go through LDS, since a block may straddle two
    // wavefronts' column runs
    const int T16 = N >> 4;
    float tm[NTMAX][2];
#pragma unroll
    for (int t = 0; t < NTMAX; ++t)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(acc[t][2 * rb][j]), fabsf(acc[t][2 * rb + 1][j])));
        tm[t][rb] = rows4_max(row16_max(a));
      }
    __syncthreads();  // red0/red1 reads above are complete before reuse
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < NTMAX; ++t)
        if (t < nt) {
          red0[(nb >> 4) + t] = tm[t][0];
          red0[T16 + (nb >> 4) + t] = tm[t][1];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTMAX; ++t)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        mq[t][rb] = 1.0f;
        if (t < nt) {
          const int ct = (nb >> 4) + t, cb = ct >> 1;
          const float a = fmaxf(red0[rb * T16 + 2 * cb], red0[rb * T16 + 2 * cb + 1]);
          const int e8 = e8m0_from_amax<1>(a);
          mq[t][rb] = e8m0_inv_multiplier(e8);
          // one writer per block: lane 0 of the wavefront owning its even tile
          if (lane == 0 && (ct & 1) == 0) {
            be8[rb * (N >> 5) + cb] = e8;
            const int64_t gb = (m0 >> 5) + rb;
            if (gb * 32 < p.M) p.sdz[gb * (N >> 5) + cb] = (uint8_t)e8;
          }
        }
      }
  } else {
    __syncthreads();  // red0/red1 reads above are complete before reuse
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      am[i] = rows4_max(am[i]);
      if (g == 0) red0[wave * kBM + 16 * i + r] = am[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const int rr = 16 * i + r;
      float a = red0[rr];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) a = fmaxf(a, red0[w * kBM + rr]);
      ScalePair sp = scales_from_amax<1>(a);
      rq[i] = sp.r;
      if (wave == 0 && g == 0) {
        rsc[rr] = sp.s;
        if (p.dz_scales && rowok[i]) p.dz_scales[m0 + rr] = sp.s;
      }
    }
  }

  if (nchn > 1) rload(1, w1);
  const int nblk = blockIdx.x;
  // dZ (fp32) of the block's 64 rows through one buffer resource: 32-bit
  // offsets instead of a 64-bit address per store
  const __amdgpu_buffer_rsrc_t dzr = __builtin_amdgcn_make_buffer_rsrc(
      p.dz + m0 * N, (short)0, (int)((FULLM ? (int64_t)kBM : min((int64_t)kBM, p.M - m0)) * N * 4), kBufferWord3);
#pragma unroll
  for (int t = 0; t < NTMAX; ++t) {
    if (t < nt) {
      const int n0 = nb + 16 * t + 4 * g;
      float cdb[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cmx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        const int lr = 16 * i + r;
        const int64_t m = m0 + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cdb[j] += acc[t][i][j];
          cmx[j] = fmaxf(cmx[j], fabsf(acc[t][i][j]));
        }
        const float mul = SQ ? mq[t][i >> 1] : rq[i];
        const uint32_t q = cvt4<1>(acc[t][i][0] * mul, acc[t][i][1] * mul, acc[t][i][2] * mul, acc[t][i][3] * mul);
        *reinterpret_cast<uint32_t*>(ds + lr * ldn + n0) = q;
        // rows past M fall outside the resource: the hardware drops them
        // (SQ: fp32 dZ only on request; the wgrad reads the codes)
        if (!SQ || p.dz != nullptr)
          __builtin_amdgcn_raw_buffer_store_b128(
              v4u{__float_as_uint(acc[t][i][0]), __float_as_uint(acc[t][i][1]), __float_as_uint(acc[t][i][2]),
                  __float_as_uint(acc[t][i][3])},
              dzr, (uint32_t)(lr * N + n0) * 4u, 0, 0);
        if (p.dz_codes && rowok[i]) *reinterpret_cast<uint32_t*>(p.dz_codes + m * N + n0) = q;
      }
      // reduce over the 16 lanes (rows) sharing these 4 columns; then lane r
      // of the group stores quantity r / 4 of column n0 + r % 4, so one store
      // instruction writes the tile's 4 x 4 partials for all four groups
      float vq[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vq[0][j] = col16_sum(colg[t][j]);
        vq[1][j] = col16_sum(colb[t][j]);
        vq[2][j] = col16_sum(cdb[j]);
        vq[3][j] = col16_max(cmx[j]);
      }
      const int qs = r >> 2, js = r & 3;
      float vj[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vj[q4] = js == 0 ? vq[q4][0] : (js == 1 ? vq[q4][1] : (js == 2 ? vq[q4][2] : vq[q4][3]));
      const float v = qs == 0 ? vj[0] : (qs == 1 ? vj[1] : (qs == 2 ? vj[2] : vj[3]));
      p.part[(size_t)qs * p.nblocks * N + (size_t)nblk * N + n0 + js] = v;
    }
  }
  __syncthreads();
  if constexpr (SQ) {
    // the block's dZ codes, transposed, into the wgrad operand: a thread
    // gathers 16 rows of column n, one 16-byte piece of the interleaved
    // [N][M padded to 128] layout; rows past M hold zero codes, and the last
    // block also writes the zero rows up to the padding
    const int64_t rows_out = blockIdx.x == gridDim.x - 1 ? p.nchm * 128 - m0 : (int64_t)kBM;
    // a thread takes 16 rows x 4 columns: 16 word reads, each 4 x 4 byte
    // block transposed with byte permutes (v_perm selects bytes 0-3 from its
    // second operand, 4-7 from its first), then one piece per column
    // The same for X's codes (staged in LDS for the Z recompute, still
    // intact): the wgrad's other operand, with no pass of its own.
    auto codes_t = [&](const uint8_t* src, int ld, int C, uint8_t* dst) {
      const int n4s = C >> 2;
      const int groups = (int)(rows_out >> 4) * n4s;
      for (int u = tid; u < groups; u += 64 * WAVES) {
        const int q = u / n4s, n = (u - q * n4s) * 4;
        uint32_t col[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          if (q < kMT) {
#pragma unroll
            for (int b = 0; b < 4; ++b) w[b] = *reinterpret_cast<const uint32_t*>(src + (16 * q + 4 * k + b) * ld + n);
          }
          const uint32_t ab_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // a0 b0 a1 b1
          const uint32_t ab_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // a2 b2 a3 b3
          const uint32_t cd_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);  // c0 d0 c1 d1
          const uint32_t cd_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);  // c2 d2 c3 d3
          col[0][k] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);           // a0 b0 c0 d0
          col[1][k] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);           // a1 b1 c1 d1
          col[2][k] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
          col[3][k] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(dst + ilv_offset(n + j, m0 + 16 * q, p.nchm)) =
              make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
      }
    };
    codes_t(ds, ldn, N, p.dzt);
    if constexpr (!NO_LN) codes_t(xs, ldk, K, p.xt);
  }

  // dgrad: D[k][m] = sum_n Wr[k][n] dZq[m][n]; each wavefront owns a run of
  // 16-column tiles of k
  v4f dacc[KTMAX][kMT];
#pragma unroll
  for (int t = 0; t < KTMAX; ++t)
#pragma unroll
    for (int i = 0; i < kMT; ++i) dacc[t][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto dstep = [&](int c, const v8i (&wc)[WB], v8i (&wn)[WB]) {
    if (c + 2 < nchn) rload(c + 2, wn);
    v8i df[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) df[i] = load_frag(ds + (16 * i + r) * ldn, g, 128 * c, N);
    if constexpr (SQ) {
      // lane group g: N block 4c + g (clamped past N, where the codes are
      // zero); W's scale for row k, dZ's for row band i / 2
      const int nbk = min(4 * c + g, (N >> 5) - 1);
      int sa[KTMAX], sb[kMT];
#pragma unroll
      for (int t = 0; t < KTMAX; ++t) sa[t] = t < kt ? p.sw8[((kb0 + 16 * t + r) >> 5) * (N >> 5) + nbk] : 127;
#pragma unroll
      for (int i = 0; i < kMT; ++i) sb[i] = be8[(i >> 1) * (N >> 5) + nbk];
#pragma unroll
      for (int t = 0; t < KTMAX; ++t)
        if (t < kt)
#pragma unroll
          for (int i = 0; i < kMT; ++i) dacc[t][i] = mfma_fp8_scaled<0, 1>(wc[t], df[i], dacc[t][i], sa[t], sb[i]);
    } else {
#pragma unroll
      for (int t = 0; t < KTMAX; ++t)
        if (t < kt)
#pragma unroll
          for (int i = 0; i < kMT; ++i) dacc[t][i] = mfma_fp8<0, 1>(wc[t], df[i], dacc[t][i]);
    }
  };
  for (int c = 0; c < nchn; c += 3) {
    dstep(c, w0, w2);
    if (c + 1 < nchn) dstep(c + 1, w1, w0);
    if (c + 2 < nchn) dstep(c + 2, w2, w1);
  }
  float dsv[kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i) dsv[i] = SQ ? 1.0f : rsc[16 * i + r];
  float swr[KTMAX][4];
#pragma unroll
  for (int t = 0; t < KTMAX; ++t) {
    swr[t][0] = swr[t][1] = swr[t][2] = swr[t][3] = 1.0f;
    if (!SQ && t < kt) {
      const float4 s4 = *reinterpret_cast<const float4*>(p.sw_row + kb0 + 16 * t + 4 * g);
      swr[t][0] = s4.x; swr[t][1] = s4.y; swr[t][2] = s4.z; swr[t][3] = s4.w;
    }
  }
  // Column maxima of |X| over the block's rows, requested here, where the
  // registers are free, so that they arrive while dX goes into LDS.
  // Wavefront w takes columns 64 w .. 64 w + 63 (K <= 512); lane l loads 8
  // columns from 8 (l % 8) of rows l / 8 + 8 j: one 16-byte piece per row.
  // Rows past M fall outside the resource and read as zero.
  constexpr bool XMAX = WAVES == 8 && !SQ;
  const bool xmax = XMAX && p.xpart != nullptr && 64 * wave < K;
  v4u xr[8];
  if constexpr (XMAX) {
    if (xmax) {
      const int64_t rows_here = FULLM ? (int64_t)kBM : min((int64_t)kBM, p.M - m0);
      const __amdgpu_buffer_rsrc_t xrs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.xb) + m0 * K, (short)0, (int)(rows_here * K * 2),
                                            kBufferWord3);
      const int c0 = 64 * wave + 8 * (lane & 7);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        xr[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (uint32_t)(((lane >> 3) + 8 * j) * K + c0) * 2u, 0, 0);
    }
  }
  // dX goes out through LDS, so that every store instruction writes whole
  // row segments: the block's tile [BM][K] (bf16, row stride 2K + 16 bytes)
  // takes the LDS from its start once every wavefront is past the dgrad
  // MFMAs (the dZ codes' last reader) and has read its row scales
  const int ldx = 2 * K + 16;
  uint8_t* dxs = smem;
  __syncthreads();
#pragma unroll
  for (int t = 0; t < KTMAX; ++t) {
    if (t < kt) {
      const int k0 = kb0 + 16 * t + 4 * g;
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = dacc[t][i][j] * dsv[i] * swr[t][j];
        *reinterpret_cast<uint2*>(dxs + (16 * i + r) * ldx + 2 * k0) =
            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
    }
  }
  __syncthreads();
  if constexpr (XMAX) {
    if (xmax) {
      // per lane over its 8 rows (fmaxf drops NaN, as the column quantizer's
      // own maxima do), then over the 8 lanes sharing l % 8: l ^ 8 by a DPP
      // row rotation, l ^ 16 and l ^ 32 by row swaps
      float cm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = xr[j][e];
          cm[2 * e] = fmaxf(cm[2 * e], fabsf(__uint_as_float(wv << 16)));
          cm[2 * e + 1] = fmaxf(cm[2 * e + 1], fabsf(__uint_as_float(wv & 0xFFFF0000u)));
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[e] = rows4_max(dpp_max<0x128>(cm[e]));
      if (lane < 8) {
        float4* dst = reinterpret_cast<float4*>(p.xpart + (size_t)blockIdx.x * K + 64 * wave + 8 * lane);
        dst[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
        dst[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
      }
    }
  }
  // 16 bytes per lane, a wavefront's 64 lanes on consecutive bytes of a row;
  // dX is not read again here: streaming (non-temporal) stores
  const int c16 = K / 8;
  for (int u = tid; u < kBM * c16; u += 64 * WAVES) {
    const int lr = u / c16, c = u - lr * c16;
    if (FULLM || m0 + lr < p.M) {
      const uint4 v = *reinterpret_cast<const uint4*>(dxs + lr * ldx + 16 * c);
      __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p.dx + (m0 + lr) * K) + c);
    }
  }
}

// wgrad partials: part[s][k][n] = sum over m in slice s of Xc^T[k][m] * dZc^T[n][m]
// (codes only).  Workgroup tile 128 (n) x 128 (k); wavefront (wn, wk) in 2 x 2
// owns 64 x 64 = 4 x 4 MFMA tiles.  A = dZc^T rows n (e5m2), B = Xc^T rows k
// (e4m3), both fragment-interleaved with M padded to 128 (zero codes), so
// lane (r, g) holds D[n = 16a + 4g + j][k = 16b + r].  Slice s covers the
// 128-row chunks [s * chunks_per_split, +chunks_per_split).
// SQ: both operands carry E8M0 scales per 32 x 32 block (dZ's [M/32][N/32],
// X's [M/32][K/32]), applied by the MFMA: lane group g of chunk c supplies
// M block 4c + g (clamped past M, where the codes are zero).
// Eight wavefronts: wavefront w owns the 64 x 64 sub-tile w % 4 over one half
// of the slice's chunks (two wavefronts per SIMD); the second half's sums
// join the first's through LDS, in a fixed order.
template <bool SQ>
__global__ __launch_bounds__(512) void k_wgrad(const uint8_t* dzt, const uint8_t* xt, int64_t M, int N, int K,
                                               int64_t chunks_per_split, float* part, const uint8_t* sdz,
                                               const uint8_t* sx8) {
  __shared__ v4f wred[4][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = wave & 3, half = wave >> 2;
  const int r = lane & 15, g = lane >> 4;
  // 1-D grid of (N/128) x (K/128) tiles x slices.  Consecutive workgroups go
  // to the 8 XCDs in turn, and each XCD has its own L2: when the count is a
  // multiple of 8, workgroup i is given the (i % 8)-th eighth of the
  // slice-major order, so the tiles of one slice -- which read the same M
  // rows of both operands -- share an XCD and its L2.
  const int nx = (N + 127) / 128, ny = (K + 127) / 128;
  const int total = (int)gridDim.x, id = (int)blockIdx.x;
  const int lin = (total & 7) == 0 ? (id & 7) * (total >> 3) + (id >> 3) : id;
  const int bz = lin / (nx * ny), tl = lin - bz * (nx * ny), by = tl / nx, bx = tl - by * nx;
  const int n0 = bx * 128 + (sub & 1) * 64;
  const int k0 = by * 128 + (sub >> 1) * 64;
  const int64_t nch = (M + 127) / 128;
  const int64_t c0s = (int64_t)bz * chunks_per_split;
  int64_t c0e = c0s + chunks_per_split;
  if (c0e > nch) c0e = nch;
  const int64_t mid = c0s + (c0e - c0s + 1) / 2;
  const int64_t cs = half ? mid : c0s, ce = half ? c0e : mid;
  v4f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const bool nin = n0 < N, kin = k0 < K;
  if (nin && kin && cs < ce) {
    // the next 128-row chunk's fragments are requested before this chunk's MFMAs
    v8i af[4], bf[4], an[4], bn[4];
    int sa[4], sb[4], san[4], sbn[4];
    const int64_t mbl = M / 32 - 1;
    auto scales = [&](int64_t c, int (&xa)[4], int (&xb)[4]) {
      if constexpr (SQ) {
        const int64_t mb = min(4 * c + g, mbl);
#pragma unroll
        for (int a = 0; a < 4; ++a) xa[a] = sdz[mb * (N >> 5) + ((n0 + 16 * a + r) >> 5)];
#pragma unroll
        for (int b = 0; b < 4; ++b) xb[b] = sx8[mb * (K >> 5) + ((k0 + 16 * b + r) >> 5)];
      }
    };
#pragma unroll
    for (int a = 0; a < 4; ++a) af[a] = load_frag_ilv(dzt, n0 / 16 + a, cs, nch, r, g);
#pragma unroll
    for (int b = 0; b < 4; ++b) bf[b] = load_frag_ilv(xt, k0 / 16 + b, cs, nch, r, g);
    scales(cs, sa, sb);
    for (int64_t c = cs; c < ce; ++c) {
      const int64_t cn = c + 1 < ce ? c + 1 : c;  // past the end: a harmless reload of this chunk
#pragma unroll
      for (int a = 0; a < 4; ++a) an[a] = load_frag_ilv(dzt, n0 / 16 + a, cn, nch, r, g);
#pragma unroll
      for (int b = 0; b < 4; ++b) bn[b] = load_frag_ilv(xt, k0 / 16 + b, cn, nch, r, g);
      scales(cn, san, sbn);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = SQ ? mfma_fp8_scaled<1, 0>(af[a], bf[b], acc[a][b], sa[a], sb[b])
                         : mfma_fp8<1, 0>(af[a], bf[b], acc[a][b]);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        af[a] = an[a];
        bf[a] = bn[a];
        sa[a] = san[a];
        sb[a] = sbn[a];
      }
    }
  }
  if (half == 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) wred[sub][4 * a + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (half == 0 && nin && kin) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v4f o = acc[a][b] + wred[sub][4 * a + b][lane];
        const int n = n0 + 16 * a + 4 * g, k = k0 + 16 * b + r;
        *reinterpret_cast<float4*>(part + ((int64_t)bz * K + k) * N + n) = make_float4(o[0], o[1], o[2], o[3]);
      }
  }
}

// dW[k][n] = (sum_s part[s][k][n]) * sxc[k] * sdzc[n] (no column scales,
// sxc == NULL, when the MFMA applied block scales).  Fixed summation order
// => deterministic.
__device__ __forceinline__ void finalize_body(int64_t blk, const float* wpart, int nsplit, const float* sxc,
                                              const float* sdzc, int K, int N, float* dw) {
  // four consecutive elements of a row of dW per thread (N % 4 == 0); up to
  // sixteen slices' 16-byte loads in flight at once, added in slice order
  const int64_t i = (blk * 256 + threadIdx.x) * 4;
  const int64_t kn = (int64_t)K * N;
  if (i >= kn) return;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto add = [&](const float4& v) {
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  };
  int sp = 0;
  for (; sp + 16 <= nsplit; sp += 16) {
    float4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = *reinterpret_cast<const float4*>(wpart + (int64_t)(sp + q) * kn + i);
#pragma unroll
    for (int q = 0; q < 16; ++q) add(v[q]);
  }
  for (; sp + 4 <= nsplit; sp += 4) {
    float4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const float4*>(wpart + (int64_t)(sp + q) * kn + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) add(v[q]);
  }
  for (; sp < nsplit; ++sp) add(*reinterpret_cast<const float4*>(wpart + (int64_t)sp * kn + i));
  if (sxc != nullptr) {
    const int k = (int)(i / N), n = (int)(i - (int64_t)k * N);
    const float sk = sxc[k];
    const float4 sn = *reinterpret_cast<const float4*>(sdzc + n);
    s = make_float4(s.x * sk * sn.x, s.y * sk * sn.y, s.z * sk * sn.z, s.w * sk * sn.w);
  }
  *reinterpret_cast<float4*>(dw + i) = s;
}

// dgamma, dbeta, dbias from the per-workgroup column partials: block of 256
// threads = 16 columns x 16 subsets of the workgroups (strided, 2 in flight),
// then the subset sums in a fixed order => deterministic.
__device__ __forceinline__ void col_vectors_body(int blk, const float* cpart, int nblocks, int N, float* dgamma,
                                                 float* dbeta, float* dbias) {
  __shared__ float red[3][16][16];
  const int cl = threadIdx.x & 15, part = threadIdx.x >> 4;
  const int n = blk * 16 + cl;
  const size_t plane = (size_t)nblocks * N;
  float a = 0.0f, b = 0.0f, c = 0.0f;
  if (n < N) {
    int bl = part;
    // eight rows of partials per quantity in flight, added in row order
    for (; bl + 112 < nblocks; bl += 128) {
      float va[8], vb[8], vc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const size_t o = (size_t)(bl + 16 * q) * N + n;
        va[q] = cpart[o];
        vb[q] = cpart[plane + o];
        vc[q] = cpart[2 * plane + o];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        a += va[q];
        b += vb[q];
        c += vc[q];
      }
    }
    for (; bl < nblocks; bl += 16) {
      const size_t o = (size_t)bl * N + n;
      a += cpart[o];
      b += cpart[plane + o];
      c += cpart[2 * plane + o];
    }
  }
  red[0][part][cl] = a;
  red[1][part][cl] = b;
  red[2][part][cl] = c;
  __syncthreads();
  if (part == 0 && n < N) {
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      a += red[0][i][cl];
      b += red[1][i][cl];
      c += red[2][i][cl];
    }
    if (dgamma) dgamma[n] = a;
    if (dbeta) dbeta[n] = b;
    if (dbias) dbias[n] = c;
  }
}

// dW (the last nf blocks) and, when requested, dgamma / dbeta / dbias (the
// blocks before them) in one launch: the two reductions are independent.
__global__ __launch_bounds__(256) void k_finalize_vectors(const float* wpart, int nsplit, const float* sxc,
                                                          const float* sdzc, int K, int N, float* dw, int nf,
                                                          const float* cpart, int nblocks, float* dgamma,
                                                          float* dbeta, float* dbias) {
  // the few column-vector blocks first: their longer reductions then overlap
  // the dW blocks instead of trailing them
  const int nv = (int)gridDim.x - nf;
  if ((int)blockIdx.x < nv) col_vectors_body((int)blockIdx.x, cpart, nblocks, N, dgamma, dbeta, dbias);
  else finalize_body((int)blockIdx.x - nv, wpart, nsplit, sxc, sdzc, K, N, dw);
}

// The square-block backward's three MFMA operands in one launch, all
// fragment-interleaved: job 0 the weight codes qw [N][K] as they are (the Z
// recompute), job 1 their transpose [K][N] (the dgrad: W's own rows), job 2
// the X codes' transpose [K][M] (the wgrad).  The transposes go through a
// 64 x 64 LDS tile; their rows are padded with zero codes up to a multiple
// of 128 columns.  One quantization per tensor: no code is recomputed.
struct TJob {
  const uint8_t* src;
  int64_t R, C;  // source [R][C], C % 64 == 0
  uint8_t* dst;  // interleaved [C][R padded to 128]
  int64_t tiles_c, blocks;
};
__global__ __launch_bounds__(256) void k_relayout_sq(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwi,
                                                     int64_t b0, TJob j1, TJob j2) {
  __shared__ uint32_t tile[64][17];  // 64 source rows x 64 bytes, padded
  const int t = threadIdx.x;
  int64_t b = blockIdx.x;
  if (b < b0) {
    const int64_t nch = (K + 127) / 128, pieces = nch * 8;
    const int64_t u = b * 256 + t;
    if (u >= N * pieces) return;
    const int64_t row = u / pieces, col = (u - row * pieces) * 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < K) v = *reinterpret_cast<const uint4*>(qw + row * K + col);
    *reinterpret_cast<uint4*>(qwi + ilv_offset(row, col, nch)) = v;
    return;
  }
  b -= b0;
  const bool first = b < j1.blocks;
  const TJob j = first ? j1 : j2;
  if (!first) b -= j1.blocks;
  const int64_t tr = b / j.tiles_c, tc = b - tr * j.tiles_c;
  // source row 64 tr + t/4, bytes 64 tc + 16 (t%4) .. +16 (rows past R: zeros)
  const int lr = t >> 2, lc = (t & 3) * 4;
  const int64_t srow = 64 * tr + lr;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (srow < j.R) v = *reinterpret_cast<const uint4*>(j.src + srow * j.C + 64 * tc + 4 * lc);
  tile[lr][lc] = v.x; tile[lr][lc + 1] = v.y; tile[lr][lc + 2] = v.z; tile[lr][lc + 3] = v.w;
  __syncthreads();
  // destination row 64 tc + t/4 (a source column), its 16 columns 64 tr + 16 (t%4) .. (source rows)
  const int oc = t >> 2, orr = (t & 3) * 16;
  uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint32_t word = tile[orr + q][oc >> 2];
    w4[q >> 2] |= ((word >> (8 * (oc & 3))) & 0xFFu) << (8 * (q & 3));
  }
  const int64_t nch = (j.R + 127) / 128;
  *reinterpret_cast<uint4*>(j.dst + ilv_offset(64 * tc + oc, 64 * tr + orr, nch)) =
      make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

// The weight's two layouts unless they arrive packed (do_w false), and X's
// transposed codes for M > 0; no launch when neither is needed.
hipError_t launch_relayout_sq(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwi, uint8_t* qwri, bool do_w,
                              const uint8_t* qx, int64_t M, uint8_t* xt, hipStream_t s) {
  const int64_t b0 = do_w ? (N * ((K + 127) / 128) * 8 + 255) / 256 : 0;
  auto job = [](const uint8_t* src, int64_t R, int64_t C, uint8_t* dst) {
    TJob j;
    j.src = src; j.R = R; j.C = C; j.dst = dst;
    j.tiles_c = C / 64;
    j.blocks = (R + 127) / 128 * 2 * j.tiles_c;  // 64-row tiles up to the 128 padding
    return j;
  };
  const TJob j1 = job(qw, do_w ? N : 0, K, qwri), j2 = job(qx, M, K, xt);
  if (b0 + j1.blocks + j2.blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_relayout_sq, dim3((unsigned)(b0 + j1.blocks + j2.blocks)), dim3(256), 0, s, qw, N, K, qwi, b0,
                     j1, j2);
  return hipGetLastError();
}

size_t bwd_lds_bytes(int K, int N, bool sdy, int waves) {
  const size_t main = (size_t)kBM * (K + 16) + (size_t)kBM * (N + 16) + (size_t)(2 * waves * kBM + kBM) * 4 +
                      (sdy ? (size_t)kBM * (2 * N + 16) : 0);
  const size_t dx_tile = (size_t)kBM * (2 * K + 16);  // reuses the LDS at the end
  return main > dx_tile ? main : dx_tile;
}

struct BwdWs {
  size_t part, dz, xt, sxc, xcolp, dzt, sdzc, dzmult, qwi, qwri, wpart, sdz, total;
  int nblocks, nsplit;
  int64_t xnp;
};
// sq: the square-block recipe needs no fp32 dZ, no column maxima or scales,
// only dZ's block scales
BwdWs bwd_ws_layout(int64_t M, int64_t N, int64_t K, bool sq) {
  BwdWs w{};
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  w.nblocks = (int)((M + kBM - 1) / kBM);
  w.nsplit = (int)((M + kWgSplitRows - 1) / kWgSplitRows);
  if (w.nsplit < 1) w.nsplit = 1;
  QuantPlan xq = quant_plan(M, K, 2);
  w.xnp = xq.np;
  size_t o = 0;
  w.part = o; o += al((size_t)4 * w.nblocks * N * 4);
  if (!sq) { w.dz = o; o += al((size_t)M * N * 4); }
  const int64_t mpad = (M + 127) / 128 * 128;
  w.xt = o; o += al((size_t)mpad * K);
  if (!sq) {
    w.sxc = o; o += al((size_t)K * 4);
    // the main kernel's per-block partials (N, K <= 512) or the column
    // quantizer's row-chunk partials, then the column multipliers
    const size_t xfl = (size_t)(w.nblocks + 1) * K;
    w.xcolp = o; o += al((xfl > (size_t)xq.ws_floats ? xfl : (size_t)xq.ws_floats) * 4);
  }
  w.dzt = o; o += al((size_t)mpad * N);
  if (!sq) {
    w.sdzc = o; o += al((size_t)N * 4);
    w.dzmult = o; o += al((size_t)N * 4);
  } else {
    w.sdz = o; o += al((size_t)(M / 32) * (N / 32));
  }
  w.qwi = o; o += al((size_t)N * ((K + 127) / 128 * 128));
  w.qwri = o; o += al((size_t)K * ((N + 127) / 128 * 128));
  w.wpart = o; o += al((size_t)w.nsplit * K * N * 4);
  w.total = o;
  return w;
}

template <int NTMAX, int KTMAX, int WAVES, bool SQ = false>
hipError_t launch_main_t(const BwdBlock& p, int no_ln, hipStream_t s) {
  const size_t lds = bwd_lds_bytes(p.K, p.N, bwd_stage_dy(NTMAX, KTMAX, WAVES), WAVES);
  const dim3 grid((unsigned)p.nblocks);
  const bool full = p.M % kBM == 0;
  auto kern = no_ln ? (full ? k_bwd_main<NTMAX, KTMAX, 1, true, WAVES, SQ> : k_bwd_main<NTMAX, KTMAX, 1, false, WAVES, SQ>)
                    : (full ? k_bwd_main<NTMAX, KTMAX, 0, true, WAVES, SQ> : k_bwd_main<NTMAX, KTMAX, 0, false, WAVES, SQ>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), lds, s, p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sq) { return bwd_ws_layout(M, N, K, sq).total; }

hipError_t launch_bwd(const BwdLaunch& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const BwdWs w = bwd_ws_layout(a.M, a.N, a.K, a.sq);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  BwdBlock p;
  p.M = a.M; p.N = (int)a.N; p.K = (int)a.K;
  p.dy = static_cast<const uint16_t*>(a.dy);
  p.qx = a.qx; p.mean = a.mean; p.rstd = a.rstd;
  p.qw = a.qw;
  p.sx = a.sq ? nullptr : static_cast<const float*>(a.sx);
  p.sw = a.sq ? nullptr : static_cast<const float*>(a.sw);
  p.sx8 = a.sq ? static_cast<const uint8_t*>(a.sx) : nullptr;
  p.sw8 = a.sq ? static_cast<const uint8_t*>(a.sw) : nullptr;
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.gamma = static_cast<const uint16_t*>(a.gamma);
  p.qw_row = a.qw_row; p.sw_row = a.sw_row;
  p.dx = static_cast<uint16_t*>(a.dx);
  p.dz = a.dz ? a.dz : (a.sq ? nullptr : reinterpret_cast<float*>(ws + w.dz));
  p.dz_codes = a.dz_codes;
  p.dz_scales = a.sq ? nullptr : static_cast<float*>(a.dz_scales);
  p.part = reinterpret_cast<float*>(ws + w.part);
  p.nblocks = w.nblocks;
  p.qwi = a.w_packed ? a.qw : ws + w.qwi;
  p.qwri = a.w_packed ? a.qw_row : ws + w.qwri;
  p.sdz = a.sq ? (a.dz_scales ? static_cast<uint8_t*>(a.dz_scales) : ws + w.sdz) : nullptr;
  p.dzt = ws + w.dzt;
  p.nchm = (a.M + 127) / 128;
  p.xt = nullptr;
  // N, K <= 512 (eight wavefronts): the main kernel also takes X's column
  // maxima per block, in place of the column quantizer's first pass
  const bool xmax_fused = !a.sq && a.N <= 512 && a.K <= 512;
  p.xb = static_cast<const uint16_t*>(a.x);
  p.xpart = xmax_fused ? reinterpret_cast<float*>(ws + w.xcolp) : nullptr;

  hipError_t e;
  if (a.sq) {
    // square-block recipe: the forward's codes, rearranged (no requantization),
    // the main kernel (dZ quantized once, in blocks), the wgrad on the codes
    // and the final sums; N, K <= 512
    // (with the LayerNorm the main kernel writes X's transposed codes from
    // its staged copy; the literal reading stages no X, so the relayout
    // transposes them; packed weights need no rearrangement)
    uint8_t* xt = ws + w.xt;
    p.xt = xt;
    if ((e = launch_relayout_sq(a.qw, a.N, a.K, ws + w.qwi, ws + w.qwri, !a.w_packed, a.qx, a.no_ln ? a.M : 0, xt,
                                s)) != hipSuccess)
      return e;
    if ((e = launch_main_t<4, 4, 8, true>(p, a.no_ln, s)) != hipSuccess) return e;
    float* wpart = reinterpret_cast<float*>(ws + w.wpart);
    dim3 g((unsigned)(((a.N + 127) / 128) * ((a.K + 127) / 128) * w.nsplit));
    hipLaunchKernelGGL(k_wgrad<true>, g, dim3(512), 0, s, p.dzt, xt, a.M, (int)a.N, (int)a.K,
                       (int64_t)(kWgSplitRows / 128), wpart, p.sdz, p.sx8);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t tot = a.K * a.N;
    const int nf = (int)((tot + 1023) / 1024);
    const int nv = (a.dgamma || a.dbeta || a.dbias) ? (int)((a.N + 15) / 16) : 0;
    hipLaunchKernelGGL(k_finalize_vectors, dim3((unsigned)(nf + nv)), dim3(256), 0, s, wpart, w.nsplit,
                       (const float*)nullptr, (const float*)nullptr, (int)a.K, (int)a.N, a.dw, nf, p.part, w.nblocks,
                       a.dgamma, a.dbeta, a.dbias);
    return hipGetLastError();
  }
  // both weights into the fragment-interleaved order, in one launch (unless
  // they arrive in it)
  if (!a.w_packed &&
      (e = launch_relayout2(a.no_ln ? nullptr : a.qw, a.N, a.K, ws + w.qwi, a.qw_row, a.K, a.N, ws + w.qwri, s)) !=
          hipSuccess)
    return e;
  // N, K <= 512: eight wavefronts of at most four 16-column tiles each;
  // else four wavefronts of at most eight or sixteen
  if (a.N <= 512 && a.K <= 512) e = launch_main_t<4, 4, 8>(p, a.no_ln, s);
  else if (a.N <= 512) e = launch_main_t<8, 16, 4>(p, a.no_ln, s);
  else if (a.K <= 512) e = launch_main_t<16, 8, 4>(p, a.no_ln, s);
  else e = launch_main_t<16, 16, 4>(p, a.no_ln, s);
  if (e != hipSuccess) return e;

  // column quantization of X (e4m3) and dZ (e5m2), both transposed to [*, M]
  // (into the caller's buffers when it asks for them)
  uint8_t* xt = a.xc_codes ? a.xc_codes : ws + w.xt;
  float* sxc = a.xc_scales ? a.xc_scales : reinterpret_cast<float*>(ws + w.sxc);
  uint8_t* dzt = a.dzc_codes ? a.dzc_codes : ws + w.dzt;
  float* sdzc = a.dzc_scales ? a.dzc_scales : reinterpret_cast<float*>(ws + w.sdzc);
  // X: column maxima (per-block partials from the main kernel, or row-chunk
  // partials); then the column scales of X and of dZ (whose partials the
  // main kernel wrote) in one launch, and both casts in one launch
  float* xcolp = reinterpret_cast<float*>(ws + w.xcolp);
  int64_t xnp = w.nblocks;
  if (!xmax_fused && (e = launch_col_amax_partials(a.x, 0, a.M, a.K, a.K, xcolp, &xnp, s)) != hipSuccess) return e;
  const float* dzmax = p.part + (size_t)3 * w.nblocks * a.N;
  ColQuantJob jx{a.x, 0, 0, a.M, a.K, a.K, xcolp, xnp, xt, sxc, xcolp + xnp * a.K};
  ColQuantJob jd{p.dz, 1, 1, a.M, a.N, a.N, dzmax, w.nblocks, dzt, sdzc, reinterpret_cast<float*>(ws + w.dzmult)};
  if ((e = launch_col_quant_pair(jx, jd, s)) != hipSuccess) return e;

  float* wpart = reinterpret_cast<float*>(ws + w.wpart);
  dim3 g((unsigned)(((a.N + 127) / 128) * ((a.K + 127) / 128) * w.nsplit));
  hipLaunchKernelGGL(k_wgrad<false>, g, dim3(512), 0, s, dzt, xt, a.M, (int)a.N, (int)a.K,
                     (int64_t)(kWgSplitRows / 128), wpart, (const uint8_t*)nullptr, (const uint8_t*)nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tot = a.K * a.N;
  const int nf = (int)((tot + 1023) / 1024);  // four elements per thread
  const int nv = (a.dgamma || a.dbeta || a.dbias) ? (int)((a.N + 15) / 16) : 0;
  hipLaunchKernelGGL(k_finalize_vectors, dim3((unsigned)(nf + nv)), dim3(256), 0, s, wpart, w.nsplit, sxc, sdzc,
                     (int)a.K, (int)a.N, a.dw, nf, p.part, w.nblocks, a.dgamma, a.dbeta, a.dbias);
  return hipGetLastError();
}

}  // namespace loka
