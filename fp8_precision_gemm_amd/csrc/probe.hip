// The Probe's statistics ([LoKA] section III-A1, "Online Distribution
// Learning" and "Sampling learned distributions"): the input tracker's
// batched mean/scatter merge (Chan, Golub and LeVeque's pairwise update,
// accumulated in fp32 as the pages note), the weight tracker's matrix-normal
// Kronecker flip-flop with an EMA (Cholesky factors and linear solves, no
// explicit inverses; the EMA results symmetrized with eps I added, then
// the trace renormalization) and the two samplers.  All work
// is fp32 vector arithmetic: the Probe runs every hundred or so steps, off
// the training step's path, on K x K and R x C problems.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace loka {
namespace {

constexpr int kPT = 256;     // threads of the element-wise and GEMM kernels
constexpr int kGT = 64;      // GEMM tile (output rows and columns)
constexpr int kGK = 64;      // GEMM depth per LDS stage

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- element-wise ----------------------------------------------------------

// column sums of a bf16 [B][K] over row chunks: part[chunk][k] (rows in order)
__global__ __launch_bounds__(kPT) void k_colsum(const uint16_t* T, int64_t B, int K, int64_t rows_per, float* part) {
  const int k = blockIdx.x * kPT + threadIdx.x;
  if (k >= K) return;
  const int64_t b0 = (int64_t)blockIdx.y * rows_per, b1 = min(b0 + rows_per, B);
  float s = 0.0f;
  // rows in order; the unrolled loop keeps 16 loads in flight per thread
#pragma unroll 16
  for (int64_t b = b0; b < b1; ++b) s += bf16_lo(T[b * K + k]);
  part[(int64_t)blockIdx.y * K + k] = s;
}

// batch mean, its difference to the running mean and the merged mean:
// mu_b = sum / B, d = mu_b - mu, mu <- mu + (B / n') d
__global__ __launch_bounds__(kPT) void k_mean_merge(const float* part, int nch, int64_t B, int K, float frac,
                                                    float* mu, float* mu_b, float* d) {
  const int k = blockIdx.x * kPT + threadIdx.x;
  if (k >= K) return;
  float s = 0.0f;
#pragma unroll 16
  for (int c = 0; c < nch; ++c) s += part[(int64_t)c * K + k];
  const float mb = s / (float)B;
  const float dd = mb - mu[k];
  mu_b[k] = mb;
  d[k] = dd;
  mu[k] = mu[k] + frac * dd;
}

// Tc = T - mu_b (fp32)
__global__ __launch_bounds__(kPT) void k_center(const uint16_t* T, int64_t n, int K, const float* mu_b, float* Tc) {
  const int64_t i = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (i < n) Tc[i] = bf16_lo(T[i]) - mu_b[i % K];
}

// weight tracker, first update: M = W, U = I, V = I
__global__ __launch_bounds__(kPT) void k_weight_init(const uint16_t* W, int64_t RC, int R, int C, float* M, float* U,
                                                     float* V) {
  const int64_t i = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (i < RC) M[i] = bf16_lo(W[i]);
  if (i < (int64_t)R * R) U[i] = (i / R == i % R) ? 1.0f : 0.0f;
  if (i < (int64_t)C * C) V[i] = (i / C == i % C) ? 1.0f : 0.0f;
}

// M <- m M + (1 - m) W; Wc = W - M [R][C] and its transpose WcT [C][R] (the
// right-hand sides of the two solves, each solved in place)
__global__ __launch_bounds__(kPT) void k_weight_ema(const uint16_t* W, int64_t RC, int C, int R, float m, float* M,
                                                    float* Wc, float* WcT) {
  const int64_t i = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (i >= RC) return;
  const float w = bf16_lo(W[i]);
  const float mm = m * M[i] + (1.0f - m) * w;
  M[i] = mm;
  Wc[i] = w - mm;
  const int64_t r = i / C, c = i - r * C;
  WcT[c * R + r] = w - mm;
}

// tr[0] = trace(U), tr[1] = trace(V) (one workgroup, fixed order)
__global__ __launch_bounds__(kPT) void k_trace_pair(const float* U, int R, const float* V, int C, float* tr) {
  __shared__ float red[2][kPT / 64];
  float tu = 0.0f, tv = 0.0f;
  for (int i = threadIdx.x; i < R; i += kPT) tu += U[(int64_t)i * R + i];
  for (int i = threadIdx.x; i < C; i += kPT) tv += V[(int64_t)i * C + i];
  tu = wave_sum(tu);
  tv = wave_sum(tv);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = tu;
    red[1][threadIdx.x >> 6] = tv;
  }
  __syncthreads();
  if (threadIdx.x < 2) tr[threadIdx.x] = red[threadIdx.x][0] + red[threadIdx.x][1] + red[threadIdx.x][2] + red[threadIdx.x][3];
}

// the EMA results made symmetric and regularized, in place:
// A <- (A + A^T) / 2 + eps I with eps = 1e-6 trace(A) / n (trace before the
// step), for U (n = R) and V (n = C).  Thread e handles the pair (i, j),
// i <= j, of element e = i n + j and writes both entries, so no entry is
// read after another thread wrote it.
__global__ __launch_bounds__(kPT) void k_sym_eps(float* U, int R, float* V, int C, const float* tr) {
  const int64_t e = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (e < (int64_t)R * R) {
    const int64_t i = e / R, j = e - i * R;
    if (i <= j) {
      float a = 0.5f * (U[i * R + j] + U[j * R + i]);
      if (i == j) a += 1e-6f * tr[0] / (float)R;
      U[i * R + j] = a;
      U[j * R + i] = a;
    }
  }
  if (e < (int64_t)C * C) {
    const int64_t i = e / C, j = e - i * C;
    if (i <= j) {
      float a = 0.5f * (V[i * C + j] + V[j * C + i]);
      if (i == j) a += 1e-6f * tr[1] / (float)C;
      V[i * C + j] = a;
      V[j * C + i] = a;
    }
  }
}

// s = trace(U) / R (one workgroup), then U /= s, V *= s
__global__ __launch_bounds__(kPT) void k_trace(const float* U, int R, float* s) {
  __shared__ float red[kPT / 64];
  float t = 0.0f;
  for (int i = threadIdx.x; i < R; i += kPT) t += U[(int64_t)i * R + i];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) s[0] = (red[0] + red[1] + red[2] + red[3]) / (float)R;
}
__global__ __launch_bounds__(kPT) void k_renorm(const float* s, int64_t RR, int64_t CC, float* U, float* V) {
  const int64_t i = (int64_t)blockIdx.x * kPT + threadIdx.x;
  const float sc = s[0];
  if (i < RR) U[i] = U[i] / sc;
  if (i < CC) V[i] = V[i] * sc;
}

// C = beta C + alpha sum_z P[z] (z in order) + coef d_i d_j + row[j] + mat[i][j];
// the result as fp32 (C, row stride ldc; 0 = N) or bf16 (Cb); absent terms
// are null; lower: only the entries j <= i.
struct ReduceJob {
  int64_t M, N;
  int splits;
  const float* P;
  float alpha, beta, coef;
  const float* d;
  const float* row;
  const float* mat;
  float* C;
  uint16_t* Cb;
  int64_t ldc;
  int lower;
};
// the output element (i, j) from the sum s of its slices
__device__ __forceinline__ void reduce_out(const ReduceJob& r, int64_t i, int64_t j, float s) {
  const int64_t e = i * r.N + j;
  const int64_t ce = r.ldc > 0 ? i * r.ldc + j : e;
  float c = r.alpha * s;
  if (r.beta != 0.0f) c += r.beta * r.C[ce];
  if (r.d != nullptr) c += r.coef * r.d[i] * r.d[j];
  if (r.row != nullptr) c += r.row[j];
  if (r.mat != nullptr) c += r.mat[e];
  if (r.Cb != nullptr) r.Cb[e] = (uint16_t)f32_to_bf16_bits(c);
  else r.C[ce] = c;
}
__global__ __launch_bounds__(kPT) void k_reduce(ReduceJob r) {
  const int64_t e = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (e >= r.M * r.N) return;
  const int64_t i = e / r.N, j = e - i * r.N;
  if (r.lower && j > i) return;
  float s = 0.0f;
  for (int z = 0; z < r.splits; ++z) s += r.P[(int64_t)z * r.M * r.N + e];
  reduce_out(r, i, j, s);
}

// ---- GEMM: P[z] = A B^T over the z-th slice of the contraction ----------------
// A(i, k) = A[i * a_rs + k * a_cs], B(j, k) = B[j * b_rs + k * b_cs]; a 64 x 64
// output tile per workgroup, 64-deep LDS stages, fp32 MFMA (fp32 products
// and sums).
struct GemmJob {
  int64_t M, N, K, kper;
  const float* A;
  int64_t a_rs, a_cs;
  const float* B;
  int64_t b_rs, b_cs;
  float* P;  // [splits][M][N]
};
// One slice (gridDim.z == 1): the reduction's output is written directly.
// Staging: an operand contiguous along the contraction is read 64 elements
// per row by consecutive threads, else 64 rows per depth step.
__global__ __launch_bounds__(kPT) void k_gemm_f32(GemmJob g, ReduceJob red) {
  __shared__ float As[kGK][kGT + 4], Bs[kGK][kGT + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wavefront (wm, wn) owns the 32 x 32 quarter (rows 32 wm.., columns 32 wn..)
  // as 2 x 2 tiles of v_mfma_f32_16x16x4_f32: lane l supplies A(i = l % 16,
  // k = l / 16) and B(k = l / 16, j = l % 16) and holds D(4 (l / 16) + r, l % 16)
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 15, lg = lane >> 4;
  const int64_t i0 = (int64_t)blockIdx.y * kGT, j0 = (int64_t)blockIdx.x * kGT;
  const int64_t k0 = (int64_t)blockIdx.z * g.kper, k1 = min(k0 + g.kper, g.K);
  v4f acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t kk = k0; kk < k1; kk += kGK) {
    // stage: 64 x 64 of each operand, 16 elements per thread, every load
    // issued before the LDS writes.  Thread (hi0, lo) takes elements
    // (hi0 + 4q, lo) of the tile, lo along the operand's contiguous axis.
    static_assert(kGK == kGT && kGT == 64, "square 64 x 64 stages");
    const int lo = threadIdx.x & 63, hi0 = threadIdx.x >> 6;
    const bool ac = g.a_cs == 1, bc = g.b_cs == 1;
    const float* pa = g.A + (ac ? (i0 + hi0) * g.a_rs + (kk + lo) : (i0 + lo) * g.a_rs + (kk + hi0) * g.a_cs);
    const float* pb = g.B + (bc ? (j0 + hi0) * g.b_rs + (kk + lo) : (j0 + lo) * g.b_rs + (kk + hi0) * g.b_cs);
    const int64_t sa = 4 * (ac ? g.a_rs : g.a_cs), sb = 4 * (bc ? g.b_rs : g.b_cs);
    // bounds: (row, depth) of element q is (i0 + hi0 + 4q, kk + lo) or (i0 + lo, kk + hi0 + 4q)
    const int64_t ra = ac ? g.M - i0 - hi0 : k1 - kk - hi0, rb = bc ? g.N - j0 - hi0 : k1 - kk - hi0;
    const bool fa = ac ? kk + lo < k1 : i0 + lo < g.M, fb = bc ? kk + lo < k1 : j0 + lo < g.N;
    float ta[16], tb[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      ta[q] = (fa && 4 * q < ra) ? pa[q * sa] : 0.0f;
      tb[q] = (fb && 4 * q < rb) ? pb[q * sb] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int hi = hi0 + 4 * q;
      if (ac) As[lo][hi] = ta[q];
      else As[hi][lo] = ta[q];
      if (bc) Bs[lo][hi] = tb[q];
      else Bs[hi][lo] = tb[q];
    }
    __syncthreads();
#pragma unroll 2
    for (int ks = 0; ks < kGK / 4; ++ks) {
      const int kq = 4 * ks + lg;
      float a[2], b[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[u] = As[kq][32 * wm + 16 * u + lr];
        b[u] = Bs[kq][32 * wn + 16 * u + lr];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[v], acc[u][v], 0, 0, 0);
    }
    __syncthreads();
  }
  float* P = g.P + (int64_t)blockIdx.z * g.M * g.N;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + 32 * wm + 16 * u + 4 * lg + r, j = j0 + 32 * wn + 16 * v + lr;
        if (i >= g.M || j >= g.N) continue;
        if (gridDim.z == 1) {
          if (!red.lower || j <= i) reduce_out(red, i, j, acc[u][v][r]);
        } else {
          P[i * g.N + j] = acc[u][v][r];
        }
      }
}

// ---- Cholesky, blocked right-looking: L L^T = a A + eps I ----------------------
// eps = 1e-6 trace(a A) / n.  L starts as the lower triangle of a A + eps I;
// per 64-column panel: one wavefront factors the diagonal block
// (k_potrf_block), the rows below solve against it (k_trsm_panel), and the
// trailing lower triangle takes the panel's product away (the GEMM, with the
// reduction in its epilogue).  A non-positive pivot sets *info to
// its 1-based column (the first one met); the factor is then not valid.
constexpr int kPanel = 64;

__global__ __launch_bounds__(kPT) void k_chol_eps(const float* A, int n, float a, float* eps, int* info) {
  __shared__ float red[kPT / 64];
  float t = 0.0f;
  for (int i = threadIdx.x; i < n; i += kPT) t += A[(int64_t)i * n + i];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    eps[0] = 1e-6f * a * (red[0] + red[1] + red[2] + red[3]) / (float)n;
    *info = 0;
  }
}
__global__ __launch_bounds__(kPT) void k_chol_init(const float* A, int n, float a, const float* eps, float* L) {
  const int64_t e = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (e >= (int64_t)n * n) return;
  const int64_t i = e / n, j = e - i * n;
  L[e] = j > i ? 0.0f : a * A[e] + (i == j ? eps[0] : 0.0f);
}

// factor the b x b diagonal block at (jb, jb) of L in place (b <= 64).  One
// wavefront, lane i holding row i in registers.  Column c: the pivot comes
// from lane c, the rows below scale by its reciprocal square root, the
// column's entries reach every lane by readlane, and each row's later columns
// take their update (fused multiply-adds in column order, as in the textbook
// right-looking factorization).  Lanes past b and the entries
// above the diagonal carry values that are never used or stored.
__global__ __launch_bounds__(64) void k_potrf_block(float* L, int n, int jb, int b, int* info) {
  const int i = threadIdx.x;
  const float* src = L + (int64_t)(jb + min(i, b - 1)) * n + jb;
  float a[kPanel];
#pragma unroll
  for (int j = 0; j < kPanel; ++j) a[j] = (j <= i && j < b) ? src[j] : 0.0f;
#pragma unroll
  for (int c = 0; c < kPanel; ++c) {
    if (c < b) {
      float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[c]), c));
      if (!(d > 0.0f)) {
        if (i == 0 && *info == 0) *info = jb + c + 1;
        d = 1e-30f;
      }
      // one reciprocal square root on the column's chain: the pivot is
      // d / sqrt(d) and the rows below scale by 1 / sqrt(d)
      const float rp = rsqrtf(d);
      a[c] = i == c ? d * rp : a[c] * rp;
      // L_kc from lane k as a scalar operand of every lane's update
#pragma unroll
      for (int k = c + 1; k < kPanel; ++k)
        a[k] = fmaf(-a[c], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[c]), k)), a[k]);
    }
  }
  if (i < b) {
    float* dst = L + (int64_t)(jb + i) * n + jb;
#pragma unroll
    for (int j = 0; j < kPanel; ++j)
      if (j < b) dst[j] = j <= i ? a[j] : 0.0f;
  }
}

// Rows v of X [count][ldx], columns jb .. jb+b: x <- x L_jj^-T with L_jj the
// b x b diagonal block of L at (jb, jb): forward substitution per row, one
// row per thread in registers.  Right-looking: once x_c is final it updates
// every later x_k with L_kc, so each x_k takes the same fused multiply-adds
// in the same order as the row-by-row form (c ascending), but the chain of
// dependent steps is b long instead of b^2 / 2.  x_c is scaled by the
// diagonal entry's reciprocal (at most one rounding more than a division).  The block is kept in LDS by
// columns (LT[c][k] = L_kc), read as broadcasts; X rows go straight between
// HBM and registers.
constexpr int kTrsmRows = 64;  // rows (threads) per workgroup
constexpr int kLTS = kPanel + 4;  // LT row stride (floats): 16-byte aligned rows
// FULL: b == 64, no per-column guards (the compiler then keeps more of the
// block's reads in flight)
template <bool FULL>
__global__ __launch_bounds__(kTrsmRows, 1) void k_trsm_panel(float* X, int64_t count, int64_t ldx, const float* L,
                                                          int ldl, int jb, int b) {
  __shared__ __align__(16) float LT[kPanel][kLTS];
  __shared__ __align__(16) float rdg[kPanel];
  if (FULL) b = kPanel;
  const int tid = threadIdx.x;
  const int64_t v = (int64_t)blockIdx.x * kTrsmRows + tid;
  // thread k stages row k of the block as column k of LT; every load in flight
  {
    const float* lrow = L + (int64_t)(jb + min(tid, b - 1)) * ldl + jb;
    float t[kPanel];
#pragma unroll
    for (int c = 0; c < kPanel; ++c) t[c] = (c <= tid && c < b && tid < b) ? lrow[c] : 0.0f;
#pragma unroll
    for (int c = 0; c < kPanel; ++c) LT[c][tid] = t[c];
  }
  // the diagonal's reciprocals, off the substitution's dependency chain (a
  // thread reads back only the entry it wrote itself); the whole-panel
  // variant keeps them in place of the diagonal
  if constexpr (FULL) LT[tid][tid] = 1.0f / LT[tid][tid];
  else rdg[tid] = tid < b ? 1.0f / LT[tid][tid] : 0.0f;
  // this thread's row straight into registers (rows past count read row 0
  // and are never stored)
  float* xrow = X + (v < count ? v : 0) * ldx + jb;
  float x[kPanel];
#pragma unroll
  for (int c = 0; c < kPanel; ++c) x[c] = c < b ? xrow[c] : 0.0f;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kPanel; ++c) {
    if (FULL || c < b) {
      x[c] = x[c] * (FULL ? LT[c][c] : rdg[c]);
#pragma unroll
      for (int k = c + 1; k < kPanel; ++k) x[k] = fmaf(-x[c], LT[c][k], x[k]);
    }
  }
  if (v < count) {
#pragma unroll
    for (int c = 0; c < kPanel; ++c)
      if (c < b) xrow[c] = x[c];
  }
}

// ---- standard normals from Philox4x64-10 (Salmon et al., SC'11) ----------------
// Block i: counter (i, 0, 0, 0), key (seed, 0); its four 64-bit outputs give
// two uniform pairs u = (w >> 11) 2^-53 and Box-Muller normals
// sqrt(-2 ln(1 - u1)) (cos 2 pi u2, sin 2 pi u2), stored in order.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}
__global__ __launch_bounds__(kPT) void k_normals(float* z, int64_t count, uint64_t seed) {
  const int64_t blk = (int64_t)blockIdx.x * kPT + threadIdx.x;
  if (blk * 4 >= count) return;
  uint64_t c[4] = {(uint64_t)blk, 0, 0, 0};
  philox4x64_10(c, seed, 0);
  const double two_pi = 6.283185307179586476925286766559;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const double u1 = (double)(c[2 * p] >> 11) * 0x1.0p-53, u2 = (double)(c[2 * p + 1] >> 11) * 0x1.0p-53;
    const double rr = sqrt(-2.0 * log(1.0 - u1)), t = two_pi * u2;
    const int64_t j = blk * 4 + 2 * p;
    if (j < count) z[j] = (float)(rr * cos(t));
    if (j + 1 < count) z[j + 1] = (float)(rr * sin(t));
  }
}

// ---- host helpers --------------------------------------------------------------

unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

constexpr int64_t kSplitDepth = 1024;  // contraction per GEMM slice
int64_t gemm_splits(int64_t K) { return K <= kSplitDepth ? 1 : (K + kSplitDepth - 1) / kSplitDepth; }

void trsm_panel(float* X, int64_t count, int64_t ldx, const float* L, int ldl, int jb, int b, hipStream_t s) {
  if (b == kPanel)
    hipLaunchKernelGGL(k_trsm_panel<true>, dim3(blocks(count, kTrsmRows)), dim3(kTrsmRows), 0, s, X, count, ldx, L, ldl,
                       jb, b);
  else
    hipLaunchKernelGGL(k_trsm_panel<false>, dim3(blocks(count, kTrsmRows)), dim3(kTrsmRows), 0, s, X, count, ldx, L,
                       ldl, jb, b);
}

hipError_t gemm(const GemmJob& j0, const ReduceJob& r0, hipStream_t s) {
  GemmJob j = j0;
  ReduceJob r = r0;
  const int64_t sp = gemm_splits(j.K);
  j.kper = (j.K + sp - 1) / sp;
  j.kper = (j.kper + kGK - 1) / kGK * kGK;
  r.M = j.M; r.N = j.N; r.splits = (int)sp; r.P = j.P;
  hipLaunchKernelGGL(k_gemm_f32, dim3(blocks(j.N, kGT), blocks(j.M, kGT), (unsigned)sp), dim3(kPT), 0, s, j, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp == 1) return e;
  hipLaunchKernelGGL(k_reduce, dim3(blocks(j.M * j.N, kPT)), dim3(kPT), 0, s, r);
  return hipGetLastError();
}

// L L^T = a A + eps I (scal: one float of workspace, P: n*n floats of workspace)
hipError_t cholesky(const float* A, int n, float a, float* L, int* info, float* scal, float* P, hipStream_t s) {
  hipLaunchKernelGGL(k_chol_eps, dim3(1), dim3(kPT), 0, s, A, n, a, scal, info);
  hipLaunchKernelGGL(k_chol_init, dim3(blocks((int64_t)n * n, kPT)), dim3(kPT), 0, s, A, n, a, scal, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int jb = 0; jb < n; jb += kPanel) {
    const int b = min(kPanel, n - jb), r = n - jb - b;
    hipLaunchKernelGGL(k_potrf_block, dim3(1), dim3(64), 0, s, L, n, jb, b, info);
    if (r > 0) {
      float* below = L + (int64_t)(jb + b) * n;
      trsm_panel(below, (int64_t)r, (int64_t)n, L, n, jb, b, s);
      ReduceJob rj{};
      rj.alpha = -1.0f; rj.beta = 1.0f; rj.C = below + jb + b; rj.ldc = n; rj.lower = 1;
      if ((e = gemm(GemmJob{r, r, b, 0, below + jb, n, 1, below + jb, n, 1, P}, rj, s)) != hipSuccess) return e;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// X [count][n] <- X L^-T in place (each row: L x = row), blocked by panels
hipError_t trsm_rows(float* X, int64_t count, int n, const float* L, float* P, hipStream_t s) {
  hipError_t e;
  for (int jb = 0; jb < n; jb += kPanel) {
    const int b = min(kPanel, n - jb), r = n - jb - b;
    trsm_panel(X, count, (int64_t)n, L, n, jb, b, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (r > 0) {
      // X[:, jb+b:] -= X[:, jb:jb+b] L[jb+b:, jb:jb+b]^T
      ReduceJob rj{};
      rj.alpha = -1.0f; rj.beta = 1.0f; rj.C = X + jb + b; rj.ldc = n;
      if ((e = gemm(GemmJob{count, r, b, 0, X + jb, n, 1, L + (int64_t)(jb + b) * n + jb, n, 1, P}, rj, s)) !=
          hipSuccess)
        return e;
    }
  }
  return hipSuccess;
}

hipError_t normals(float* z, int64_t count, uint64_t seed, hipStream_t s) {
  hipLaunchKernelGGL(k_normals, dim3(blocks((count + 3) / 4, kPT)), dim3(kPT), 0, s, z, count, seed);
  return hipGetLastError();
}

size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// ---- the four operations ---------------------------------------------------------

int64_t probe_colsum_chunks(int64_t B) { return B < 256 ? 1 : min((int64_t)64, B / 256); }

size_t probe_input_ws(int64_t B, int64_t K) {
  const int64_t nch = probe_colsum_chunks(B);
  return al256((size_t)nch * K * 4) + 2 * al256((size_t)K * 4) + al256((size_t)B * K * 4) +
         al256((size_t)gemm_splits(B) * K * K * 4);
}

hipError_t probe_input_update(const ProbeInputLaunch& a, hipStream_t s) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const int64_t nch = probe_colsum_chunks(a.B), K = a.K;
  float* part = reinterpret_cast<float*>(ws);
  float* mu_b = reinterpret_cast<float*>(ws + al256((size_t)nch * K * 4));
  float* d = mu_b + al256((size_t)K * 4) / 4;
  float* Tc = d + al256((size_t)K * 4) / 4;
  float* P = Tc + al256((size_t)a.B * K * 4) / 4;
  const int64_t rows_per = (a.B + nch - 1) / nch;
  const uint16_t* T = static_cast<const uint16_t*>(a.T);
  hipLaunchKernelGGL(k_colsum, dim3(blocks(K, kPT), (unsigned)nch), dim3(kPT), 0, s, T, a.B, (int)K, rows_per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_new = a.n_old + a.B;
  hipLaunchKernelGGL(k_mean_merge, dim3(blocks(K, kPT)), dim3(kPT), 0, s, part, (int)nch, a.B, (int)K,
                     (float)((double)a.B / (double)n_new), a.mu, mu_b, d);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_center, dim3(blocks(a.B * K, kPT)), dim3(kPT), 0, s, T, a.B * K, (int)K, mu_b, Tc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // S <- S + Tc^T Tc + (n B / n') d d^T
  GemmJob g{K, K, a.B, 0, Tc, 1, K, Tc, 1, K, P};
  ReduceJob r{};
  r.alpha = 1.0f; r.beta = 1.0f; r.coef = (float)((double)a.n_old * (double)a.B / (double)n_new);
  r.d = d; r.C = a.S;
  return gemm(g, r, s);
}


size_t probe_weight_ws(int64_t R, int64_t C) {
  const size_t p = max(max((size_t)R * C, (size_t)max(R * R, C * C)),
                       (size_t)max(gemm_splits(C) * R * R, gemm_splits(R) * C * C));
  return 2 * al256((size_t)R * C * 4) + al256((size_t)R * R * 4) + al256((size_t)C * C * 4) + al256(p * 4) + 256;
}

hipError_t probe_weight_update(const ProbeWeightLaunch& a, hipStream_t s) {
  const int64_t R = a.R, C = a.C, RC = R * C;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  if (a.first) {
    hipLaunchKernelGGL(k_weight_init, dim3(blocks(max(RC, max(R * R, C * C)), kPT)), dim3(kPT), 0, s, W, RC, (int)R,
                       (int)C, a.M, a.U, a.V);
    return hipGetLastError();
  }
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const size_t rc = al256((size_t)RC * 4);
  float* Wt = reinterpret_cast<float*>(ws);        // Wc, then Wc LV^-T
  float* WuT = reinterpret_cast<float*>(ws + rc);  // Wc^T, then (LU^-1 Wc)^T
  float* LU = reinterpret_cast<float*>(ws + 2 * rc);
  float* LV = LU + al256((size_t)R * R * 4) / 4;
  float* P = LV + al256((size_t)C * C * 4) / 4;
  const size_t pn = max(max((size_t)R * C, (size_t)max(R * R, C * C)),
                        (size_t)max(gemm_splits(C) * R * R, gemm_splits(R) * C * C));
  float* sc = P + al256(pn * 4) / 4;
  hipLaunchKernelGGL(k_weight_ema, dim3(blocks(RC, kPT)), dim3(kPT), 0, s, W, RC, (int)C, (int)R, a.m, a.M, Wt, WuT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // both factors from the U and V before this update
  if ((e = cholesky(a.V, (int)C, 1.0f, LV, a.info, sc, P, s)) != hipSuccess) return e;
  if ((e = cholesky(a.U, (int)R, 1.0f, LU, a.info + 1, sc, P, s)) != hipSuccess) return e;
  // Wt = Wc LV^-T (rows of Wc); WuT = Wc^T LU^-T = (LU^-1 Wc)^T (rows of Wc^T)
  if ((e = trsm_rows(Wt, R, (int)C, LV, P, s)) != hipSuccess) return e;
  if ((e = trsm_rows(WuT, C, (int)R, LU, P, s)) != hipSuccess) return e;
  // U <- m U + (1 - m) Wt Wt^T / C;  V <- m V + (1 - m) Wu^T Wu / R
  ReduceJob r{};
  r.beta = a.m;
  r.alpha = (1.0f - a.m) / (float)C;
  r.C = a.U;
  if ((e = gemm(GemmJob{R, R, C, 0, Wt, C, 1, Wt, C, 1, P}, r, s)) != hipSuccess) return e;
  r.alpha = (1.0f - a.m) / (float)R;
  r.C = a.V;
  if ((e = gemm(GemmJob{C, C, R, 0, WuT, R, 1, WuT, R, 1, P}, r, s)) != hipSuccess) return e;
  // U <- (U'' + U''^T) / 2 + eps I, V likewise, then s = trace(U) / R
  hipLaunchKernelGGL(k_trace_pair, dim3(1), dim3(kPT), 0, s, a.U, (int)R, a.V, (int)C, sc + 1);
  hipLaunchKernelGGL(k_sym_eps, dim3(blocks(max(R * R, C * C), kPT)), dim3(kPT), 0, s, a.U, (int)R, a.V, (int)C,
                     sc + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_trace, dim3(1), dim3(kPT), 0, s, a.U, (int)R, sc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_renorm, dim3(blocks(max(R * R, C * C), kPT)), dim3(kPT), 0, s, sc, R * R, C * C, a.U, a.V);
  return hipGetLastError();
}

size_t probe_sample_input_ws(int64_t B, int64_t K) {
  return al256((size_t)K * K * 4) + al256((size_t)B * K * 4) +
         al256((size_t)max(gemm_splits(K) * B * K, K * K) * 4) + 256;
}

hipError_t probe_sample_input(const ProbeSampleInputLaunch& a, hipStream_t s) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const int64_t K = a.K, B = a.B;
  float* L = reinterpret_cast<float*>(ws);
  float* Z = reinterpret_cast<float*>(ws + al256((size_t)K * K * 4));
  float* P = Z + al256((size_t)B * K * 4) / 4;
  float* sc = P + al256((size_t)max(gemm_splits(K) * B * K, K * K) * 4) / 4;
  // L L^T = S / (n - 1) + eps I
  hipError_t e = cholesky(a.S, (int)K, (float)(1.0 / (double)(a.n - 1)), L, a.info, sc, P, s);
  if (e != hipSuccess) return e;
  if ((e = normals(Z, B * K, a.seed, s)) != hipSuccess) return e;
  // T' = 1 mu^T + Z L^T, bf16
  ReduceJob r{};
  r.alpha = 1.0f;
  r.row = a.mu;
  r.Cb = static_cast<uint16_t*>(a.out);
  return gemm(GemmJob{B, K, K, 0, Z, K, 1, L, K, 1, P}, r, s);
}

size_t probe_sample_weight_ws(int64_t R, int64_t C) {
  return al256((size_t)R * R * 4) + al256((size_t)C * C * 4) + 2 * al256((size_t)R * C * 4) +
         al256((size_t)max(max(gemm_splits(C), gemm_splits(R)) * R * C, max(R * R, C * C)) * 4) + 256;
}

hipError_t probe_sample_weight(const ProbeSampleWeightLaunch& a, hipStream_t s) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const int64_t R = a.R, C = a.C;
  float* LU = reinterpret_cast<float*>(ws);
  float* LV = reinterpret_cast<float*>(ws + al256((size_t)R * R * 4));
  float* Z = LV + al256((size_t)C * C * 4) / 4;
  float* Y = Z + al256((size_t)R * C * 4) / 4;
  float* P = Y + al256((size_t)R * C * 4) / 4;
  float* sc = P + al256((size_t)max(max(gemm_splits(C), gemm_splits(R)) * R * C, max(R * R, C * C)) * 4) / 4;
  hipError_t e;
  if ((e = cholesky(a.U, (int)R, 1.0f, LU, a.info, sc, P, s)) != hipSuccess) return e;
  if ((e = cholesky(a.V, (int)C, 1.0f, LV, a.info + 1, sc, P, s)) != hipSuccess) return e;
  if ((e = normals(Z, R * C, a.seed, s)) != hipSuccess) return e;
  // Y = Z LV^T, then W' = M + LU Y (bf16)
  ReduceJob r{};
  r.alpha = 1.0f;
  r.C = Y;
  if ((e = gemm(GemmJob{R, C, C, 0, Z, C, 1, LV, C, 1, P}, r, s)) != hipSuccess) return e;
  ReduceJob r2{};
  r2.alpha = 1.0f;
  r2.mat = a.M;
  r2.Cb = static_cast<uint16_t*>(a.out);
  return gemm(GemmJob{R, C, R, 0, LU, R, 1, Y, 1, C, P}, r2, s);
}

}  // namespace loka
