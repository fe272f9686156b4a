// Standalone amax -> scale -> saturating RNE cast (loka_quant_fp8) on gfx950.
//
// Source: LoKA section II-C (quantization is a first-order cost of an FP8
// linear) and section III-C (tensorwise / rowwise / blockwise recipes); GEM
// "Low Precision Flash Attention" (MX block scales along K, E8M0 from a
// max-abs reduction by bit manipulation) and "Mixed Ultra-Low-Precision
// Training" (weights quantized once, separately from the activations).
//
// Pass 1 (amax):  tensor -> per-block partial maxima; row -> one wavefront
//                 per row; column -> per row-chunk partial maxima.
// Pass 2 (cast):  64 x 64 tiles, 256 threads, each thread 16 consecutive
//                 elements of one row; the group multipliers come from pass 1
//                 (MX blocks are reduced inside the tile).  Transposed output
//                 goes through LDS so both the loads and the stores are
//                 coalesced.
#include "common.hpp"
#include "launch.hpp"

namespace loka {
namespace {

constexpr int kTile = 64;

template <int DT>
__device__ __forceinline__ void load16(const void* base, int64_t off, bool ok, float v[16]) {
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    return;
  }
  if (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
}

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float v[8]) {
  if (DT == 0) {
    uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ---- pass 1 ---------------------------------------------------------------

// Partial max |x| of the whole array: block b covers 8-element units
// b, b + gridDim.x, ... (unit u = row u / c8, columns 8 * (u % c8) ...).
template <int DT>
__global__ __launch_bounds__(256) void k_amax_tensor(const void* src, int64_t rows, int64_t cols, int64_t ld,
                                                     float* partials) {
  __shared__ float red[4];
  const int64_t c8 = cols / 8;
  const int64_t units = rows * c8;
  float m = 0.0f;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    int64_t r = u / c8, c = (u - r * c8) * 8;
    float v[8];
    load8<DT>(src, r * ld + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One wavefront per row: amax[r] = max_c |x[r, c]|.
template <int DT>
__global__ __launch_bounds__(256) void k_amax_row(const void* src, int64_t rows, int64_t cols, int64_t ld,
                                                  float* amax) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float m = 0.0f;
  for (int64_t c = (int64_t)lane * 8; c < cols; c += 512) {
    float v[8];
    load8<DT>(src, r * ld + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = wave_max(m);
  if (lane == 0) amax[r] = m;
}

// partials[chunk][c] = max over rows [chunk * rpc, (chunk + 1) * rpc) of |x[r, c]|.
// Block: 4 wavefronts x 64 lanes x 8 columns = 512 columns; the wavefronts
// take every 4th row of the chunk, 4 rows in flight each, and combine in LDS.
// Grid (ceil(cols/512), nchunks).
template <int DT>
__global__ __launch_bounds__(256) void k_amax_col(const void* src, int64_t rows, int64_t cols, int64_t ld,
                                                  int64_t rpc, float* partials) {
  __shared__ float red[4][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rpc;
  const int64_t r1 = r0 + rpc < rows ? r0 + rpc : rows;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < cols) {
    int64_t r = r0 + wave;
    for (; r + 12 < r1; r += 16) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<DT>(src, (r + 4 * u) * ld + c, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[u][i]));
    }
    for (; r < r1; r += 4) {
      float v[8];
      load8<DT>(src, r * ld + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
  __syncthreads();
  for (int u = threadIdx.x; u < 512; u += 256) {
    const int64_t cc = (int64_t)blockIdx.x * 512 + u;
    if (cc < cols)
      partials[(int64_t)blockIdx.y * cols + cc] = fmaxf(fmaxf(red[0][u], red[1][u]), fmaxf(red[2][u], red[3][u]));
  }
}

// Column scales from the row-chunk partial maxima, once per column; writes
// the stored scale s, the multiplier r (for the cast) and optionally amax.
// A block of 256 threads takes 4 columns: thread (part, cl) = (t / 4, t % 4)
// reads partial rows part, part + 64, ... of column 4 blk + cl with all its
// loads in flight at once (one memory round trip for np <= 256), then the
// 64 parts meet by lane shuffles within each wavefront and through LDS
// across the four.  The max is order-free: the result does not depend on
// the grouping.
template <int FMT>
__device__ __forceinline__ void col_scales_body(int64_t blk, const float* partials, int64_t np, int64_t cols,
                                                float* scales, float* mult, float* amax_out) {
  __shared__ float red[4][4];
  const int cl = threadIdx.x & 3, part = threadIdx.x >> 2;
  const int64_t c = blk * 4 + cl;
  float m = 0.0f;
  if (c < cols) {
    int64_t k = part;
    for (; k + 192 < np; k += 256) {
      const float a = partials[k * cols + c], b = partials[(k + 64) * cols + c];
      const float d = partials[(k + 128) * cols + c], e = partials[(k + 192) * cols + c];
      m = fmaxf(m, fmaxf(fmaxf(a, b), fmaxf(d, e)));
    }
    for (; k < np; k += 64) m = fmaxf(m, partials[k * cols + c]);
  }
  m = fmaxf(m, __shfl_xor(m, 4, 64));
  m = fmaxf(m, __shfl_xor(m, 8, 64));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < 4) red[wave][cl] = m;
  __syncthreads();
  if (threadIdx.x < 4 && c < cols) {
    m = fmaxf(fmaxf(red[0][cl], red[1][cl]), fmaxf(red[2][cl], red[3][cl]));
    const ScalePair sp = scales_from_amax<FMT>(m);
    scales[c] = sp.s;
    mult[c] = sp.r;
    if (amax_out) amax_out[c] = m;
  }
}
template <int FMT>
__global__ __launch_bounds__(256) void k_col_scales(const float* partials, int64_t np, int64_t cols, float* scales,
                                                    float* mult, float* amax_out) {
  col_scales_body<FMT>(blockIdx.x, partials, np, cols, scales, mult, amax_out);
}

// ---- pass 2 ---------------------------------------------------------------

struct CastParams {
  const void* src;
  int64_t rows, cols, ld;
  uint8_t* codes;
  void* scales;
  float* amax_out;
  const float* amax_in;  // tensor: partials[np]; row: amax[rows]; col: multipliers[cols]
  int64_t np;
};

// Tile (blockIdx.y, blockIdx.x) covers rows [64 by, +64), cols [64 bx, +64).
// Thread t: tile row t / 4, tile columns 16 (t % 4) .. +16.
// mult_local (COL only, optional): the tile's 64 column multipliers in LDS,
// in place of p.amax_in
template <int DT, int FMT, int MODE, int TRANS>
__device__ __forceinline__ void cast_tile_body(const CastParams& p, int64_t bx, int64_t by,
                                               const float* mult_local = nullptr) {
  __shared__ float r_col[kTile];             // COL: multiplier per tile column
  __shared__ float red[4];
  __shared__ float colmax[kTile][kTile + 1];  // MX32_COL: |x| staging
  __shared__ int e8_col[2][kTile];            // MX32_COL: E8M0 per (row block, column)
  __shared__ float sq_max[4][2];              // MX32_SQ: per wavefront, per 32-column half
  __shared__ uint8_t tcodes[kTile][kTile + 4];  // transposed output staging

  const int t = threadIdx.x;
  const int tr = t >> 2, tc = (t & 3) * 16;
  const int64_t row = by * kTile + tr;
  const int64_t col0 = bx * kTile + tc;
  const bool ok = row < p.rows && col0 < p.cols;

  float v[16];
  load16<DT>(p.src, row * p.ld + col0, ok, v);

  float mult[16];
  if (MODE == 0) {  // tensor: reduce the partial maxima
    float m = 0.0f;
    for (int64_t i = t; i < p.np; i += 256) m = fmaxf(m, p.amax_in[i]);
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    ScalePair sp = scales_from_amax<FMT>(m);
    if (bx == 0 && by == 0 && t == 0) {
      static_cast<float*>(p.scales)[0] = sp.s;
      if (p.amax_out) p.amax_out[0] = m;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = sp.r;
  } else if (MODE == 1) {  // row
    float a = row < p.rows ? p.amax_in[row] : 0.0f;
    ScalePair sp = scales_from_amax<FMT>(a);
    if (bx == 0 && (t & 3) == 0 && row < p.rows) {
      static_cast<float*>(p.scales)[row] = sp.s;
      if (p.amax_out) p.amax_out[row] = a;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = sp.r;
  } else if (MODE == 2) {  // column: the multipliers from k_col_scales
    if (t < kTile) {
      const int64_t c = bx * kTile + t;
      r_col[t] = c < p.cols ? (mult_local != nullptr ? mult_local[t] : p.amax_in[c]) : 1.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = r_col[tc + i];
  } else if (MODE == 3) {  // MX32 along rows: this thread's 16 columns are half a block
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));  // partner thread holds the other half
    int e8 = e8m0_from_amax<FMT>(m);
    float mu = e8m0_inv_multiplier(e8);
    if ((t & 1) == 0 && ok) {
      int64_t nb = p.cols / 32;
      static_cast<uint8_t*>(p.scales)[row * nb + col0 / 32] = (uint8_t)e8;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = mu;
  } else if (MODE == 5) {  // MX32 square: the tile's 2 x 2 blocks of 32 x 32
    // wavefront w holds tile rows 16w .. +16 (block row w / 2); lane bit 1
    // selects the 32-column half (block column); reduce over the other bits
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    m = fmaxf(m, __shfl_xor(m, 8, 64));
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const int w = t >> 6, h = (t >> 1) & 1;
    if ((t & 63) < 4 && (t & 1) == 0) sq_max[w][h] = m;  // lanes 0 and 2
    __syncthreads();
    const int b = w >> 1;
    m = fmaxf(sq_max[2 * b][h], sq_max[2 * b + 1][h]);
    const int e8 = e8m0_from_amax<FMT>(m);
    const float mu = e8m0_inv_multiplier(e8);
    const int64_t grb = by * 2 + b, gcb = bx * 2 + h;
    if ((t & 127) < 4 && (t & 1) == 0 && grb * 32 < p.rows && gcb * 32 < p.cols)
      static_cast<uint8_t*>(p.scales)[grb * (p.cols / 32) + gcb] = (uint8_t)e8;
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = mu;
  } else {  // MX32 down columns: 32-row blocks of each column, via LDS
#pragma unroll
    for (int i = 0; i < 16; ++i) colmax[tr][tc + i] = fabsf(v[i]);
    __syncthreads();
    if (t < 2 * kTile) {
      int c = t & (kTile - 1), b = t >> 6;
      float m = 0.0f;
      for (int i = 0; i < 32; ++i) m = fmaxf(m, colmax[32 * b + i][c]);
      int e8 = e8m0_from_amax<FMT>(m);
      e8_col[b][c] = e8;
      int64_t gc = bx * kTile + c;
      int64_t grb = by * 2 + b;  // global row block
      if (gc < p.cols && grb * 32 < p.rows) static_cast<uint8_t*>(p.scales)[gc * (p.rows / 32) + grb] = (uint8_t)e8;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) mult[i] = e8m0_inv_multiplier(e8_col[tr >> 5][tc + i]);
  }

  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = cvt4<FMT>(v[4 * q] * mult[4 * q], v[4 * q + 1] * mult[4 * q + 1], v[4 * q + 2] * mult[4 * q + 2],
                     v[4 * q + 3] * mult[4 * q + 3]);

  if (TRANS == 0) {
    if (ok) *reinterpret_cast<uint4*>(p.codes + row * p.cols + col0) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if (TRANS == 3) {
    // fragment-interleaved [rows][cols padded to 128], not transposed: the
    // grid covers the padding, whose columns load as zeros (zero codes)
    const int64_t nchc = (p.cols + 127) / 128;
    if (row < p.rows && col0 < nchc * 128)
      *reinterpret_cast<uint4*>(p.codes + ilv_offset(row, col0, nchc)) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int b = 0; b < 4; ++b) tcodes[tr][tc + 4 * q + b] = (uint8_t)(w[q] >> (8 * b));
    __syncthreads();
    // thread t: tile column t / 4, tile rows 16 (t % 4) .. +16
    const int oc = t >> 2, orow = (t & 3) * 16;
    const int64_t gc = bx * kTile + oc;
    const int64_t gr = by * kTile + orow;
    // TRANS 2: fragment-interleaved [cols][rows padded to 128]; the rows past
    // `rows` (up to the padding) are written as zero codes
    const int64_t nch = (p.rows + 127) / 128;
    if (gc < p.cols && gr < (TRANS == 2 ? nch * 128 : p.rows)) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)tcodes[orow + 4 * q][oc] | ((uint32_t)tcodes[orow + 4 * q + 1][oc] << 8) |
               ((uint32_t)tcodes[orow + 4 * q + 2][oc] << 16) | ((uint32_t)tcodes[orow + 4 * q + 3][oc] << 24);
      uint8_t* dst = TRANS == 2 ? p.codes + ilv_offset(gc, gr, nch) : p.codes + gc * p.rows + gr;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}
template <int DT, int FMT, int MODE, int TRANS>
__global__ __launch_bounds__(256) void k_cast_tile(CastParams p) {
  cast_tile_body<DT, FMT, MODE, TRANS>(p, blockIdx.x, blockIdx.y);
}

// Column scaling of a short bf16 array (rows <= kStripRows) in one launch
// instead of three: workgroup (x, y) casts tile (x, y) of 64 x 64 (columns
// covered as the two-pass path covers them, TRANS 3 padding them to 128),
// after taking the column maxima of its whole 64-column strip over all rows
// itself (the strip's workgroups read the same 64 KiB, from L2 after the
// first), so no workgroup waits for another.  The workgroups of tile row 0
// write the scales.  A max does not depend on the order of its operands, and
// the tile body is the two-pass path's, so scales and codes are the same bit
// for bit.  Thread t: columns 8 (t % 8) .. +8 of the strip, rows t / 8,
// t / 8 + 32, ...; eight rows' loads are issued before their maxima.
constexpr int64_t kStripRows = 1024;
template <int FMT, int TRANS>
__global__ __launch_bounds__(256) void k_quant_col_strip(CastParams p) {
  __shared__ float cm[32][kTile + 1];
  __shared__ float mult[kTile];
  const int t = threadIdx.x, c8 = t & 7, ph = t >> 3;
  const int64_t col = (int64_t)blockIdx.x * kTile + c8 * 8;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col < p.cols) {
    int64_t r = ph;
    for (; r + 7 * 32 < p.rows; r += 8 * 32) {
      float v[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) load8<0>(p.src, (r + 32 * u) * p.ld + col, v[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[u][i]));
    }
    for (; r < p.rows; r += 32) {
      float v[8];
      load8<0>(p.src, r * p.ld + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) cm[ph][c8 * 8 + i] = m[i];
  __syncthreads();
  if (t < kTile) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) a = fmaxf(a, cm[j][t]);
    const int64_t c = (int64_t)blockIdx.x * kTile + t;
    const ScalePair sp = scales_from_amax<FMT>(a);
    mult[t] = sp.r;
    if (blockIdx.y == 0 && c < p.cols) {
      static_cast<float*>(p.scales)[c] = sp.s;
      if (p.amax_out) p.amax_out[c] = a;
    }
  }
  __syncthreads();
  cast_tile_body<0, FMT, 2, TRANS>(p, blockIdx.x, blockIdx.y, mult);
}

// Two column-scaled casts to the fragment-interleaved transposed layout in
// one launch (blocks [0, na) the first, the rest the second; each with its
// own 2-D tile grid of width gxa / gxb).
template <int DTA, int FMTA, int DTB, int FMTB>
__global__ __launch_bounds__(256) void k_cast_col_pair(CastParams a, CastParams b, int64_t na, int64_t gxa,
                                                       int64_t gxb) {
  const int64_t blk = blockIdx.x;
  if (blk < na) cast_tile_body<DTA, FMTA, 2, 2>(a, blk % gxa, blk / gxa);
  else cast_tile_body<DTB, FMTB, 2, 2>(b, (blk - na) % gxb, (blk - na) / gxb);
}
// Two sets of column scales in one launch (blocks [0, na) the first).
template <int FMTA, int FMTB>
__global__ __launch_bounds__(256) void k_col_scales_pair(const float* pa, int64_t npa, int64_t ca, float* sa,
                                                         float* ma, const float* pb, int64_t npb, int64_t cb,
                                                         float* sb, float* mb, int64_t na) {
  const int64_t blk = blockIdx.x;
  if (blk < na) col_scales_body<FMTA>(blk, pa, npa, ca, sa, ma, nullptr);
  else col_scales_body<FMTB>(blk - na, pb, npb, cb, sb, mb, nullptr);
}

// trans: 0 plain, 1 transposed row-major, 2 transposed fragment-interleaved
// (internal; the row count is covered up to the next multiple of 128),
// 3 fragment-interleaved without transposing (the column count is covered
// up to the next multiple of 128)
template <int DT, int FMT, int MODE>
void launch_cast(const CastParams& cp, int trans, hipStream_t s) {
  const int64_t rows = trans == 2 ? (cp.rows + 127) / 128 * 128 : cp.rows;
  const int64_t cols = trans == 3 ? (cp.cols + 127) / 128 * 128 : cp.cols;
  dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
  if (trans == 3)
    hipLaunchKernelGGL((k_cast_tile<DT, FMT, MODE, 3>), grid, dim3(256), 0, s, cp);
  else if (trans == 2)
    hipLaunchKernelGGL((k_cast_tile<DT, FMT, MODE, 2>), grid, dim3(256), 0, s, cp);
  else if (trans == 1)
    hipLaunchKernelGGL((k_cast_tile<DT, FMT, MODE, 1>), grid, dim3(256), 0, s, cp);
  else
    hipLaunchKernelGGL((k_cast_tile<DT, FMT, MODE, 0>), grid, dim3(256), 0, s, cp);
}

template <int DT, int FMT>
void dispatch_cast(const CastParams& cp, int mode, int trans, hipStream_t s) {
  switch (mode) {
    case 0: launch_cast<DT, FMT, 0>(cp, trans, s); break;
    case 1: launch_cast<DT, FMT, 1>(cp, trans, s); break;
    case 2: launch_cast<DT, FMT, 2>(cp, trans, s); break;
    case 3: launch_cast<DT, FMT, 3>(cp, trans, s); break;
    case 4: launch_cast<DT, FMT, 4>(cp, trans, s); break;
    default: launch_cast<DT, FMT, 5>(cp, trans, s); break;
  }
}

}  // namespace

QuantPlan quant_plan(int64_t rows, int64_t cols, int mode) {
  QuantPlan q{};
  if (mode == 0) {
    int64_t units = rows * (cols / 8);
    int64_t nb = (units + 256 * 16 - 1) / (256 * 16);
    q.np = nb < 1 ? 1 : (nb > 1024 ? 1024 : nb);
    q.ws_floats = q.np;
  } else if (mode == 1) {
    q.np = rows;
    q.ws_floats = rows;
  } else if (mode == 2) {
    int64_t rpc = 64;
    int64_t nch = (rows + rpc - 1) / rpc;
    if (nch > 256) {  // keep the per-column reduction in pass 2 short
      nch = 256;
      rpc = (rows + nch - 1) / nch;
      nch = (rows + rpc - 1) / rpc;
    }
    if (nch < 1) nch = 1;
    q.np = nch;
    q.rpc = rpc;
    q.ws_floats = nch * cols + cols;  // partials, then the column multipliers
  }
  return q;
}

hipError_t launch_quant(const QuantLaunch& a, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  QuantPlan q = quant_plan(a.rows, a.cols, a.mode);
  float* ws = static_cast<float*>(a.workspace);
  CastParams cp{a.src, a.rows, a.cols, a.ld, a.codes, a.scales, a.amax_out, ws, q.np};
  const bool f32 = a.src_dtype == 1;
  if (a.mode == 0) {
    if (f32) hipLaunchKernelGGL(k_amax_tensor<1>, dim3((unsigned)q.np), dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, ws);
    else hipLaunchKernelGGL(k_amax_tensor<0>, dim3((unsigned)q.np), dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, ws);
  } else if (a.mode == 1) {
    dim3 g((unsigned)((a.rows + 3) / 4));
    if (f32) hipLaunchKernelGGL(k_amax_row<1>, g, dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, ws);
    else hipLaunchKernelGGL(k_amax_row<0>, g, dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, ws);
  } else if (a.mode == 2 && !f32 && a.rows <= kStripRows) {
    // one launch: every 64 x 64 tile's workgroup takes its strip's maxima
    const int tr = a.transpose_out;
    const int64_t rows_cov = tr == 2 ? (a.rows + 127) / 128 * 128 : a.rows;
    const int64_t cols_cov = tr == 3 ? (a.cols + 127) / 128 * 128 : a.cols;
    const dim3 g((unsigned)((cols_cov + kTile - 1) / kTile), (unsigned)((rows_cov + kTile - 1) / kTile));
    if (a.fmt == 0) {
      if (tr == 3) hipLaunchKernelGGL((k_quant_col_strip<0, 3>), g, dim3(256), 0, s, cp);
      else if (tr == 2) hipLaunchKernelGGL((k_quant_col_strip<0, 2>), g, dim3(256), 0, s, cp);
      else if (tr == 1) hipLaunchKernelGGL((k_quant_col_strip<0, 1>), g, dim3(256), 0, s, cp);
      else hipLaunchKernelGGL((k_quant_col_strip<0, 0>), g, dim3(256), 0, s, cp);
    } else {
      if (tr == 3) hipLaunchKernelGGL((k_quant_col_strip<1, 3>), g, dim3(256), 0, s, cp);
      else if (tr == 2) hipLaunchKernelGGL((k_quant_col_strip<1, 2>), g, dim3(256), 0, s, cp);
      else if (tr == 1) hipLaunchKernelGGL((k_quant_col_strip<1, 1>), g, dim3(256), 0, s, cp);
      else hipLaunchKernelGGL((k_quant_col_strip<1, 0>), g, dim3(256), 0, s, cp);
    }
    return hipGetLastError();
  } else if (a.mode == 2) {
    dim3 g((unsigned)((a.cols + 511) / 512), (unsigned)q.np);
    if (f32) hipLaunchKernelGGL(k_amax_col<1>, g, dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, q.rpc, ws);
    else hipLaunchKernelGGL(k_amax_col<0>, g, dim3(256), 0, s, a.src, a.rows, a.cols, a.ld, q.rpc, ws);
    float* mult = ws + q.np * a.cols;
    dim3 gs((unsigned)((a.cols + 3) / 4));
    if (a.fmt == 0)
      hipLaunchKernelGGL(k_col_scales<0>, gs, dim3(256), 0, s, ws, q.np, a.cols, static_cast<float*>(a.scales), mult,
                         a.amax_out);
    else
      hipLaunchKernelGGL(k_col_scales<1>, gs, dim3(256), 0, s, ws, q.np, a.cols, static_cast<float*>(a.scales), mult,
                         a.amax_out);
    cp.amax_in = mult;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f32) {
    if (a.fmt == 0) dispatch_cast<1, 0>(cp, a.mode, a.transpose_out, s);
    else dispatch_cast<1, 1>(cp, a.mode, a.transpose_out, s);
  } else {
    if (a.fmt == 0) dispatch_cast<0, 0>(cp, a.mode, a.transpose_out, s);
    else dispatch_cast<0, 1>(cp, a.mode, a.transpose_out, s);
  }
  return hipGetLastError();
}

}  // namespace loka

namespace loka {

// Tensor-mode amax partials of a bf16 array (used by the tensor-recipe forward).
hipError_t launch_amax_tensor_partials(const void* src, int64_t rows, int64_t cols, int64_t ld, float* partials,
                                       hipStream_t s) {
  QuantPlan q = quant_plan(rows, cols, 0);
  hipLaunchKernelGGL(k_amax_tensor<0>, dim3((unsigned)q.np), dim3(256), 0, s, src, rows, cols, ld, partials);
  return hipGetLastError();
}

// Column maxima of a [rows, cols] array as row-chunk partials (np x cols
// floats at `partials`, np returned); the first pass of the column recipe.
hipError_t launch_col_amax_partials(const void* src, int src_dtype, int64_t rows, int64_t cols, int64_t ld,
                                   float* partials, int64_t* np, hipStream_t s) {
  const QuantPlan q = quant_plan(rows, cols, 2);
  *np = q.np;
  dim3 g((unsigned)((cols + 511) / 512), (unsigned)q.np);
  if (src_dtype == 1) hipLaunchKernelGGL(k_amax_col<1>, g, dim3(256), 0, s, src, rows, cols, ld, q.rpc, partials);
  else hipLaunchKernelGGL(k_amax_col<0>, g, dim3(256), 0, s, src, rows, cols, ld, q.rpc, partials);
  return hipGetLastError();
}

// Two column quantizations from their partial maxima: both sets of scales
// in one launch, then both casts (to the fragment-interleaved transposed
// layout, rows padded to 128) in one launch.  The backward's pair: X (bf16,
// e4m3) and dZ (fp32, e5m2).
hipError_t launch_col_quant_pair(const ColQuantJob& a, const ColQuantJob& b, hipStream_t s) {
  if (!(a.src_dtype == 0 && a.fmt == 0 && b.src_dtype == 1 && b.fmt == 1)) return hipErrorInvalidValue;
  const int64_t sa = (a.cols + 3) / 4, sb = (b.cols + 3) / 4;
  hipLaunchKernelGGL((k_col_scales_pair<0, 1>), dim3((unsigned)(sa + sb)), dim3(256), 0, s, a.partials, a.np, a.cols,
                     a.scales, a.mult, b.partials, b.np, b.cols, b.scales, b.mult, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const CastParams ca{a.src, a.rows, a.cols, a.ld, a.codes_t, a.scales, nullptr, a.mult, a.np};
  const CastParams cb{b.src, b.rows, b.cols, b.ld, b.codes_t, b.scales, nullptr, b.mult, b.np};
  const int64_t gxa = (a.cols + kTile - 1) / kTile, gya = ((a.rows + 127) / 128 * 128 + kTile - 1) / kTile;
  const int64_t gxb = (b.cols + kTile - 1) / kTile, gyb = ((b.rows + 127) / 128 * 128 + kTile - 1) / kTile;
  hipLaunchKernelGGL((k_cast_col_pair<0, 0, 1, 1>), dim3((unsigned)(gxa * gya + gxb * gyb)), dim3(256), 0, s, ca, cb,
                     gxa * gya, gxa, gxb);
  return hipGetLastError();
}

}  // namespace loka
