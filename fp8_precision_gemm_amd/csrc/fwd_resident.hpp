// The weight-resident fused forward: one persistent workgroup per compute
// unit holds the whole FP8 weight in registers and streams row tiles of X
// through it.
//
// Source: LoKA section III-B2 (Block-wise Normalization, Case 1): with a
// large batch and a small output dimension a whole output row lives in one
// block of the GEMM, so the LayerNorm runs in the GEMM epilogue while the
// tile is still on chip; section III-B (the GEMM output is dequantized and
// normalized in high precision); section III-B1 (No Bias).  GEM "Mixed
// Ultra-Low-Precision Training": the activation cast is fused into the
// neighbouring kernel instead of taking an extra pass over HBM; "Low
// Precision Flash Attention": MX block scales along K.
//
// Shape of the work.  In the recommendation shapes (M >> K, N <= 512) the
// weight is small (K*N <= 256 KiB of e4m3 codes) and X and Y dominate the
// bytes.  A workgroup of 8 wavefronts splits the N columns into 8 slices of
// 16*NT columns; wavefront w keeps the W^T rows of its slice for all of K in
// VGPRs (NT x KC MFMA A-fragments, at most 128 registers per lane), loaded
// once per workgroup straight into the fragment registers: W^T is stored in
// the fragment-interleaved layout (ilv_offset: per 16 columns and 128-deep K
// chunk one 2 KiB block in exactly the order the 64 lanes hold it), so each
// fragment is two 1 KiB coalesced loads with no rearrangement on chip.  The
// workgroup then walks a contiguous range of 16-row tiles.  Per tile:
//   * X rows are requested D tiles ahead into registers: each wavefront owns
//     2 rows, 32 lanes per row, 16 B per lane per 256 columns, so HBM reads
//     stay in flight across the loop;
//   * each wavefront quantizes its 2 rows of the next tile into one of two
//     LDS code buffers: the two rows' max-abs reductions (DPP within rows of
//     16 lanes, a permlane swap across them) and their scale divisions run
//     side by side in the two halves of the wavefront;
//   * v_mfma_scale_f32_16x16x128_f8f6f4 multiplies the resident W^T
//     fragments (A) by the tile's codes read from LDS (B);
//   * epilogue: dequant + bias in registers, each wavefront's row sum and
//     centred sum of squares over its slice, one LDS exchange and barrier,
//     the slices' statistics combined exactly (sum of the slices' centred
//     sums plus the between-slice term, Chan, Golub and LeVeque's pairwise
//     update), then gamma/beta and bf16 stores straight from registers.
// One barrier per tile; X is read once and Y written once.
//
// Column order.  MFMA tile t of wavefront w covers the 16 output columns
// 16(w NT + t) .. +16 in order, so its A-row i is column c0 + 16t + i and
// lane (r, g) ends up holding columns c0 + 16t + 4g .. +4 of row r: 8-byte Y
// stores and float4 reads of the per-column vectors.
//
// Cast without a clamp (tensor and row recipes).  With r = RN32(448/amax)
// every |x*r| is at most 448*(1 + 2^-23); the hardware convert rounds
// everything up to the 448/480 midpoint (464) to the 448 code, so the
// saturation the format definition asks for is already what it produces.
// MX scaling can reach 512*2^e before the cast and keeps the clamp.
#pragma once

#include <utility>

#include "common.hpp"
#include "fwd_block.hpp"
#include "launch.hpp"

namespace loka {
namespace fwd {

constexpr int kResRows = 16;  // rows per tile
// float2 slots per row of the statistics exchange: the 8 wavefronts' (sum,
// centred sum of squares) plus 2 of padding, so that the 16 rows of a tile
// (80 bytes apart) fall on distinct LDS banks when a wavefront writes or
// reads them all at once
constexpr int kRedRow = 10;

// Shapes: NT column tiles per wavefront (N <= 128*NT) and KC resident 128-deep
// K chunks (K <= 128*KC); NT*KC fragments of 8 VGPRs stay within 128
// registers.  Instantiated chunk counts: 2, 4 and the per-NT maximum (8, 8,
// 5, 4), so a small K keeps a small weight footprint.
template <int NT, int KC>
struct Res {
  static constexpr int KQ = (KC * 128 + 255) / 256;           // 16-byte X loads per lane (32 lanes per row)
  // software pipeline (two accumulator sets: the next tile's GEMM overlaps
  // the previous tile's normalization) where the registers allow it; the
  // largest weights run the steps one after another with one slot of X in
  // flight
  static constexpr bool PIPE = NT * KC <= 12 || (NT == 4 && KC == 4);
  // tiles of X requested ahead: small weights run short steps, so they
  // keep four tiles in flight (the registers are there); a tile of one
  // 16-byte load per lane (K <= 256: 4-8 KiB per tile) keeps eight
  static constexpr int D = !PIPE ? 1 : (KQ == 1 ? 8 : (NT * KC <= 8 ? 4 : 2));
  static constexpr int LDX = KC * 128 + 16;                    // LDS code row stride (bytes)
  static constexpr int KP = (KC + 3) / 4;                     // E8M0 words per lane group
  static constexpr int XE = 16 * KP;                           // E8M0 bytes per LDS row ([g][KP words])
};

__host__ __device__ constexpr int res_nt(int N) { return (N + 127) / 128; }
__host__ __device__ constexpr int res_kc_max(int nt) { return nt <= 2 ? 8 : (nt == 3 ? 5 : 4); }
// the instantiated chunk count for K: 2, 4, else the maximum
__host__ __device__ constexpr int res_kc(int nt, int K) {
  return (K + 127) / 128 <= 2 ? 2 : ((K + 127) / 128 <= 4 ? 4 : res_kc_max(nt));
}
// Does (K, N) fit the weight-resident kernel?
__host__ __device__ constexpr bool res_fits(int K, int N) {
  return N >= 16 && N <= 512 && N % 16 == 0 && K >= 16 && K % 16 == 0 && (K + 127) / 128 <= res_kc_max(res_nt(N));
}
// FULL shape (no partial-shape guards): whole column tiles per wavefront,
// whole 256-column pieces per lane, whole 16-row tiles
__host__ __device__ constexpr bool res_full(int64_t M, int N, int K, int nt, int kc) {
  return N == 128 * nt && K == 256 * ((kc * 128 + 255) / 256) && M % 16 == 0;
}
// the instantiated (NT, KC) pairs, numbered 0..10
constexpr int kResShapes = 11;
__host__ __device__ constexpr int res_shape(int nt, int kc) {
  return nt == 1 ? (kc == 2 ? 0 : kc == 4 ? 1 : 2)
       : nt == 2 ? (kc == 2 ? 3 : kc == 4 ? 4 : 5)
       : nt == 3 ? (kc == 2 ? 6 : kc == 4 ? 7 : 8)
                 : (kc == 2 ? 9 : 10);
}

// LDS carve-up (bytes, every part 16-byte aligned; nb = 2, or 4 for B2):
//   codes [nb][16][LDX] u8 | xe8 [nb][16][XE] u8 | rs [nb][16] f32 |
//   red [nb][16][kRedRow] float2 | cvec [4][N] f32 (s_w, bias, gamma, beta) |
//   wmx [3][8] f32 | ystg [8][16][32*NT + 16] (each wavefront's Y block) |
//   yprev [8][16][32*NT + 16] (the previous tile's Y block, for the Y output
//   quantized in 32 x 32 blocks)
struct ResLds {
  int codes, xe8, rs, red, cvec, wmx, ystg, yprev, total;
};
__host__ __device__ constexpr int res_yst(int nt) { return 32 * nt + 16; }  // Y staging row stride (bytes)
// nb: tiles in flight through the code, scale and statistics buffers (two,
// or four when a step takes two tiles)
__host__ __device__ inline ResLds res_lds(int nt, int kc, int N, int nb = 2) {
  const int ldx = kc * 128 + 16, xe = 16 * ((kc + 3) / 4);
  ResLds l;
  l.codes = 0;
  l.xe8 = l.codes + nb * kResRows * ldx;
  l.rs = l.xe8 + ((nb * kResRows * xe + 15) / 16) * 16;
  l.red = l.rs + nb * kResRows * 4;
  l.cvec = l.red + nb * kResRows * kRedRow * 8;
  l.wmx = l.cvec + 4 * N * 4;
  l.ystg = l.wmx + 32 * 4;
  l.yprev = l.ystg + kWaves * kResRows * res_yst(nt);
  l.total = l.yprev + kWaves * kResRows * res_yst(nt);
  return l;
}

// Staged variant (all of a workgroup's tiles at once, at most kXlTiles):
//   xraw [kXlTiles][16][2K] (the bf16 X rows, as loaded) | codes
//   [kXlTiles][16][LDX] | xe8 [kXlTiles][16][XE] | rs [kXlTiles][16] f32 |
//   red [kXlTiles][16][kRedRow] float2 | cvec [4][N] f32 | wmx [32] f32 |
//   ystg [8][16][32*NT + 16]
constexpr int kXlTiles = 4;
struct XlLds {
  int xraw, codes, xe8, rs, red, cvec, wmx, ystg, total;
};
__host__ __device__ inline XlLds xl_lds(int nt, int kc, int N, int K) {
  const int ldx = kc * 128 + 16, xe = 16 * ((kc + 3) / 4);
  XlLds l;
  l.xraw = 0;
  l.codes = l.xraw + kXlTiles * kResRows * 2 * K;
  l.xe8 = l.codes + kXlTiles * kResRows * ldx;
  l.rs = l.xe8 + ((kXlTiles * kResRows * xe + 15) / 16) * 16;
  l.red = l.rs + kXlTiles * kResRows * 4;
  l.cvec = l.red + kXlTiles * kResRows * kRedRow * 8;
  l.wmx = l.cvec + 4 * N * 4;
  l.ystg = l.wmx + 32 * 4;
  l.total = l.ystg + kWaves * kResRows * res_yst(nt);
  return l;
}

// Max over each 32-lane half of the wavefront, returned in every lane of
// that half: quads and rows of 16 by DPP, then the two rows of a half
// exchanged by v_permlane16_swap.  Non-negative values only.
__device__ __forceinline__ float half_max(float v) {
  v = quad_max(v);
  v = dpp_max<0x124>(v);  // row_ror:4
  v = dpp_max<0x128>(v);  // row_ror:8
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(max((uint32_t)s[0], (uint32_t)s[1]));  // non-negative: unsigned order
}
// Sum over the 4 lanes l, l^16, l^32, l^48 (the lanes holding one output
// row of a 16x16 MFMA tile), returned in all four.
__device__ __forceinline__ float sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum of n values as a balanced tree (pairs of neighbours first).
template <int n>
__device__ __forceinline__ float tree_sum(const float (&v)[n]) {
  if constexpr (n == 1) {
    return v[0];
  } else {
    constexpr int h = (n + 1) / 2;
    float a[h];
#pragma unroll
    for (int i = 0; i < h; ++i) a[i] = (2 * i + 1 < n) ? v[2 * i] + v[2 * i + 1] : v[2 * i];
    return tree_sum<h>(a);
  }
}

// 8 bf16 (one 16-byte piece) -> fp32
__device__ __forceinline__ void unpack8(const uint4& u, float v[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// Largest sign-cleared bf16 bit pattern of 8 finite bf16 values (= the bits of max |x|).
__device__ __forceinline__ uint32_t absmax_bits8(const uint4& u) {
  const u16x2 a = __builtin_bit_cast(u16x2, u.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, u.y & 0x7FFF7FFFu);
  const u16x2 c = __builtin_bit_cast(u16x2, u.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, u.w & 0x7FFF7FFFu);
  const u16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)mx.x, (uint32_t)mx.y);
}

// MX MFMA with both E8M0 operands taken from byte `sel` (0..3) of packed
// scale words (the instruction's op_sel byte select; sel is a constant
// after unrolling).
__device__ __forceinline__ v4f mfma_mx_sel(int sel, const v8i& a, const v8i& b, v4f c, uint32_t sa, uint32_t sb) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 3, (int)sa, 3, (int)sb);
  }
}

// OPT: the optional outputs (fp32 Z, mean/rstd, the X codes and scales) are
// requested; the variant without them carries none of their branches.
// FULL: N = 128*NT, K = 256*KQ and M a multiple of 16, so every wavefront
// owns NT whole column tiles, every lane a whole share of each row and every
// tile 16 real rows: no partial-shape guards.
// EPI: 0 = LayerNorm over the row (gamma, beta); 1 = BlockNorm over blocks
// of 256 columns (RMS, no affine parameters) followed by Hard Swish
// ([LoKA] section III-B2 Fig. 7d and III-B3).  With EPI 1 the block covers
// one column slab of 128*NT columns (a whole number of 256-blocks).
constexpr int kBlockNorm = 256;
// MODE: 0 tensor, 1 row, 3 MX32 along K (X quantized here), 4 MX32 square
// blocks (X given as e4m3 codes with E8M0 scales per 32 x 32 block; the
// weight's scales per 32 x 32 block of W[K][N]).
// XL: the staged run (run_xl): the workgroup's whole tile range (at most
// kXlTiles tiles, FULL shapes, LayerNorm) is loaded, quantized, multiplied
// and normalized as one batch.
template <int MODE, int NT, int KC, bool OPT, bool FULL, int EPI = 0, bool XL = false, bool B2 = false>
struct ResBlock {
  using R = Res<NT, KC>;
  static constexpr bool MX = MODE >= 3;  // E8M0 block scales inside the MFMA
  // B2 keeps four tiles (two pairs) of X in flight
  static constexpr int KQ = R::KQ, D = B2 && R::D > 4 ? 4 : R::D, LDX = R::LDX, XE = R::XE, KP = R::KP;
  static constexpr bool PIPE = R::PIPE;
  // sequential steps, guard-free shape, LayerNorm, no optional outputs: Y
  // leaves as whole rows after the next barrier (two staging buffers by tile
  // parity), so no 128-byte line is written in parts by two wavefronts
  static constexpr bool COOP = FULL && !OPT && !PIPE && EPI == 0 && !XL;
  // B2: two tiles per step (one barrier, one statistics exchange and one
  // round of latencies for both), for small weights whose steps are mostly
  // fixed latency; the pipelined LayerNorm path only
  static_assert(!B2 || (PIPE && EPI == 0 && !XL && D % 2 == 0), "B2 runs the pipelined LayerNorm steps");

  const FwdBlock& p;
  int64_t tb, te;  // tile range [tb, te)
  int K, N, ldy, kcv, kb, T16, nv, c0, tid, lane, wave, r, g, hrow, hl;
  uint8_t* codes;
  uint8_t* xe8;
  float* rs;
  float2* red;
  float* cvec;
  float* wmx;
  uint8_t* ystg;  // this wavefront's Y staging block [16][res_yst(NT)]
  uint8_t* yprev;  // its copy of the previous (even) tile's block, square-block Y output
  float sq_prev[NT / 2 > 0 ? NT / 2 : 1];  // that tile's 16 x 32 maxima per 32-column block
  float bw, bb;   // bound on |z|: row factor (tensor/row: 448^2 K max s_w; MX: 448^2 K 2^(ew_max-127)), max |bias|
  float inv_nw;   // 1 / (columns of this wavefront's slice)

  v8i wf[NT][KC];
  uint32_t wsc[NT][KP];
  uint4 xr[D][KQ];
  uint32_t xq8[D][KQ];  // MODE 4: the E8M0 byte of each loaded piece's block
  uint32_t xl_e8[kXlTiles][KQ];  // MODE 4, staged run: those bytes for each tile of the batch
  // two accumulator sets: the GEMM of tile j fills one while the epilogue
  // of tile j-1 reads the other
  v4f acc0[NT], acc1[NT];
  v4f acc2[NT], acc3[NT];  // B2: the other pair's tiles
  // the staged run: the bf16 X rows in LDS
  uint8_t* xraw;
  float cs0, cs1;   // per set: this lane's row rescale factor (power of two, 1 for ordinary rows)
  float cs2, cs3;   // B2: the other pair's
  // set-up values in flight: this thread's column (tid < N) and the MX scale bytes
  float cv_sw;
  uint16_t cv_b, cv_g, cv_be;
  uint8_t wse[NT][KC];

  __device__ __forceinline__ bool tv(int t) const { return FULL || t < nv; }  // column tile t of the slice is real
  __device__ __forceinline__ bool kv(int k) const { return FULL || k < K; }   // column k of X is real

  __device__ __forceinline__ ResBlock(const FwdBlock& p_, int64_t tb_, int64_t te_, uint8_t* smem)
      : p(p_), tb(tb_), te(te_) {
    K = p.K;
    N = p.N;
    ldy = p.ldy > 0 ? p.ldy : p.N;
    kcv = FULL ? KC : (K + 127) >> 7;
    kb = K >> 5;
    T16 = N >> 4;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    r = lane & 15;
    g = lane >> 4;
    hrow = 2 * wave + (lane >> 5);  // the tile row this lane quantizes
    hl = lane & 31;                  // its lane within that row's half
    nv = FULL ? NT : min(max(T16 - wave * NT, 0), NT);
    c0 = 16 * NT * wave;
    inv_nw = nv > 0 ? 1.0f / (float)(16 * nv) : 0.0f;
    const ResLds l = res_lds(NT, KC, N, B2 ? 4 : 2);
    codes = smem + l.codes;
    xe8 = smem + l.xe8;
    rs = reinterpret_cast<float*>(smem + l.rs);
    red = reinterpret_cast<float2*>(smem + l.red);
    cvec = reinterpret_cast<float*>(smem + l.cvec);
    wmx = reinterpret_cast<float*>(smem + l.wmx);
    ystg = smem + l.ystg + wave * (kResRows * res_yst(NT));
    yprev = smem + l.yprev + wave * (kResRows * res_yst(NT));
  }

  // ---- X row of tile `t` for this lane into register slot S: elements
  // 256q + 8*hl .. +8.  The tile is read through a bounds-checked buffer
  // that covers only its rows inside both M and the workgroup's range, so
  // rows past M and tiles past the range read as zeros without a branch (a
  // zero never changes a max, and such rows are never stored); columns are
  // clamped to K-8 (duplicates, never stored either).
  template <int S>
  __device__ __forceinline__ void load_x(int64_t t) {
    if (MODE == 4) {
      // codes: 8 bytes per piece, the same elements as the bf16 path; the
      // scale byte of each piece's 32 x 32 block (rows clamped into M: a
      // row past M has zero codes, its scale is never used)
      const int64_t row0 = min(t * kResRows, p.M);
      const int64_t left = min(min(te * kResRows, p.M) - row0, (int64_t)kResRows);
      const int bytes = left > 0 ? (int)left * K : 0;
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.xq + row0 * K), (short)0, bytes, kBufferWord3);
      const uint32_t rb = (uint32_t)hrow * (uint32_t)K;
      const int64_t mc = min(t * kResRows + hrow, p.M - 1);
      const uint8_t* srow = p.xs + (mc >> 5) * kb;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        int k = q * 256 + hl * 8;
        if (!FULL) k = k < K ? k : K - 8;
        const uint2 c = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, rb + (uint32_t)k, 0, 0));
        xr[S][q] = make_uint4(c.x, c.y, 0u, 0u);
        xq8[S][q] = srow[k >> 5];
      }
      return;
    }
    const int64_t row0 = min(t * kResRows, p.M);
    const int64_t left = min(min(te * kResRows, p.M) - row0, (int64_t)kResRows);
    const int bytes = left > 0 ? (int)left * K * 2 : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x + row0 * K), (short)0, bytes, kBufferWord3);
    const uint32_t rb = (uint32_t)hrow * (uint32_t)(2 * K);
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      int k = q * 256 + hl * 8;
      if (!FULL) k = k < K ? k : K - 8;
      xr[S][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, rb + 2 * (uint32_t)k, 0, 0));
    }
  }

  // ---- quantize register slot S (tile t) into code buffer `buf`.  Values
  // are unpacked 8 at a time; with more than two 16-byte pieces per lane
  // the row max-abs is taken on the packed bf16 bit patterns instead
  // (|x| ordering equals the ordering of the sign-cleared bits).  Per-row
  // values go to LDS from every lane of the half (same address, same value)
  // so that the FULL variant has no divergent branch.
  template <int S>
  __device__ __forceinline__ void quantize(int64_t t, int buf) {
    const int64_t m = t * kResRows + hrow;
    // past this workgroup's range the tile is a stale slot: LDS only, never
    // the optional global outputs (those rows belong to another workgroup)
    const bool out_ok = OPT && t < te && m < p.M;
    uint8_t* crow = codes + (buf * kResRows + hrow) * LDX;
    if (MODE == 4) {
      // the codes are the input: into the code buffer, the block scales into
      // the same LDS slots as MODE 3's (block 8q + hl/4 at (g, c) = ((hl/4)%4, 2q + hl/16))
      uint8_t* erow = xe8 + (buf * kResRows + hrow) * XE + ((hl >> 2) & 3) * (4 * KP) + (hl >> 4);
      float emax = 0.0f;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        const int k = q * 256 + hl * 8;
        if (kv(k)) {
          const uint32_t e8 = xq8[S][q];
          emax = fmaxf(emax, (float)e8);
          erow[2 * q] = (uint8_t)e8;
          *reinterpret_cast<uint2*>(crow + k) = make_uint2(xr[S][q].x, xr[S][q].y);
        }
      }
      emax = half_max(emax);
      rs[buf * kResRows + hrow] = emax;
      return;
    }
    if (MODE == 3) {
      // block of piece q: 8q + hl/4, stored at LDS slot (g = (hl/4)%4, c = 2q + hl/16)
      uint8_t* erow = xe8 + (buf * kResRows + hrow) * XE + ((hl >> 2) & 3) * (4 * KP) + (hl >> 4);
      float emax = 0.0f;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        float v[8];
        unpack8(xr[S][q], v);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
        a = quad_max(a);  // a 32-element block is held by 4 consecutive lanes
        const int e8 = e8m0_from_amax<0>(a);
        const float mu = e8m0_inv_multiplier(e8);
        const int k = q * 256 + hl * 8;
        if (kv(k)) {
          emax = fmaxf(emax, (float)e8);
          erow[2 * q] = (uint8_t)e8;  // the quad's 4 lanes write the same byte
          if (out_ok && p.sx_out != nullptr && (hl & 3) == 0)
            static_cast<uint8_t*>(p.sx_out)[m * kb + (k >> 5)] = (uint8_t)e8;
          const uint32_t lo = cvt4<0>(v[0] * mu, v[1] * mu, v[2] * mu, v[3] * mu);
          const uint32_t hi = cvt4<0>(v[4] * mu, v[5] * mu, v[6] * mu, v[7] * mu);
          *reinterpret_cast<uint2*>(crow + k) = make_uint2(lo, hi);
          if (out_ok && p.qx_out != nullptr) *reinterpret_cast<uint2*>(p.qx_out + m * K + k) = make_uint2(lo, hi);
        }
      }
      emax = half_max(emax);
      rs[buf * kResRows + hrow] = emax;
      return;
    }
    float rmul;
    if (MODE == 1) {
      float a = 0.0f;
      if (KQ <= 2) {
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
          float v[8];
          unpack8(xr[S][q], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
        }
      } else {
        uint32_t mb = 0;
#pragma unroll
        for (int q = 0; q < KQ; ++q) mb = max(mb, absmax_bits8(xr[S][q]));
        a = __uint_as_float(mb << 16);
      }
      a = half_max(a);
      const ScalePair sp = scales_from_amax<0>(a);  // both rows' divisions in one pass
      rs[buf * kResRows + hrow] = sp.s;
      if (out_ok && p.sx_out != nullptr && hl == 0) static_cast<float*>(p.sx_out)[m] = sp.s;
      rmul = sp.r;
    } else {
      rmul = p.x_r;
    }
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int k = q * 256 + hl * 8;
      if (kv(k)) {
        float v[8];
        unpack8(xr[S][q], v);
        // the first convert of each word leaves bits 16-31 of its `old`
        // operand (here the input word) for the second one to overwrite
        uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * rmul, v[1] * rmul, (int)xr[S][q].x, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * rmul, v[3] * rmul, (int)lo, true);
        uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * rmul, v[5] * rmul, (int)xr[S][q].z, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * rmul, v[7] * rmul, (int)hi, true);
        *reinterpret_cast<uint2*>(crow + k) = make_uint2(lo, hi);
        if (out_ok && p.qx_out != nullptr) *reinterpret_cast<uint2*>(p.qx_out + m * K + k) = make_uint2(lo, hi);
      }
    }
  }

  // ---- set-up, part 1: the weight slice straight into the fragment
  // registers (fragment-interleaved W^T: lane l reads bytes 16l of both
  // 1 KiB halves of each 2 KiB block; chunks in the order the GEMM uses
  // them) and the MX scale bytes.  Nothing here waits for a load.
  template <int C0 = 0, int C1 = KC>
  __device__ __forceinline__ void request_weights() {
    const int64_t nch = (K + 127) >> 7;
    const uint8_t* base = p.qw + (int64_t)(wave * NT) * nch * 2048 + lane * 16;
#pragma unroll
    for (int c = C0; c < C1; ++c) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (FULL || (tv(t) && c < kcv)) {
          const uint8_t* blk = base + ((int64_t)t * nch + c) * 2048;
          a = *reinterpret_cast<const uint4*>(blk);
          b = *reinterpret_cast<const uint4*>(blk + 1024);
        }
        v8i f;
        f[0] = (int)a.x; f[1] = (int)a.y; f[2] = (int)a.z; f[3] = (int)a.w;
        f[4] = (int)b.x; f[5] = (int)b.y; f[6] = (int)b.z; f[7] = (int)b.w;
        wf[t][c] = f;
      }
    }
    if (MX && C0 == 0) {
      // MODE 3: W's scales [N][K/32] (32 consecutive k of column col);
      // MODE 4: [K/32][N/32] (32 x 32 blocks of W[K][N])
      const uint8_t* sw8 = static_cast<const uint8_t*>(p.sw);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = c0 + 16 * t + r;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int blk = 4 * c + g;
          const int64_t si = MODE == 4 ? (int64_t)blk * (N >> 5) + (col >> 5) : (int64_t)col * kb + blk;
          wse[t][c] = (tv(t) && (FULL || blk < kb)) ? sw8[si] : (uint8_t)127;
        }
      }
    }
  }

  // ---- this thread's column vectors (column tid; threads past N load
  // column 0 and never use it).  No branch: a missing vector reads element 0
  // of X instead and the value is replaced by its default, so no load sits
  // in a branch that would have to wait for it there.
  __device__ __forceinline__ void request_vectors() {
    const int ct = tid < N ? tid : 0;
    // a valid address to read in place of a missing vector (MODE 4 has X as codes)
    const uint16_t* x0 = MODE == 4 ? reinterpret_cast<const uint16_t*>(p.xq) : p.x;
    cv_sw = MODE == 1 ? static_cast<const float*>(p.sw)[ct] : (MODE == 0 ? static_cast<const float*>(p.sw)[0] : 1.0f);
    const uint16_t b = *(p.bias ? p.bias + ct : x0), gm = *(p.gamma ? p.gamma + ct : x0);
    const uint16_t be = *(p.beta ? p.beta + ct : x0);
    cv_b = p.bias ? b : (uint16_t)0;
    cv_g = p.gamma ? gm : (uint16_t)0x3F80;
    cv_be = p.beta ? be : (uint16_t)0;
  }

  // ---- set-up, part 2: MX scale words, column vectors into LDS with their
  // maxima, LDS padding
  __device__ __forceinline__ void stage_vectors() {
    float msw = 0.0f, mb = 0.0f, ewm = 0.0f;
    if (MX) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int q = 0; q < KP; ++q) wsc[t][q] = 0;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          wsc[t][c >> 2] |= (uint32_t)wse[t][c] << (8 * (c & 3));
          if (tv(t) && (FULL || 4 * c + g < kb)) ewm = fmaxf(ewm, (float)wse[t][c]);
        }
      }
    }
    if (tid < N) {
      const float b = bf16_lo(cv_b);
      cvec[tid] = cv_sw;
      cvec[N + tid] = b;
      cvec[2 * N + tid] = bf16_lo(cv_g);
      cvec[3 * N + tid] = bf16_lo(cv_be);
      msw = cv_sw;
      mb = fabsf(b);
    }
    msw = wave_max_dpp(msw);
    mb = wave_max_dpp(mb);
    ewm = wave_max_dpp(ewm);
    if (lane == 0) {
      wmx[wave] = msw;
      wmx[8 + wave] = mb;
      wmx[16 + wave] = ewm;
    }
    // zero the code rows past K (up to the last chunk) and give the padded
    // MX blocks a unit scale, in every buffer (two, or four for B2: a stale
    // NaN code there would turn its zero weight into a NaN)
    if (!FULL) {
      constexpr int NB = B2 ? 4 : 2;
      const int padb = kcv * 128 - K;  // multiple of 16
      if (padb > 0) {
        const int per = padb >> 4;
        for (int u = tid; u < NB * kResRows * per; u += kThreads) {
          const int row = u / per, o = K + 16 * (u - row * per);
          *reinterpret_cast<uint4*>(codes + row * LDX + o) = make_uint4(0, 0, 0, 0);
        }
      }
      if (MX) {
        for (int u = tid; u < NB * kResRows * XE; u += kThreads) {
          const int sl = u % XE, c = sl % (4 * KP);  // LDS slot (g, c) holds block 4c+g
          if (4 * c + sl / (4 * KP) >= kb) xe8[u] = 127;
        }
      }
    }
  }

  // after the set-up barrier
  __device__ __forceinline__ void read_bounds() {
    float msw = 0.0f, mb = 0.0f, ewm = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      msw = fmaxf(msw, wmx[w]);
      mb = fmaxf(mb, wmx[8 + w]);
      ewm = fmaxf(ewm, wmx[16 + w]);
    }
    const float kk = (448.0f * 448.0f) * (float)K;
    // launch constants: kept in scalar registers
    bw = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(MX ? ldexpf(kk, (int)ewm - 127) : kk * msw)));
    bb = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mb)));
  }

  // ---- GEMM of the tile in code buffer `buf`
  __device__ __forceinline__ void mma(int buf, v4f (&acc)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t* brow = codes + (buf * kResRows + r) * LDX + 16 * g;
    const uint32_t* erow = reinterpret_cast<const uint32_t*>(xe8 + (buf * kResRows + r) * XE + g * (4 * KP));
    uint32_t xsw[KP];
    if (MX) {
#pragma unroll
      for (int q = 0; q < KP; ++q) xsw[q] = erow[q];
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (!FULL && c >= kcv) break;
      const uint4 a = *reinterpret_cast<const uint4*>(brow + c * 128);
      const uint4 b = *reinterpret_cast<const uint4*>(brow + c * 128 + 64);
      v8i xf;
      xf[0] = (int)a.x; xf[1] = (int)a.y; xf[2] = (int)a.z; xf[3] = (int)a.w;
      xf[4] = (int)b.x; xf[5] = (int)b.y; xf[6] = (int)b.z; xf[7] = (int)b.w;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (MX)
          acc[t] = mfma_mx_sel(c & 3, wf[t][c], xf, acc[t], wsc[t][c >> 2], xsw[c >> 2]);
        else
          acc[t] = mfma_fp8<0, 0>(wf[t][c], xf, acc[t]);
      }
      // keep at most two chunks of B fragments in flight (with 8 chunks the
      // scheduler would otherwise hoist every LDS read and spill)
      if (KC > 4 && (c & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // This lane's per-column constants (its 4 columns of each of the NT tiles):
  // s_w and bias for the statistics, gamma and beta for the output.  The
  // pipelined run reads them from LDS at every tile; the staged run holds
  // them in the registers the weight leaves free after its GEMM.
  struct ColSB {
    float4 sw[NT], b[NT];
  };
  struct ColGB {
    float4 g[NT], be[NT];
  };
  __device__ __forceinline__ ColSB col_sb() const {
    ColSB v;
    const float* cb = cvec + c0 + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      v.sw[t] = tv(t) ? *reinterpret_cast<const float4*>(cb + 16 * t) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      v.b[t] = tv(t) ? *reinterpret_cast<const float4*>(cb + N + 16 * t) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    return v;
  }
  __device__ __forceinline__ ColGB col_gb() const {
    ColGB v;
    const float* cb = cvec + 2 * N + c0 + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      v.g[t] = tv(t) ? *reinterpret_cast<const float4*>(cb + 16 * t) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      v.be[t] = tv(t) ? *reinterpret_cast<const float4*>(cb + N + 16 * t) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    return v;
  }

  // ---- epilogue, part 1: z = dequant(acc) + b in place; this slice's row
  // sum and centred sum of squares to LDS
  // (the pipelined run: the constants from LDS, tile by tile, so they never
  // occupy registers across the loop)
  __device__ __forceinline__ void epilogue_stats(int buf, v4f (&acc)[NT], float& cs) {
    epilogue_stats_t<false>(buf, acc, cs, nullptr);
  }
  // (the staged run: the constants already in registers)
  __device__ __forceinline__ void epilogue_stats(int buf, v4f (&acc)[NT], float& cs, const ColSB& cv) {
    epilogue_stats_t<true>(buf, acc, cs, &cv);
  }
  template <bool REG>
  __device__ __forceinline__ void epilogue_stats_t(int buf, v4f (&acc)[NT], float& cs, const ColSB* cv) {
    const float* cb = cvec + c0 + 4 * g;
    const float rsv = rs[buf * kResRows + r];
    const float sx = MODE == 1 ? rsv : (MODE == 0 ? p.x_s : 1.0f);
    const float bound = MX ? ldexpf(bw, (int)rsv - 127) + bb : sx * bw + bb;
    cs = row_rescale(bound);
    // sums as short trees (per tile, then over the tiles) rather than one
    // long chain: the statistics sit on the step's critical path
    float st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      st[t] = 0.0f;
      if (tv(t)) {
        float4 sw4, b4;
        if constexpr (REG) {
          sw4 = cv->sw[t];
          b4 = cv->b[t];
        } else {
          sw4 = *reinterpret_cast<const float4*>(cb + 16 * t);
          b4 = *reinterpret_cast<const float4*>(cb + N + 16 * t);
        }
        const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[t][j] = MX ? acc[t][j] + bv[j] : fmaf(acc[t][j], sx * swv[j], bv[j]);
        st[t] = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
      }
    }
    if constexpr (EPI == 1) {  // BlockNorm: the slice's sum of squares (scaled by cs like the LayerNorm path)
      float qt[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float d0 = acc[t][0] * cs, d1 = acc[t][1] * cs, d2 = acc[t][2] * cs, d3 = acc[t][3] * cs;
        qt[t] = fmaf(d1, d1, d0 * d0) + fmaf(d3, d3, d2 * d2);
      }
      red[(buf * kResRows + r) * kRedRow + wave] = make_float2(sum4(tree_sum<NT>(qt)), 0.0f);
      return;
    }
    const float s = sum4(tree_sum<NT>(st));
    const float mw = s * inv_nw;
    // deviations scaled by cs before squaring (rows too large to square in
    // fp32); one fma rounds (z - mw) * cs once, which for cs = 1 is z - mw
    // and otherwise its exact power-of-two scaling: no branch on the rare case
    const float nmc = -mw * cs;
    float qt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qt[t] = 0.0f;
      if (tv(t)) {
        const float d0 = fmaf(acc[t][0], cs, nmc), d1 = fmaf(acc[t][1], cs, nmc);
        const float d2 = fmaf(acc[t][2], cs, nmc), d3 = fmaf(acc[t][3], cs, nmc);
        qt[t] = fmaf(d1, d1, d0 * d0) + fmaf(d3, d3, d2 * d2);
      }
    }
    const float q = sum4(tree_sum<NT>(qt));
    red[(buf * kResRows + r) * kRedRow + wave] = make_float2(s, q);  // the row's 4 lanes write the same pair
  }

  // ---- epilogue, part 2 (after the barrier): combine the slices, normalize, store
  __device__ __forceinline__ void epilogue_out(int buf, int64_t t, const v4f (&acc)[NT], float cs) {
    epilogue_out_t<false>(buf, t, acc, cs, nullptr);
  }
  __device__ __forceinline__ void epilogue_out(int buf, int64_t t, const v4f (&acc)[NT], float cs, const ColGB& cv) {
    epilogue_out_t<true>(buf, t, acc, cs, &cv);
  }
  template <bool REG>
  __device__ __forceinline__ void epilogue_out_t(int buf, int64_t t, const v4f (&acc)[NT], float cs, const ColGB* cv) {
    if constexpr (EPI == 1) {
      blocknorm_out(buf, t, acc, cs);
      return;
    }
    // The 4 lanes of a row (g = 0..3) each take two of the 8 slices (2g and
    // 2g + 1) and the partial terms are summed across them with permlane
    // swaps: one LDS read per lane and a quarter of the combine each.
    const float4 u = reinterpret_cast<const float4*>(red + (buf * kResRows + r) * kRedRow)[g];
    const float S = sum4(u.x + u.z);
    // guard-free shapes: N = 128 NT, a compile-time reciprocal (exact: a power of two for NT = 1, 2, 4)
    const float invn = FULL ? 1.0f / (float)(128 * NT) : 1.0f / (float)N;
    const float mean = S * invn;
    // within-slice centred sums plus the between-slice term
    // (s_w - n_w mean)^2 / n_w, the deviations scaled by cs like the
    // within-slice sums (cs = 1: unscaled)
    float V;
    if (FULL || N == 128 * NT) {  // every slice has 16*NT columns
      const float ns = (float)(16 * NT);
      float d0, d1;
      if ((NT & (NT - 1)) == 0) {  // ns and cs powers of two: -ns*mean*cs is exact
        const float nsm = -ns * mean * cs;
        d0 = fmaf(u.x, cs, nsm);
        d1 = fmaf(u.z, cs, nsm);
      } else {
        d0 = fmaf(-ns, mean, u.x) * cs;
        d1 = fmaf(-ns, mean, u.z) * cs;
      }
      V = (u.y + u.w) + fmaf(d0, d0, d1 * d1) * (1.0f / ns);
    } else {
      V = u.y + u.w;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nw = 16 * min(max(T16 - (2 * g + h) * NT, 0), NT);
        if (nw > 0) {
          const float d = fmaf(-(float)nw, mean, h ? u.z : u.x) * cs;
          V = fmaf(d * (1.0f / (float)nw), d, V);
        }
      }
    }
    V = sum4(V);
    // variance of the scaled deviations is var * cs^2: rstd = cs / sqrt(var cs^2 + eps cs^2)
    const float rstd = cs * __builtin_amdgcn_rsqf(fmaf(V, invn, p.eps * cs * cs));
    const int64_t m = t * kResRows + r;
    const bool row_ok = FULL || m < p.M;
    if (OPT && row_ok && wave == 0 && g == 0) {
      if (p.mean) p.mean[m] = mean;
      if (p.rstd) p.rstd[m] = rstd;
    }
    const float nmr = -mean * rstd;
    const int cl = c0 + 4 * g;  // this lane's first column (tile t adds 16t)
    const float* gb = cvec + 2 * N + cl;
    constexpr int YST = res_yst(NT);
    uint8_t* ys = COOP && (t & 1) ? ystg + kWaves * kResRows * YST : ystg;
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2) {
      if (tv(t2)) {
        float4 ga, be;
        if constexpr (REG) {
          ga = cv->g[t2];
          be = cv->be[t2];
        } else {
          ga = *reinterpret_cast<const float4*>(gb + 16 * t2);
          be = *reinterpret_cast<const float4*>(gb + N + 16 * t2);
        }
        const float gv[4] = {ga.x, ga.y, ga.z, ga.w}, bv[4] = {be.x, be.y, be.z, be.w};
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = fmaf(fmaf(acc[t2][j], rstd, nmr), gv[j], bv[j]);
        *reinterpret_cast<uint2*>(ys + r * YST + (16 * t2 + 4 * g) * 2) =
            make_uint2(pack_bf16_hw(o[0], o[1]), pack_bf16_hw(o[2], o[3]));
        if (OPT && p.z != nullptr && row_ok)
          *reinterpret_cast<float4*>(p.z + m * ldy + cl + 16 * t2) =
              make_float4(acc[t2][0], acc[t2][1], acc[t2][2], acc[t2][3]);
      }
    }
    if constexpr (!COOP) store_y(t);
    if constexpr (OPT && NT % 2 == 0) {
      if (p.y_codes != nullptr) square_y(t);
    }
  }

  // Y also leaves quantized in 32 x 32 blocks (e4m3 codes and E8M0 scales,
  // the square-block recipe's input for the next layer: the activation
  // quantization fused into the normalization that produces it, the GEM
  // page's PreNorm fusion).  The codes are those of the bf16 Y: the same as
  // quantizing the stored Y.  A block is two 16-row tiles (the workgroup's
  // tile range starts on a pair) by two of this wavefront's 16-column tiles;
  // the even tile keeps its Y block and its maxima, the odd one completes
  // the block.  N = 128 NT with NT even and M % 32 == 0 (checked by the
  // entry point), so every tile and row is real.
  __device__ __forceinline__ void square_y(int64_t t) {
    constexpr int YST = res_yst(NT), NB = NT / 2;
    uint2 cur[NT];
    float bm[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) bm[cb] = 0.0f;
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2) {
      cur[t2] = *reinterpret_cast<const uint2*>(ystg + r * YST + (16 * t2 + 4 * g) * 2);
      bm[t2 >> 1] = fmaxf(bm[t2 >> 1], fmaxf(fmaxf(fabsf(bf16_lo(cur[t2].x)), fabsf(bf16_hi(cur[t2].x))),
                                             fmaxf(fabsf(bf16_lo(cur[t2].y)), fabsf(bf16_hi(cur[t2].y)))));
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) bm[cb] = rows4_max(row16_max(bm[cb]));
    if ((t & 1) == 0) {
#pragma unroll
      for (int t2 = 0; t2 < NT; ++t2) *reinterpret_cast<uint2*>(yprev + r * YST + (16 * t2 + 4 * g) * 2) = cur[t2];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) sq_prev[cb] = bm[cb];
      return;
    }
    const int64_t m1 = t * kResRows + r, m0 = m1 - kResRows;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int e8 = e8m0_from_amax<0>(fmaxf(bm[cb], sq_prev[cb]));
      const float mu = e8m0_inv_multiplier(e8);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t2 = 2 * cb + h, col = c0 + 16 * t2 + 4 * g;
        const uint2 pv = *reinterpret_cast<const uint2*>(yprev + r * YST + (16 * t2 + 4 * g) * 2);
        const uint32_t qp = cvt4<0>(bf16_lo(pv.x) * mu, bf16_hi(pv.x) * mu, bf16_lo(pv.y) * mu, bf16_hi(pv.y) * mu);
        const uint32_t qc = cvt4<0>(bf16_lo(cur[t2].x) * mu, bf16_hi(cur[t2].x) * mu, bf16_lo(cur[t2].y) * mu,
                                    bf16_hi(cur[t2].y) * mu);
        *reinterpret_cast<uint32_t*>(p.y_codes + m0 * N + col) = qp;
        *reinterpret_cast<uint32_t*>(p.y_codes + m1 * N + col) = qc;
      }
      if (lane == 0) p.y_scales[(t >> 1) * (N >> 5) + (c0 >> 5) + cb] = (uint8_t)e8;
    }
  }

  // BlockNorm + Hard Swish (after the barrier): the 256-column block of this
  // wavefront's slice has 256 / (16 NT) slices, whose sums of squares the
  // row's lanes add (NT = 2: all 8 slices, two per lane; NT = 4: the four
  // slices of the block, two per lane, paired across g and g^1); then
  // y = h(z / sqrt(mean z^2 + eps)) with h(t) = t * clamp(t / 6 + 1/2, 0, 1).
  __device__ __forceinline__ void blocknorm_out(int buf, int64_t t, const v4f (&acc)[NT], float cs) {
    static_assert(NT == 2 || NT == 4, "BlockNorm slabs are 256 or 512 columns");
    const float4* rw = reinterpret_cast<const float4*>(red + (buf * kResRows + r) * kRedRow);
    float V;
    if (NT == 2) {
      const float4 u = rw[g];
      V = sum4(u.x + u.z);
    } else {
      const float4 u = rw[2 * (wave >> 2) + (g & 1)];
      const float v = u.x + u.z;
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      V = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    const float rinv = cs * __builtin_amdgcn_rsqf(fmaf(V, 1.0f / (float)kBlockNorm, p.eps * cs * cs));
    const int64_t m = t * kResRows + r;
    const bool row_ok = FULL || m < p.M;
    const int cl = c0 + 4 * g;
    constexpr int YST = res_yst(NT);
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2) {
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = acc[t2][j] * rinv;
        o[j] = v * __builtin_amdgcn_fmed3f(fmaf(v, 1.0f / 6.0f, 0.5f), 0.0f, 1.0f);
      }
      *reinterpret_cast<uint2*>(ystg + r * YST + (16 * t2 + 4 * g) * 2) =
          make_uint2(pack_bf16_hw(o[0], o[1]), pack_bf16_hw(o[2], o[3]));
      if (OPT && p.z != nullptr && row_ok)
        *reinterpret_cast<float4*>(p.z + m * ldy + cl + 16 * t2) =
            make_float4(acc[t2][0], acc[t2][1], acc[t2][2], acc[t2][3]);
    }
    store_y(t);
  }

  __device__ __forceinline__ void store_y(int64_t t) {
    constexpr int YST = res_yst(NT);
    // The wavefront's 16 x 16*NT block of Y goes out from the staging rows in
    // 16-byte pieces, consecutive lanes along a row: each store instruction
    // writes whole 32*NT-byte row segments (for NT = 4, eight 128-byte
    // lines), as non-temporal (streaming) stores: Y is not read again here,
    // and streaming it keeps the write-back of one launch from holding up
    // the next launch's loads.  LDS operations of one wavefront complete in
    // order, so the reads see the writes above and the next tile's writes
    // come after them.
    constexpr int CPR = 2 * NT, TOT = kResRows * CPR;  // 16-byte pieces per row / per block
    // the tile's first row of Y (wave-uniform); each piece's offset from it fits 32 bits
    uint16_t* ytile = p.y + t * kResRows * ldy + c0;
#pragma unroll
    for (int i = 0; i < (TOT + 63) / 64; ++i) {
      const int u = lane + 64 * i;
      if (TOT % 64 == 0 || u < TOT) {
        const int row = u / CPR, ch = u - row * CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(ystg + row * YST + ch * 16);
        if (FULL || (t * kResRows + row < p.M && ch < 2 * nv))
          __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(ytile + (row * ldy + ch * 8)));
      }
    }
  }

  // MFMAs of the current tile interleaved with the VALU work around them
  // (the previous tile's normalization and stores, the next tile's
  // quantization): one MFMA, then a few VALU instructions, repeatedly
  __device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int i = 0; i < NT * KC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
    }
  }

  // one tile of the loop (j >= 1): GEMM of tile j into set A alongside the
  // normalization and stores of tile j-1 (set !A) and the quantization of
  // tile j+1 (slot S1 = (j+1) % D; past the range it quantizes a stale slot
  // into the unused buffer); then tile j+1+D is requested into that slot and
  // tile j's statistics go to LDS
  template <int S1, int A>
  __device__ __forceinline__ void step(int64_t j) {
    const int buf = (int)(j & 1);
    const int64_t t = tb + j;
    v4f (&cur)[NT] = A ? acc1 : acc0;
    v4f (&prev)[NT] = A ? acc0 : acc1;
    mma(buf, cur);
    epilogue_out(buf ^ 1, t - 1, prev, A ? cs0 : cs1);
    quantize<S1>(t + 1, buf ^ 1);
    if (FULL && !OPT) interleave_hint();
    load_x<S1>(t + 1 + D);
    epilogue_stats(buf, cur, A ? cs1 : cs0);
    __syncthreads();
  }

  // ---- B2: two tiles per step -------------------------------------------
  // Pair j = tiles tb + 2j, tb + 2j + 1 (LDS buffers 2A, 2A + 1 with A = j & 1,
  // accumulator sets acc0/acc1 for A = 0 and acc2/acc3 for A = 1; tile t in
  // register slot (t - tb) % D).  Step j: GEMM of pair j alongside the
  // normalization and stores of pair j - 1 and the quantization of pair j + 1
  // (slots S2, S3), whose refills (D tiles on) are then requested; pair j's
  // statistics; one barrier.  Each tile runs the same functions as in the
  // one-tile steps, so the results are the same bit for bit.
  template <int S2, int S3, int A>
  __device__ __forceinline__ void step2(int64_t j) {
    const int64_t t = tb + 2 * j;
    v4f (&ca)[NT] = A ? acc2 : acc0;
    v4f (&cb)[NT] = A ? acc3 : acc1;
    v4f (&pa)[NT] = A ? acc0 : acc2;
    v4f (&pb)[NT] = A ? acc1 : acc3;
    mma(2 * A, ca);
    mma(2 * A + 1, cb);
    epilogue_out(2 * (1 - A), t - 2, pa, A ? cs0 : cs2);
    epilogue_out(2 * (1 - A) + 1, t - 1, pb, A ? cs1 : cs3);
    quantize<S2>(t + 2, 2 * (1 - A));
    quantize<S3>(t + 3, 2 * (1 - A) + 1);
    load_x<S2>(t + 2 + D);
    load_x<S3>(t + 3 + D);
    epilogue_stats(2 * A, ca, A ? cs2 : cs0);
    epilogue_stats(2 * A + 1, cb, A ? cs3 : cs1);
    __syncthreads();
  }
  // groups of G = max(D / 2, 2) pairs from j = 1 + G i: pair m of the group
  // quantizes tiles 2j + 2 and 2j + 3 from slots (4 + 2m) % D and (5 + 2m) % D
  // and fills sets (1 + m) & 1
  template <int... M>
  __device__ __forceinline__ void step2_group(int64_t j, std::integer_sequence<int, M...>) {
    (step2<(4 + 2 * M) % D, (5 + 2 * M) % D, (1 + M) & 1>(j + M), ...);
  }
  template <int... M>
  __device__ __forceinline__ void step2_tail(int64_t& j, int64_t np, std::integer_sequence<int, M...>) {
    ((j < np ? (step2<(4 + 2 * M) % D, (5 + 2 * M) % D, (1 + M) & 1>(j), ++j) : j), ...);
  }
  // the last pair's normalization; its second tile only when it exists
  template <int A>
  __device__ __forceinline__ void last_pair_out(int64_t t) {
    epilogue_out(2 * A, t, A ? acc2 : acc0, A ? cs2 : cs0);
    if (t + 1 < te) epilogue_out(2 * A + 1, t + 1, A ? acc3 : acc1, A ? cs3 : cs1);
  }
  __device__ __forceinline__ void run_b2() {
    if (tb >= te) return;
    load_x<0>(tb);
    request_vectors();
    request_weights();
    prologue_loads(std::make_integer_sequence<int, D - 1>{});
    __builtin_amdgcn_sched_barrier(0);
    quantize<0>(tb, 0);
    quantize<1>(tb + 1, 1);
    load_x<0>(tb + D);
    load_x<1>(tb + 1 + D);
    stage_vectors();
    __syncthreads();
    read_bounds();
    // pair 0: GEMM alongside the quantization of pair 1
    mma(0, acc0);
    mma(1, acc1);
    quantize<(2 % D)>(tb + 2, 2);
    quantize<(3 % D)>(tb + 3, 3);
    load_x<(2 % D)>(tb + 2 + D);
    load_x<(3 % D)>(tb + 3 + D);
    epilogue_stats(0, acc0, cs0);
    epilogue_stats(1, acc1, cs1);
    __syncthreads();
    // whole groups of pairs, then the tail (see run() on why)
    constexpr int G = D / 2 > 2 ? D / 2 : 2;
    const int64_t np = (te - tb + 1) / 2;
    int64_t j = 1;
    for (int64_t i = (np - 1) / G; i > 0; --i, j += G) step2_group(j, std::make_integer_sequence<int, G>{});
    step2_tail(j, np, std::make_integer_sequence<int, G - 1>{});
    const int64_t l = np - 1;
    if (l & 1) last_pair_out<1>(tb + 2 * l);
    else last_pair_out<0>(tb + 2 * l);
  }

  // the prologue's requests of tiles 1 .. D-1 (tile k into slot k)
  template <int... I>
  __device__ __forceinline__ void prologue_loads(std::integer_sequence<int, I...>) {
    (load_x<I + 1>(tb + I + 1), ...);
  }
  // one period of the slot and set pattern: steps j .. j + D - 1
  template <int... M>
  __device__ __forceinline__ void step_group(int64_t j, std::integer_sequence<int, M...>) {
    (step<(M + 2) % D, (M + 1) % 2>(j + M), ...);
  }
  // the remaining steps (fewer than D), in the same pattern
  template <int... M>
  __device__ __forceinline__ void step_tail(int64_t& j, int64_t n, std::integer_sequence<int, M...>) {
    ((j < n ? (step<(M + 2) % D, (M + 1) % 2>(j), ++j) : j), ...);
  }

  // COOP: the workgroup's 16 x N block of Y of tile t as whole rows, each
  // 16-byte piece read from the staging buffer (t & 1) of the wavefront that
  // produced it; called after a barrier that follows every wavefront's
  // staging writes of tile t
  __device__ __forceinline__ void coop_store(int64_t t) {
    constexpr int YST = res_yst(NT), PPR = 16 * NT, TOT = kResRows * PPR;  // pieces per row of N = 128 NT
    const uint8_t* yb = ystg - wave * (kResRows * YST) + ((t & 1) ? kWaves * kResRows * YST : 0);
#pragma unroll
    for (int i = 0; i < (TOT + kThreads - 1) / kThreads; ++i) {
      const int u = tid + kThreads * i;
      if (TOT % kThreads == 0 || u < TOT) {
        const int row = u / PPR, pc = u - row * PPR;
        const int w = pc / (2 * NT), ch = pc - w * (2 * NT);
        const uint4 v = *reinterpret_cast<const uint4*>(yb + (w * kResRows + row) * YST + ch * 16);
        __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<v4u*>(p.y + (t * kResRows + row) * ldy + pc * 8));
      }
    }
  }

  // one tile without the pipeline (deep K): GEMM of tile j, quantization of
  // tile j+1 from the single slot, request of tile j+2, statistics, barrier,
  // normalization and stores
  __device__ __forceinline__ void step_seq(int64_t j) {
    const int buf = (int)(j & 1);
    const int64_t t = tb + j;
    mma(buf, acc0);
    quantize<0>(t + 1, buf ^ 1);
    load_x<0>(t + 2);
    epilogue_stats(buf, acc0, cs0);
    __syncthreads();
    if (COOP && j > 0) coop_store(t - 1);
    epilogue_out(buf, t, acc0, cs0);
  }

  // ---- the staged run ----------------------------------------------------
  // LDS pointers of the staged layout (replacing the constructor's)
  __device__ __forceinline__ void xl_layout(uint8_t* smem) {
    const XlLds l = xl_lds(NT, KC, N, K);
    xraw = smem + l.xraw;
    codes = smem + l.codes;
    xe8 = smem + l.xe8;
    rs = reinterpret_cast<float*>(smem + l.rs);
    red = reinterpret_cast<float2*>(smem + l.red);
    cvec = reinterpret_cast<float*>(smem + l.cvec);
    wmx = reinterpret_cast<float*>(smem + l.wmx);
    ystg = smem + l.ystg + wave * (kResRows * res_yst(NT));
  }

  // This wavefront's two rows (2w, 2w+1) of tile slots [I0, I1) of the
  // batch, straight from HBM into LDS (buffer loads with the LDS destination: lane
  // l's 16 bytes land at the wave-uniform LDS address + 16 l, so each
  // instruction moves 1 KiB of contiguous X).  The two rows are 4K
  // contiguous bytes in X and in LDS (row stride 2K), so a tile takes
  // K/256 = KQ instructions.  The buffer covers exactly the batch's rows;
  // slots past the batch read zeros.  Slots are requested with no branch,
  // so the compiler keeps them where they stand in the issue order (loads
  // complete in issue order: a tile requested after the weight waits for
  // it).
  // MODE 4 (X given as e4m3 codes, K = 512): the two rows are 2K = 1 KiB of
  // codes, one instruction per tile, at row stride K in LDS; the E8M0 byte of
  // each of this lane's pieces (block (m/32, k/32), rows clamped into M: a row
  // past M has zero codes, its scale is never used) with byte loads.
  template <int I0, int I1>
  __device__ __forceinline__ void xl_request_x() {
    const int64_t row0 = tb * kResRows;
    const int64_t rows = min(te * kResRows, p.M) - row0;
    if constexpr (MODE == 4) {
      static_assert(KQ == 2, "staged code input: K = 512");
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(p.xq + row0 * K), (short)0, (int)(rows * K), kBufferWord3);
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const uint32_t off = (uint32_t)((i * kResRows + 2 * wave) * K);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(xraw + off), 16,
                                                 off + 16u * (uint32_t)lane, 0, 0, 0);
      }
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const int64_t mc = min((tb + i) * kResRows + hrow, p.M - 1);
        const uint8_t* srow = p.xs + (mc >> 5) * kb;
#pragma unroll
        for (int q = 0; q < KQ; ++q) xl_e8[i][q] = srow[(q * 256 + hl * 8) >> 5];
      }
      return;
    }
    const int bytes = (int)(rows * K * 2);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x + row0 * K), (short)0, bytes, kBufferWord3);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
#pragma unroll
      for (int part = 0; part < KQ; ++part) {
        const uint32_t off = (uint32_t)((i * kResRows + 2 * wave) * 2 * K + part * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(xraw + off), 16,
                                                 off + 16u * (uint32_t)lane, 0, 0, 0);
      }
    }
  }

  // this lane's share of its row of tile i, from LDS into register slot 0
  // (the same elements load_x would fetch: 256q + 8 hl .. +8)
  __device__ __forceinline__ void xl_fetch(int i) {
    if constexpr (MODE == 4) {  // 8 codes per piece (the same elements) and the piece's block scale
      const uint8_t* row = xraw + (i * kResRows + hrow) * K;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        const uint2 c = *reinterpret_cast<const uint2*>(row + q * 256 + hl * 8);
        xr[0][q] = make_uint4(c.x, c.y, 0u, 0u);
        xq8[0][q] = xl_e8[i][q];
      }
      return;
    }
    const uint8_t* row = xraw + (i * kResRows + hrow) * 2 * K;
#pragma unroll
    for (int q = 0; q < KQ; ++q) xr[0][q] = *reinterpret_cast<const uint4*>(row + q * 512 + hl * 16);
  }

  // GEMM of the whole batch into `acc`, K chunk outermost: chunk c of the
  // weight serves every tile as soon as it has arrived (its loads were issued
  // chunk by chunk), so the MFMAs follow the weight as it lands.
  __device__ __forceinline__ void xl_mma(v4f (&acc)[kXlTiles][NT]) {
#pragma unroll
    for (int i = 0; i < kXlTiles; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[i][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int i = 0; i < kXlTiles; ++i) {
        const uint8_t* brow = codes + (i * kResRows + r) * LDX + 16 * g + c * 128;
        const uint4 a = *reinterpret_cast<const uint4*>(brow);
        const uint4 b = *reinterpret_cast<const uint4*>(brow + 64);
        v8i xf;
        xf[0] = (int)a.x; xf[1] = (int)a.y; xf[2] = (int)a.z; xf[3] = (int)a.w;
        xf[4] = (int)b.x; xf[5] = (int)b.y; xf[6] = (int)b.z; xf[7] = (int)b.w;
        uint32_t xsw = 0;
        if (MX) xsw = reinterpret_cast<const uint32_t*>(xe8 + (i * kResRows + r) * XE + g * (4 * KP))[c >> 2];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (MX)
            acc[i][t] = mfma_mx_sel(c & 3, wf[t][c], xf, acc[i][t], wsc[t][c >> 2], xsw);
          else
            acc[i][t] = mfma_fp8<0, 0>(wf[t][c], xf, acc[i][t]);
        }
      }
    }
  }

  // weight chunks [c0, c1) of the KC, requested between the quantization of
  // tile I and the next (the chunks spread evenly over the four tiles)
  template <int I>
  __device__ __forceinline__ void xl_weights_for() {
    request_weights<(I * KC) / kXlTiles, ((I + 1) * KC) / kXlTiles>();
  }
  template <int I>
  __device__ __forceinline__ void xl_quantize_tile() {
    xl_fetch(I);
    quantize<0>(tb + I, I);
  }

  // The staged run.  Order of requests: the whole batch's X (HBM, into LDS),
  // then the column vectors, then the weight chunk by chunk with one tile's
  // quantization after each part (a wavefront stalls once its memory
  // requests fill the queue, so its quantization work goes between them, and
  // every X tile was requested ahead of the weight).  One barrier; the GEMM
  // of the whole batch, chunk by chunk; the row statistics of every tile;
  // one barrier; normalization and stores.  At two wavefronts per SIMD the
  // MFMAs and the VALU work take turns on a SIMD, so the phases are ordered
  // by their dependencies rather than interleaved.
  template <bool EXACT>
  __device__ __forceinline__ void run_xl() {
    const int nt = EXACT ? kXlTiles : (int)(te - tb);
    if (nt <= 0) return;
    if (OPT && MODE == 0 && p.sx_out != nullptr && tb == 0 && tid == 0) static_cast<float*>(p.sx_out)[0] = p.x_s;
    static_assert(kXlTiles == 4, "the staged run covers four tiles");
    xl_request_x<0, kXlTiles>();
    request_vectors();
    __builtin_amdgcn_sched_barrier(0);
    xl_weights_for<0>();
    __builtin_amdgcn_sched_barrier(0);
    xl_quantize_tile<0>();
    __builtin_amdgcn_sched_barrier(0);
    xl_weights_for<1>();
    __builtin_amdgcn_sched_barrier(0);
    xl_quantize_tile<1>();
    __builtin_amdgcn_sched_barrier(0);
    xl_weights_for<2>();
    __builtin_amdgcn_sched_barrier(0);
    xl_quantize_tile<2>();
    __builtin_amdgcn_sched_barrier(0);
    xl_weights_for<3>();
    __builtin_amdgcn_sched_barrier(0);
    xl_quantize_tile<3>();
    stage_vectors();
    __syncthreads();
    read_bounds();
    v4f acc[kXlTiles][NT];
    float cs[kXlTiles];
    xl_mma(acc);
    // the per-column constants once, into the registers the weight held
    // (reading them from LDS at every tile made the epilogue LDS-bound).
    // The rowwise recipe leaves the tiles' epilogues to the scheduler to
    // interleave (independent chains: 0.15 us less per launch than with a
    // scheduling barrier after each tile); the tensor and MX recipes keep one
    // tile at a time, which they need to stay within their registers.
    constexpr bool ONE_AT_A_TIME = MODE != 1;
    const ColSB sb = col_sb();
#pragma unroll
    for (int i = 0; i < kXlTiles; ++i) {
      if (i < nt) epilogue_stats(i, acc[i], cs[i], sb);
      if constexpr (ONE_AT_A_TIME) __builtin_amdgcn_sched_barrier(0);
    }
    const ColGB gbv = col_gb();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kXlTiles; ++i) {
      if (i < nt) epilogue_out(i, tb + i, acc[i], cs[i], gbv);
      if constexpr (ONE_AT_A_TIME) __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ void run() {
    if constexpr (B2) {
      static_assert(MODE == 1, "B2 serves the rowwise recipe");
      run_b2();
      return;
    }
    if (tb >= te) return;
    if (OPT && MODE == 0 && p.sx_out != nullptr && tb == 0 && tid == 0) static_cast<float*>(p.sx_out)[0] = p.x_s;
    // every request first, in the order they are needed (load completions
    // are counted in issue order): X tile 0 (HBM), the column vectors, the
    // weight slice (L2-resident after its first reader), then the next X
    // tiles; the scheduling barrier keeps the first wait (tile 0's
    // quantization) from being hoisted above any of them
    load_x<0>(tb);
    request_vectors();
    request_weights();
    prologue_loads(std::make_integer_sequence<int, D - 1>{});
    __builtin_amdgcn_sched_barrier(0);
    quantize<0>(tb, 0);
    load_x<0>(tb + D);
    stage_vectors();
    __syncthreads();
    read_bounds();
    if (!PIPE) {
      for (int64_t j = 0; j < te - tb; ++j) step_seq(j);
      if (COOP) {
        __syncthreads();
        coop_store(te - 1);
      }
      return;
    }
    // tile 0: GEMM alongside the quantization of tile 1
    mma(0, acc0);
    quantize<(1 % D)>(tb + 1, 1);
    if (FULL && !OPT) interleave_hint();
    load_x<(1 % D)>(tb + 1 + D);
    epilogue_stats(0, acc0, cs0);
    __syncthreads();
    const int64_t n = te - tb;
    // Step j quantizes tile j+1 from slot (j+1) % D and fills accumulator
    // set j % 2.  The loop runs whole groups of steps (one period of the
    // slot and set pattern) with no exit in between, then a tail of the
    // remaining steps: an exit between the steps of the loop body would give
    // the loop header a path on which the X loads just issued are the
    // latest memory operations, and every iteration would then wait for them.
    // Step j uses slot (j + 1) % D and set j % 2; a group of D steps starting
    // at j = 1 + D i runs step m with slot (m + 2) % D and set (m + 1) % 2.
    int64_t j = 1;
    for (int64_t i = (n - 1) / D; i > 0; --i, j += D) step_group(j, std::make_integer_sequence<int, D>{});
    step_tail(j, n, std::make_integer_sequence<int, D - 1>{});
    // the last tile's normalization and stores
    const int64_t l = n - 1;
    if (l & 1) epilogue_out(1, tb + l, acc1, cs1);
    else epilogue_out(0, tb + l, acc0, cs0);
  }
};

}  // namespace fwd
}  // namespace loka
