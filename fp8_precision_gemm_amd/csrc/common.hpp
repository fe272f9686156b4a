// Device helpers shared by the gfx950 kernels of liblokafp8: bf16 and FP8
// conversions, scale arithmetic, wavefront reductions and the FP8 MFMA.
//
// Numerics (stated once; every kernel follows them):
//  * tensor/row/column scales: s = amax / FMAX and r = FMAX / amax, both IEEE
//    fp32 divisions (correctly rounded: the library is built without fast
//    math), r clamped to the largest finite fp32, amax == 0 -> s = r = 1.
//  * cast: t = x * r (one fp32 multiply), clamped to +-FMAX, then the
//    hardware RNE convert (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32).  The clamp
//    makes saturation explicit; the convert rounds to nearest even with
//    gradual underflow, which was checked bit for bit against exact
//    round-to-nearest-even on every bf16 value and the FP8 grid midpoints.
//  * MX32: E8M0 exponent e = clamp(floor(log2 amax) - emax_elem, -127, 127)
//    read from the fp32 exponent field (leading-zero count for subnormal
//    amax), as the GEM page's bit-manipulation scale derivation does;
//    x * 2^-e is one exact fp32 multiply.
//
// MFMA operand layout (v_mfma_scale_f32_16x16x128_f8f6f4): lane l supplies
// operand row (l % 16) and, with g = l / 16, the K bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of the 128-wide K chunk (the hardware's own K order,
// in which the E8M0 scale held by lane group G covers K block [32G, 32G+32)).
// The result lane l holds D[4*(l/16) + j][l % 16], j = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loka {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;
constexpr float kFltMax = 3.40282346638528859812e+38f;
// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle): loads at offsets past the record count return zeros.
constexpr int kBufferWord3 = 0x00020000;

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<0> {  // OCP e4m3
  static constexpr float fmax = kE4M3Max;
  static constexpr int emax_elem = 8;
};
template <>
struct Fp8Traits<1> {  // OCP e5m2
  static constexpr float fmax = kE5M2Max;
  static constexpr int emax_elem = 15;
};

__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two fp32 -> two FP8 codes (saturating RNE), in bits [0,16) of the result
// merged into `old` at word HI (false: bits 0-15, true: bits 16-31).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
  constexpr float m = Fp8Traits<FMT>::fmax;
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  if (FMT == 0) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  uint32_t lo = cvt_pk<FMT, false>(a, b, 0u);
  return cvt_pk<FMT, true>(c, d, lo);
}

struct ScalePair {
  float s;  // dequantization scale (stored)
  float r;  // quantization multiplier
};
// Branch-free: amax == 0 divides FMAX by itself, giving s = r = 1 exactly.
template <int FMT>
__device__ __forceinline__ ScalePair scales_from_amax(float amax) {
  const float a = amax == 0.0f ? Fp8Traits<FMT>::fmax : amax;
  ScalePair p;
  p.s = a / Fp8Traits<FMT>::fmax;
  p.r = fminf(Fp8Traits<FMT>::fmax / a, kFltMax);
  return p;
}

// E8M0 code of an fp32 block amax (>= 0, finite).
template <int FMT>
__device__ __forceinline__ int e8m0_from_amax(float amax) {
  uint32_t u = __float_as_uint(amax);
  if (u == 0u) return 0;
  int ef = (int)(u >> 23);
  int flog2 = ef != 0 ? ef - 127 : (31 - __clz((int)(u & 0x7FFFFFu))) - 149;
  int e = flog2 - Fp8Traits<FMT>::emax_elem;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e + 127;
}
// 2^-(code-127) as an fp32 multiplier; exact for every code an fp32 amax can
// produce (the exponent stays within [-119, 127]).
__device__ __forceinline__ float e8m0_inv_multiplier(int code) {
  int neg = 127 - code;  // -e
  return __uint_as_float((uint32_t)(neg + 127) << 23);
}

// DPP max of v with the value of another lane (dpp control CTRL); rows
// outside ROW_MASK keep their own value.  Only for non-negative values
// (amaxes, scales, +0): their fp32 order is the unsigned order of their
// bits, so the max is one v_max_u32 with the DPP operand folded in (an fp32
// max would first canonicalize the moved value).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_max(float v) {
  const uint32_t iv = __float_as_uint(v);
  // all rows written: bound_ctrl with the max identity 0 lets the move fold
  // into the max; rows masked off must keep their own value instead
  const uint32_t ov = ROW_MASK == 0xF ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)iv, CTRL, 0xF, 0xF, true)
                                      : (uint32_t)__builtin_amdgcn_update_dpp((int)iv, (int)iv, CTRL, ROW_MASK, 0xF, false);
  return __uint_as_float(iv > ov ? iv : ov);
}
// Max over each quad of lanes (4 consecutive lanes); non-negative values.
__device__ __forceinline__ float quad_max(float v) {
  v = dpp_max<0xB1>(v);  // quad_perm [1,0,3,2]
  return dpp_max<0x4E>(v);  // quad_perm [2,3,0,1]
}
// Max over the whole wavefront, returned uniformly (DPP within rows of 16,
// row broadcasts across rows, then lane 63 read back).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = quad_max(v);
  v = dpp_max<0x124>(v);        // row_ror:4
  v = dpp_max<0x128>(v);        // row_ror:8
  v = dpp_max<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the 16 lanes of each DPP row (lanes 16g .. 16g+15), returned in
// all of them: four rotate-and-add steps within the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, true));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, true));  // row_ror:1
  return v;
}
// Max over the 16 lanes of each DPP row; non-negative values.
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max<0x128>(v);
  v = dpp_max<0x124>(v);
  v = dpp_max<0x122>(v);
  return dpp_max<0x121>(v);
}
// Sum / max over the 4 lanes l, l^16, l^32, l^48 (one per DPP row),
// returned in all four: row swaps by v_permlane16_swap / v_permlane32_swap.
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float v) {  // non-negative values
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const uint32_t m = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return __uint_as_float(max((uint32_t)b[0], (uint32_t)b[1]));
}

// Wavefront (64-lane) reductions through LDS permutes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Reduction over the 4 lane groups that share l % 16 (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// FP8 MFMA, fp32 accumulate.  FA/FB: 0 = e4m3, 1 = e5m2 (the instruction's
// cbsz / blgp format selectors).  Scale operands 0 select the unscaled form.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}
// MX form: sa / sb are the E8M0 codes this lane supplies.
__device__ __forceinline__ v4f mfma_mx_e4m3(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Load one MFMA operand fragment: 16 bytes at p + 16g and 16 bytes at
// p + 64 + 16g, each half only when it lies below `limit` bytes (else 0).
__device__ __forceinline__ v8i load_frag(const uint8_t* p, int g, int kc, int limit) {
  v8i f;
  int o0 = kc + 16 * g, o1 = kc + 64 + 16 * g;
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (o0 < limit) a = *reinterpret_cast<const uint4*>(p + o0);
  if (o1 < limit) b = *reinterpret_cast<const uint4*>(p + o1);
  f[0] = (int)a.x; f[1] = (int)a.y; f[2] = (int)a.z; f[3] = (int)a.w;
  f[4] = (int)b.x; f[5] = (int)b.y; f[6] = (int)b.z; f[7] = (int)b.w;
  return f;
}

// Fragment-interleaved layout of an [R][C] byte matrix (R a multiple of 16,
// C padded with zeros to a multiple of 128), internal to the backward: the
// 16 x 128 block (R/16, C/128) is 2 KiB holding its eight 16-byte column
// pieces one after another, each piece being the 16 rows' bytes side by
// side.  An MFMA operand fragment (lane (r, g) reading pieces g and g+4 of
// row r) then reads 256 contiguous bytes per 16 lanes instead of 16 scattered
// rows.
__host__ __device__ inline size_t ilv_offset(int64_t row, int64_t col, int64_t nch) {
  return ((size_t)((row >> 4) * nch + (col >> 7)) * 8 + (size_t)((col & 127) >> 4)) * 256 + (size_t)(row & 15) * 16 +
         (size_t)(col & 15);
}
// Fragment of row tile rt (rows 16 rt .. +16), 128-column chunk c.
__device__ __forceinline__ v8i load_frag_ilv(const uint8_t* base, int64_t rt, int64_t c, int64_t nch, int r, int g) {
  const uint8_t* b = base + (size_t)(rt * nch + c) * 2048 + r * 16;
  const uint4 x = *reinterpret_cast<const uint4*>(b + g * 256);
  const uint4 y = *reinterpret_cast<const uint4*>(b + (4 + g) * 256);
  v8i f;
  f[0] = (int)x.x; f[1] = (int)x.y; f[2] = (int)x.z; f[3] = (int)x.w;
  f[4] = (int)y.x; f[5] = (int)y.y; f[6] = (int)y.z; f[7] = (int)y.w;
  return f;
}

}  // namespace loka
