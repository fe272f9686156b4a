"""amax, scales and saturating RNE casts for every scaling mode.

Test infrastructure only (see the package docstring).

The pages fix the recipes but not their arithmetic:
  * tensorwise, rowwise and blockwise recipes -- [LoKA] section III-C
    (Dispatch chooses among library recipes "tensorwise, rowwise, blockwise");
  * block scales along each GEMM's K dimension, E8M0 power-of-two scales
    derived by bit manipulation, a max-abs reduction per block -- [GEM]
    "Low Precision Flash Attention" (scale factors along K; online
    P-to-MXFP8 conversion; block-wise quantization);
  * quantization overhead comes from both weights and activations --
    [GEM] "Mixed Ultra-Low-Precision Training".

Readings taken where the pages are silent (each is stated once here):
  R1  tensor/row/column scaling: amax is exact (max of |x| over the group,
      an fp32 value); the stored dequantization scale is s = RN32(amax/FMAX)
      and the quantization multiplier r = RN32(FMAX/amax), both correctly
      rounded fp32 divisions, r saturating to the largest finite fp32 when
      the quotient overflows; the code is satRNE_fp8(RN32(x*r)).  No margin,
      no power-of-two rounding of s.
  R2  amax == 0 gives s = r = 1; -0 encodes as 0x80; values past +-FMAX
      saturate to the +-FMAX code.
  R3  MX32: one E8M0 scale per 32 consecutive elements, exponent
      e = clamp(floor(log2 amax) - emax_elem, -127, 127) (the OCP MX v1.0
      rule), stored as e + 127, amax == 0 -> code 0; elements are
      satRNE_fp8(x * 2**-e), where the scaling is exact.
  R3b MX32 square blocks ([GEM] "Low Precision Flash Attention",
      Block-wise Quantization: one scale factor per 32 x 32 block, which
      makes the quantization transpose-invariant so each tensor is quantized
      once): the block is 32 consecutive rows by 32 consecutive columns; its
      scale is R3's E8M0 exponent of the block's max-abs, and every element
      is satRNE_fp8(x * 2**-e).  Scales are stored [R/32][C/32].
"""

import numpy as np

from .codec import encode_fp8, decode_fp8, decode_e8m0, f32

TENSOR, ROW, COL, MX32_ROW, MX32_COL = "tensor", "row", "col", "mx32_row", "mx32_col"
MX32_SQ = "mx32_sq"
MODES = (TENSOR, ROW, COL, MX32_ROW, MX32_COL, MX32_SQ)
FLT_MAX = np.float32(np.finfo(np.float32).max)


def amax(x, mode):
    """max |x| over each scaling group of a 2-D array x[R, C].

    tensor -> shape (1,); row -> (R,) (over each row); col -> (C,) (down each
    column); mx32_row -> (R, C/32) (32 consecutive elements along a row);
    mx32_col -> (C, R/32) (32 consecutive elements down a column);
    mx32_sq -> (R/32, C/32) (32 x 32 blocks)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    R, C = a.shape
    if mode == TENSOR:
        return np.array([a.max() if a.size else 0.0])
    if mode == ROW:
        return a.max(axis=1) if C else np.zeros(R)
    if mode == COL:
        return a.max(axis=0) if R else np.zeros(C)
    if mode == MX32_ROW:
        return a.reshape(R, C // 32, 32).max(axis=2)
    if mode == MX32_COL:
        return a.T.reshape(C, R // 32, 32).max(axis=2)
    if mode == MX32_SQ:
        return a.reshape(R // 32, 32, C // 32, 32).max(axis=(1, 3))
    raise ValueError(mode)


def scales_from_amax(am, fmt):
    """Reading R1/R2: (s, r) as fp32 arrays from an fp32-exact amax."""
    am32 = f32(am)
    fmax32 = np.float32(fmt.fmax)
    zero = am32 == 0
    safe = np.where(zero, np.float32(1), am32).astype(np.float32)
    with np.errstate(over="ignore", divide="ignore"):
        s = (safe / fmax32).astype(np.float32)   # correctly rounded fp32 division
        r = (fmax32 / safe).astype(np.float32)
    r = np.minimum(r, FLT_MAX).astype(np.float32)
    s = np.where(zero, np.float32(1), s).astype(np.float32)
    r = np.where(zero, np.float32(1), r).astype(np.float32)
    return s, r


def cast_scaled(x, r, fmt):
    """Reading R1: code = satRNE_fp8(RN32(x * r)).  x holds fp32-exact values
    and r fp32 values, so the float64 product is exact and one rounding to
    fp32 gives RN32(x*r)."""
    t = f32(np.asarray(x, dtype=np.float64) * np.asarray(r, dtype=np.float64))
    return encode_fp8(t.astype(np.float64), fmt)


def mx_exponent(am, fmt):
    """Reading R3: E8M0 code of each block amax (exponent-field arithmetic:
    floor(log2 amax) is the binary exponent of amax)."""
    am = np.asarray(am, dtype=np.float64)
    _, e = np.frexp(am)
    e = np.clip(e - 1 - fmt.emax_elem, -127, 127)
    return np.where(am == 0, 0, e + 127).astype(np.uint8)


def quantize(x, mode, fmt):
    """Quantize a 2-D array x[R, C] (fp32-exact values).

    Returns (codes[R, C] uint8, scales) where scales are the fp32 dequant
    scales s (tensor (1,), row (R,), col (C,)) or the E8M0 codes (mx32_row
    (R, C/32), mx32_col (C, R/32), mx32_sq (R/32, C/32))."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    am = amax(x, mode)
    if mode in (TENSOR, ROW, COL):
        s, r = scales_from_amax(am, fmt)
        if mode == TENSOR:
            rb = r[0]
        elif mode == ROW:
            rb = r[:, None]
        else:
            rb = r[None, :]
        return cast_scaled(x, rb, fmt), s
    e8 = mx_exponent(am, fmt)
    e = e8.astype(np.int64) - 127
    if mode == MX32_ROW:
        sh = np.repeat(-e, 32, axis=1)              # [R, C]
    elif mode == MX32_COL:
        sh = np.repeat(-e, 32, axis=1).T            # [C, R] -> [R, C]
    else:
        sh = np.repeat(np.repeat(-e, 32, axis=0), 32, axis=1)  # [R/32, C/32] -> [R, C]
    t = np.ldexp(x, sh)                              # exact power-of-two scaling
    return encode_fp8(t, fmt), e8


def dequantize(codes, scales, mode, fmt):
    """float64 values code * scale of quantize()'s output (exact)."""
    v = decode_fp8(codes, fmt)
    R, C = v.shape
    if mode == TENSOR:
        return v * np.float64(scales[0])
    if mode == ROW:
        return v * np.asarray(scales, np.float64)[:, None]
    if mode == COL:
        return v * np.asarray(scales, np.float64)[None, :]
    sc = decode_e8m0(scales)
    if mode == MX32_ROW:
        return v * np.repeat(sc, 32, axis=1)
    if mode == MX32_COL:
        return v * np.repeat(sc, 32, axis=1).T
    if mode == MX32_SQ:
        return v * np.repeat(np.repeat(sc, 32, axis=0), 32, axis=1)
    raise ValueError(mode)
