"""Exact encoders and decoders for the number formats the block uses.

Test infrastructure only (see the package docstring).

Formats (the pages name them; their definitions are the OCP ones):
  * FP8 e4m3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 fraction bits,
    no infinities, S.1111.111 is NaN, largest finite 448 = 0x7E.
  * FP8 e5m2: 1 sign, 5 exponent bits (bias 15), 2 fraction bits,
    IEEE-style infinities, largest finite 57344 = 0x7B.
    [LoKA] section II-C and [GEM] "Mixed Ultra-Low-Precision Training" name
    FP8 as the target precision; e4m3 carries activations and weights, e5m2
    the gradients.
  * E8M0: the MX block scale, an 8-bit biased exponent (bias 127), value
    2**(code-127), code 255 = NaN ([GEM] "Low Precision Flash Attention":
    scales generated along each GEMM's K dimension; MX v1.0).
  * bf16: the activations' storage format.

Rounding is round-to-nearest, ties-to-even (RNE) on the exact value, done in
float64 where every step below is exact: a value in [2**e, 2**(e+1)) divided
by its quantum 2**(e - mbits) lies below 2**(mbits+1), so np.rint (which
rounds halves to even) applies RNE exactly.
"""

import numpy as np


class Fp8Format:
    """Parameters of one OCP FP8 format."""

    def __init__(self, name, ebits, mbits, bias, fmax, has_inf, emax_elem):
        self.name = name
        self.ebits = ebits
        self.mbits = mbits
        self.bias = bias
        self.fmax = float(fmax)
        self.has_inf = has_inf
        # exponent of the largest power of two not above fmax: the MX
        # "emax_elem" of the element format (8 for e4m3, 15 for e5m2)
        self.emax_elem = emax_elem

    @property
    def emin(self):
        """Exponent of the smallest normal number (1 - bias)."""
        return 1 - self.bias

    def __repr__(self):
        return f"Fp8Format({self.name})"


E4M3 = Fp8Format("e4m3", ebits=4, mbits=3, bias=7, fmax=448.0, has_inf=False, emax_elem=8)
E5M2 = Fp8Format("e5m2", ebits=5, mbits=2, bias=15, fmax=57344.0, has_inf=True, emax_elem=15)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}

BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bf16


def round_rne_grid(a, mbits, emin):
    """Round non-negative float64 values to the nearest point (ties to even)
    of the binary floating-point grid with `mbits` fraction bits whose
    exponent never goes below `emin` (spacing 2**(emin-mbits) below 2**emin,
    i.e. gradual underflow).  The grid has no upper bound here: saturation
    and overflow are the callers' business."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)  # a = f * 2**e with f in [0.5, 1)  => floor(log2 a) = e - 1
    expo = np.maximum(e - 1, emin)
    quantum = np.ldexp(1.0, expo - mbits)
    return np.rint(a / quantum) * quantum


def encode_fp8(t, fmt):
    """Saturating RNE encode of float64 values to FP8 codes (uint8).

    Finite values beyond +-fmax saturate to the +-fmax code; -0 keeps its
    sign (0x80).  NaN encodes as 0x7F / 0xFF.  Infinities saturate like any
    other out-of-range value (the method never produces them)."""
    t = np.asarray(t, dtype=np.float64)
    sign = np.signbit(t).astype(np.uint8)
    nan = np.isnan(t)
    a = np.where(nan, 0.0, np.minimum(np.abs(t), fmt.fmax))
    q = round_rne_grid(a, fmt.mbits, fmt.emin)
    # q is on the grid and 0 <= q <= fmax
    min_normal = np.ldexp(1.0, fmt.emin)
    sub = q < min_normal
    _, e = np.frexp(np.where(sub, 1.0, q))
    e = e - 1  # floor(log2 q) for normal q
    exp_field = np.where(sub, 0, e + fmt.bias)
    frac = np.where(
        sub,
        q / np.ldexp(1.0, fmt.emin - fmt.mbits),
        (q / np.ldexp(1.0, e) - 1.0) * (1 << fmt.mbits),
    )
    code = (sign.astype(np.int64) << 7) | (exp_field.astype(np.int64) << fmt.mbits) | frac.astype(np.int64)
    code = np.where(nan, 0x7F | (sign.astype(np.int64) << 7), code)
    return code.astype(np.uint8)


def decode_fp8(code, fmt):
    """Exact float64 value of FP8 codes (NaN codes -> nan, e5m2 inf codes -> inf).

    The 256 values are computed once from the field definitions below and
    then looked up."""
    table = _decode_table.get(fmt.name)
    if table is None:
        table = _decode_table[fmt.name] = _decode_fields(np.arange(256), fmt)
    return table[np.asarray(code, dtype=np.uint8)]


_decode_table = {}


def _decode_fields(code, fmt):
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    emask = (1 << fmt.ebits) - 1
    mmask = (1 << fmt.mbits) - 1
    E = (c >> fmt.mbits) & emask
    m = c & mmask
    sub = np.ldexp(m.astype(np.float64), fmt.emin - fmt.mbits)
    nrm = np.ldexp(1.0 + m / float(1 << fmt.mbits), (E - fmt.bias).astype(np.int64))
    v = sign * np.where(E == 0, sub, nrm)
    if fmt.has_inf:
        v = np.where((E == emask) & (m == 0), sign * np.inf, v)
        v = np.where((E == emask) & (m != 0), np.nan, v)
    else:
        v = np.where((E == emask) & (m == mmask), np.nan, v)
    return v


def fp8_grid(fmt):
    """All finite non-negative values of the format, ascending, with codes."""
    codes = np.arange(0, 0x80, dtype=np.uint8)
    vals = decode_fp8(codes, fmt)
    ok = np.isfinite(vals)
    return vals[ok], codes[ok]


def decode_e8m0(code):
    """Exact value 2**(code-127) of E8M0 scale codes (255 -> nan)."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def bf16_to_f64(bits):
    """Exact float64 value of bf16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """Round float64 values to bf16 bit patterns, RNE, in one rounding
    (overflow -> inf as IEEE requires, NaN -> 0x7FC0)."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    sign = np.signbit(v)
    a = np.where(nan, 0.0, np.abs(v))
    q = round_rne_grid(a, 7, -126)
    q = np.where(q > BF16_MAX, np.inf, q)
    q = np.where(sign, -q, q)
    bits = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)


def f32(v):
    """Round to the nearest fp32 (RNE): the precision the method's scale and
    product steps are defined in."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)
