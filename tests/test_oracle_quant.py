"""Pins for the oracle's amax / scale / cast steps (CPU only).

Pinned against: the hand-worked scale table (tests/golden/scale_pins.txt),
correctly rounded fp32 division checked with exact rationals, and
invariants every correct scaled quantizer must satisfy whatever its code
(the group maximum lands on the +-FMAX code, the per-element error bound,
power-of-two rescaling invariance).  A wrong reduction axis, a swapped s/r,
a missing saturation or a wrong MX exponent each break one of them.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, quant
from synth.workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(s):
    return float.fromhex(s) if "0x" in s else float(s)


def _pins():
    rows = []
    with open(os.path.join(GOLDEN, "scale_pins.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.mark.parametrize("row", _pins(), ids=lambda r: "-".join(r[:3]))
def test_scale_pins(row):
    kind, fmt = row[0], codec.FORMATS[row[1]]
    amax = _num(row[2])
    if kind == "sr":
        s, r = quant.scales_from_amax(np.array([amax]), fmt)
        es = _num(row[3].split("=")[1])
        er = _num(row[4].split("=")[1])
        assert float(s[0]) == es and float(r[0]) == er
    elif kind == "mx":
        assert int(quant.mx_exponent(np.array([amax]), fmt)[0]) == int(row[3], 16)
    elif kind == "mxel":
        elem = _num(row[3])
        e = int(quant.mx_exponent(np.array([amax]), fmt)[0]) - 127
        code = codec.encode_fp8(np.ldexp(np.array([elem]), -e), fmt)[0]
        assert int(code) == int(row[4], 16)


def _nearest_f32(fr):
    """Correctly rounded fp32 of an exact rational, by exact comparison of
    the neighbouring fp32 candidates (ties -> even significand)."""
    c = np.float32(float(fr))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for v in cands:
        d = abs(Fraction(float(v)) - fr)
        key = (d, int(np.array(v, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


@pytest.mark.parametrize("f", [codec.E4M3, codec.E5M2], ids=lambda f: f.name)
def test_scales_are_correctly_rounded_divisions(f):
    """Every positive finite bf16 amax (normals and subnormals): s and r are
    the correctly rounded fp32 quotients, r saturating at the largest fp32."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)          # positive finite bf16
    am = codec.bf16_to_f64(bits)
    s, r = quant.scales_from_amax(am, f)
    flt_max = np.float32(np.finfo(np.float32).max)
    idx = np.unique(np.concatenate([np.arange(0, len(am), 37), [0, 1, len(am) - 1]]))
    for i in idx:
        a = Fraction(am[i])
        assert s[i] == _nearest_f32(a / Fraction(f.fmax)), (am[i], s[i])
        rq = Fraction(f.fmax) / a
        if rq >= Fraction(float(flt_max)) * (1 + Fraction(1, 1 << 25)):
            assert r[i] == flt_max
        else:
            assert r[i] == _nearest_f32(rq), (am[i], r[i])


def _random_bits(shape, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    if spread:  # rows and columns with very different magnitudes
        x *= np.exp(2 * rng.standard_normal(shape[0]))[:, None]
        x *= np.exp(2 * rng.standard_normal(shape[1]))[None, :]
    return to_bf16_bits(x)


def _groups(mode, R, C):
    """Index arrays of every scaling group (independent of the oracle)."""
    if mode == quant.TENSOR:
        yield (slice(None), slice(None)), 0
    elif mode == quant.ROW:
        for i in range(R):
            yield (slice(i, i + 1), slice(None)), i
    elif mode == quant.COL:
        for j in range(C):
            yield (slice(None), slice(j, j + 1)), j
    elif mode == quant.MX32_ROW:
        for i in range(R):
            for b in range(C // 32):
                yield (slice(i, i + 1), slice(32 * b, 32 * b + 32)), (i, b)
    elif mode == quant.MX32_COL:
        for j in range(C):
            for b in range(R // 32):
                yield (slice(32 * b, 32 * b + 32), slice(j, j + 1)), (j, b)


@pytest.mark.parametrize("mode", quant.MODES)
@pytest.mark.parametrize("f", [codec.E4M3, codec.E5M2], ids=lambda f: f.name)
def test_group_invariants(mode, f):
    """For every group: the element of largest magnitude encodes to the
    format's extreme magnitude (tensor/row/col: exactly +-FMAX; MX: an
    exponent-8 (e4m3) / exponent-15 (e5m2) code), no code exceeds FMAX, and
    every element's dequantized value is within half an FP8 spacing of x
    (relative to the scale)."""
    R, C = 64, 96
    x = codec.bf16_to_f64(_random_bits((R, C), 5))
    codes, sc = quant.quantize(x, mode, f)
    deq = quant.dequantize(codes, sc, mode, f)
    dec = codec.decode_fp8(codes, f)
    assert np.all(np.abs(dec) <= f.fmax)
    vals, _ = codec.fp8_grid(f)
    for (ri, ci), key in _groups(mode, R, C):
        gx = x[ri, ci]
        gd = dec[ri, ci]
        i = np.unravel_index(np.argmax(np.abs(gx)), gx.shape)
        if mode in (quant.TENSOR, quant.ROW, quant.COL):
            assert abs(gd[i]) == f.fmax
            s = float(sc[key] if mode != quant.TENSOR else sc[0])
        else:
            e8 = int(sc[key])
            assert 2.0 ** f.emax_elem <= abs(gd[i]) <= f.fmax
            s = 2.0 ** (e8 - 127)
        # error bound: |deq - x| <= s * (half the spacing at |x/s|) + fp32 rounding of x*r
        t = np.abs(gx) / s
        j = np.clip(np.searchsorted(vals, np.minimum(t, f.fmax)), 1, len(vals) - 1)
        half_gap = (vals[j] - vals[j - 1]) / 2
        # MX only: a block maximum in (448, 512) * 2**e clips to 448 (the
        # known MX clipping), which adds (t - FMAX) * s
        clip = np.maximum(t - f.fmax, 0.0)
        bound = s * (half_gap + clip) * (1 + 2.0 ** -20) + np.abs(gx) * 2.0 ** -23
        assert np.all(np.abs(deq[ri, ci] - gx) <= bound)


def test_power_of_two_row_rescaling():
    """Scaling a row by 2**j leaves its codes unchanged and scales s by 2**j
    exactly (row mode), for every fp8 format."""
    x = codec.bf16_to_f64(_random_bits((32, 64), 7))
    j = np.arange(-6, 26, dtype=np.int64)
    x2 = np.ldexp(x, j[:, None])
    for f in (codec.E4M3, codec.E5M2):
        c1, s1 = quant.quantize(x, quant.ROW, f)
        c2, s2 = quant.quantize(x2, quant.ROW, f)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(np.ldexp(s1.astype(np.float64), j), s2.astype(np.float64))
        m1, e1 = quant.quantize(x, quant.MX32_ROW, f)
        m2, e2 = quant.quantize(x2, quant.MX32_ROW, f)
        np.testing.assert_array_equal(m1, m2)
        np.testing.assert_array_equal(e1.astype(np.int64) + j[:, None], e2.astype(np.int64))


def test_zero_groups_and_signed_zero():
    x = np.zeros((64, 64))
    x[1, 3] = -0.0
    x[2] = -0.0
    for mode in quant.MODES:
        codes, sc = quant.quantize(x, mode, codec.E4M3)
        assert set(np.unique(codes).tolist()) <= {0x00, 0x80}
        assert codes[2, 5] == 0x80
        if mode in (quant.TENSOR, quant.ROW, quant.COL):
            assert np.all(sc == 1.0)
        else:
            assert np.all(sc == 0)


def test_lossless_when_on_grid():
    """Rows drawn from the e4m3 grid with row amax 448 * 2**j quantize
    losslessly under ROW scaling: dequant(q(x)) == x exactly."""
    rng = np.random.default_rng(11)
    vals, _ = codec.fp8_grid(codec.E4M3)
    R, C = 16, 64
    x = rng.choice(np.concatenate([vals, -vals]), size=(R, C))
    x[:, 0] = 448.0
    j = rng.integers(-20, 20, size=R)
    x = np.ldexp(x, j[:, None])
    codes, s = quant.quantize(x, quant.ROW, codec.E4M3)
    np.testing.assert_array_equal(quant.dequantize(codes, s, quant.ROW, codec.E4M3), x)
