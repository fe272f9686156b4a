"""Pins for the oracle's FP8 / E8M0 / bf16 codec (CPU only).

Each check compares the oracle with something other than itself: the
hand-worked encodings in tests/golden/fp8_encodings.txt, a brute-force
nearest search over the format's full value list, PyTorch's own float8
conversion (after clamping, since PyTorch does not saturate), and exact
rational arithmetic.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_encodings():
    rows = []
    with open(os.path.join(GOLDEN, "fp8_encodings.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            fmt, val, code = line.split()[:3]
            rows.append((fmt, float.fromhex(val) if "0x" in val else float(val), int(code, 16)))
    return rows


@pytest.mark.parametrize("fmt,val,code", _golden_encodings())
def test_hand_worked_encodings(fmt, val, code):
    f = codec.FORMATS[fmt]
    got = int(codec.encode_fp8(np.array([val]), f)[0])
    assert got == code, f"{fmt} {val}: {got:#04x} != {code:#04x}"
    # and the code decodes back to the saturated, rounded value's sign/magnitude
    dec = codec.decode_fp8(np.array([code]), f)[0]
    assert np.signbit(dec) == np.signbit(val)


@pytest.mark.parametrize("f", [codec.E4M3, codec.E5M2], ids=lambda f: f.name)
def test_roundtrip_all_codes(f):
    codes = np.arange(256)
    vals = codec.decode_fp8(codes, f)
    finite = np.isfinite(vals)
    back = codec.encode_fp8(vals[finite], f)
    np.testing.assert_array_equal(back, codes[finite].astype(np.uint8))
    # count of finite codes: e4m3 has 2 NaN codes, e5m2 2 inf + 6 NaN
    assert finite.sum() == (254 if f is codec.E4M3 else 248)


def _brute_force_nearest(t, f):
    """Nearest finite grid value to each |t| (ties -> even code), by search."""
    vals, codes = codec.fp8_grid(f)
    a = np.minimum(np.abs(t), f.fmax)
    i = np.searchsorted(vals, a)           # vals[i-1] < a <= vals[i]
    i = np.clip(i, 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[i] % 2 == 0))
    pick_hi |= a == hi
    code = np.where(pick_hi, codes[i], codes[i - 1]).astype(np.int64)
    code |= np.signbit(t).astype(np.int64) << 7
    return code.astype(np.uint8)


@pytest.mark.parametrize("f", [codec.E4M3, codec.E5M2], ids=lambda f: f.name)
def test_encode_matches_brute_force_nearest(f):
    rng = np.random.default_rng(1)
    # every bf16 pattern (finite) times a spread of scales, plus grid midpoints
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_to_f64(bits)
    v = v[np.isfinite(v)]
    t = np.concatenate([v * 2.0 ** -100, v * 2.0 ** -120, v, rng.standard_normal(200000) * f.fmax / 3])
    t = t[np.isfinite(t)]
    vals, _ = codec.fp8_grid(f)
    mids = (vals[1:] + vals[:-1]) / 2
    t = np.concatenate([t, mids, -mids, vals, -vals])
    t = t.astype(np.float32).astype(np.float64)  # the cast is applied to fp32 values
    np.testing.assert_array_equal(codec.encode_fp8(t, f), _brute_force_nearest(t, f))


@pytest.mark.parametrize("f,tdt", [(codec.E4M3, torch.float8_e4m3fn), (codec.E5M2, torch.float8_e5m2)],
                         ids=["e4m3", "e5m2"])
def test_encode_matches_torch_after_clamp(f, tdt):
    """PyTorch's CPU float8 conversion rounds to nearest-even but does not
    saturate, so the library cross-check clamps to +-FMAX first."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_to_f64(bits)
    v = v[np.isfinite(v)]
    rng = np.random.default_rng(2)
    t = np.concatenate([v, v * f.fmax, rng.standard_normal(100000) * 300]).astype(np.float32)
    ref = torch.from_numpy(t).clamp(-f.fmax, f.fmax).to(tdt).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codec.encode_fp8(t.astype(np.float64), f), ref)


@pytest.mark.parametrize("f", [codec.E4M3, codec.E5M2], ids=lambda f: f.name)
def test_monotone_and_saturating(f):
    t = np.linspace(-2 * f.fmax, 2 * f.fmax, 200001)
    d = codec.decode_fp8(codec.encode_fp8(t, f), f)
    assert np.all(np.diff(d) >= 0)
    assert d.max() == f.fmax and d.min() == -f.fmax


def test_nan_encoding():
    assert codec.encode_fp8(np.array([np.nan]), codec.E4M3)[0] == 0x7F
    assert codec.encode_fp8(np.array([-np.nan]), codec.E4M3)[0] == 0xFF
    assert np.isnan(codec.decode_fp8(np.array([0x7F, 0xFF]), codec.E4M3)).all()
    assert np.isinf(codec.decode_fp8(np.array([0x7C, 0xFC]), codec.E5M2)).all()


def test_decode_exact_rationals():
    """Decode against exact rational field arithmetic for every code."""
    for f in (codec.E4M3, codec.E5M2):
        vals = codec.decode_fp8(np.arange(256), f)
        for c in range(256):
            s, e, m = c >> 7, (c >> f.mbits) & ((1 << f.ebits) - 1), c & ((1 << f.mbits) - 1)
            if not np.isfinite(vals[c]):
                continue
            if e == 0:
                exact = Fraction(m, 1 << f.mbits) * Fraction(2) ** (1 - f.bias)
            else:
                exact = (1 + Fraction(m, 1 << f.mbits)) * Fraction(2) ** (e - f.bias)
            assert Fraction(vals[c]) == (-exact if s else exact)


def test_e8m0_decode():
    v = codec.decode_e8m0(np.array([0, 1, 127, 128, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 1.0 and v[3] == 2.0 and v[4] == 2.0 ** 127
    assert np.isnan(v[5])


def test_bf16_roundtrip_and_rounding():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_to_f64(bits)
    fin = np.isfinite(v)
    np.testing.assert_array_equal(codec.f64_to_bf16(v[fin]), bits[fin])
    # fp32 values: PyTorch's fp32 -> bf16 conversion is a single RNE rounding
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e30]).astype(np.float32)
    # exact bf16 midpoints too
    mids = ((bits[fin][:-1].astype(np.uint32) << 16) + 0x8000).view(np.float32)
    x = np.concatenate([x, mids[np.isfinite(mids)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(codec.f64_to_bf16(x.astype(np.float64)), ref)


def test_bf16_single_rounding_from_f64():
    """A float64 value just above a bf16 midpoint must round up even though
    its fp32 rounding would land exactly on the midpoint (double rounding)."""
    one_plus_half_ulp = 1.0 + 2.0 ** -8          # the midpoint between 1 and 1+2^-7
    v = one_plus_half_ulp + 2.0 ** -40            # above it; fp32 rounds it back to the midpoint
    assert np.float32(v) == np.float32(one_plus_half_ulp)
    got = codec.bf16_to_f64(codec.f64_to_bf16(np.array([v])))[0]
    assert got == 1.0 + 2.0 ** -7
    assert codec.bf16_to_f64(codec.f64_to_bf16(np.array([one_plus_half_ulp])))[0] == 1.0  # tie -> even
