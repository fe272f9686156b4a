"""Pins of the oracle's square-block recipe ([GEM] "Low Precision Flash
Attention", Block-wise Quantization: one scale per 32 x 32 block, so the
quantization is transpose-invariant and each tensor is quantized once).

Each pin checks the oracle against something its square-block code does not
compute itself:
  * the transpose invariance the pages give as the point of the recipe;
  * reduction to the 1 x 32 MX modes (pinned on their own in
    test_oracle_quant.py) when the rows, or the columns, of every block
    repeat;
  * independence of the blocks, and closed-form scales of one-element blocks;
  * exactly representable inputs (FP8 grid values times one power of two
    per block), for which the dequantized forward and backward must equal
    plain fp64 products of the inputs -- a transposed scale index or a
    swapped operand fails these, since the powers differ from block to block;
  * the RNE half-spacing bound of the element format.
A wrong block shape or axis, a dropped scaling or an off-by-one exponent
fails one of them."""

import numpy as np
import pytest
import torch

from oracle import backward, codec, forward, quant
from oracle.codec import E4M3, E5M2, bf16_to_f64

SQ = quant.MX32_SQ


def _f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_transpose_invariant(fmt):
    rng = np.random.default_rng(1)
    x = _f32(rng, (96, 160)) * np.exp(rng.standard_normal((96, 1)))
    q, s = quant.quantize(x, SQ, fmt)
    qt, st = quant.quantize(x.T, SQ, fmt)
    np.testing.assert_array_equal(qt, q.T)
    np.testing.assert_array_equal(st, s.T)
    np.testing.assert_array_equal(quant.dequantize(qt, st, SQ, fmt), quant.dequantize(q, s, SQ, fmt).T)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_reduces_to_mx32_rows_and_columns(fmt):
    rng = np.random.default_rng(2)
    v = _f32(rng, (3, 128), 3.0)
    x = np.repeat(v, 32, axis=0)                    # every block's 32 rows equal
    q, s = quant.quantize(x, SQ, fmt)
    qr, sr = quant.quantize(v, quant.MX32_ROW, fmt)
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(q, np.repeat(qr, 32, axis=0))
    c = _f32(rng, (128, 2), 3.0)
    y = np.repeat(c, 32, axis=1)                    # every block's 32 columns equal
    q2, s2 = quant.quantize(y, SQ, fmt)
    qc, sc = quant.quantize(c, quant.MX32_COL, fmt)
    np.testing.assert_array_equal(s2, sc.T)
    np.testing.assert_array_equal(q2, np.repeat(qc, 32, axis=1))


def test_blocks_are_independent():
    rng = np.random.default_rng(3)
    x = _f32(rng, (64, 96))
    q, s = quant.quantize(x, SQ, E4M3)
    y = x.copy()
    y[32:64, 32:64] *= 1000.0
    q2, s2 = quant.quantize(y, SQ, E4M3)
    changed = np.zeros((2, 3), bool)
    changed[1, 1] = True
    np.testing.assert_array_equal(s2[~changed], s[~changed])
    assert s2[1, 1] != s[1, 1]
    mask = np.ones_like(q, bool)
    mask[32:64, 32:64] = False
    np.testing.assert_array_equal(q2[mask], q[mask])


@pytest.mark.parametrize("fmt,top,code", [(E4M3, 448.0, 0x7E), (E5M2, 57344.0, 0x7B)])
@pytest.mark.parametrize("j", [-20, -3, 0, 5])
def test_single_element_block_closed_form(fmt, top, code, j):
    # one nonzero element fmax * 2^j in an otherwise zero block: its exponent
    # is floor(log2 fmax) + j = emax_elem + j, so the scale is 2^j (E8M0
    # 127 + j) and the element encodes as fmax; the zero blocks get code 0
    x = np.zeros((64, 64))
    x[37, 5] = -top * 2.0 ** j
    q, s = quant.quantize(x, SQ, fmt)
    assert s[1, 0] == 127 + j and s[0, 0] == 0 and s[0, 1] == 0 and s[1, 1] == 0
    assert q[37, 5] == (code | 0x80)
    assert np.count_nonzero(q & 0x7F) == 1


def _exact_blocks(rng, R, C, fmt, lo, hi):
    """FP8 grid values times 2^j per 32 x 32 block (j in [lo, hi]), each
    block holding one element of the top binade so that its scale is 2^j."""
    vals, _ = codec.fp8_grid(fmt)
    vals = vals[vals > 0]
    top = vals[vals >= 2.0 ** fmt.emax_elem]
    g = rng.choice(vals, (R, C)) * rng.choice([-1.0, 1.0], (R, C))
    j = rng.integers(lo, hi + 1, (R // 32, C // 32))
    for a in range(R // 32):
        for b in range(C // 32):
            g[32 * a + rng.integers(32), 32 * b + rng.integers(32)] = rng.choice(top) * rng.choice([-1.0, 1.0])
    return g * np.exp2(np.repeat(np.repeat(j, 32, axis=0), 32, axis=1)), j


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_exact_inputs_round_trip(fmt):
    rng = np.random.default_rng(4)
    x, j = _exact_blocks(rng, 64, 128, fmt, -6, 6)
    q, s = quant.quantize(x, SQ, fmt)
    np.testing.assert_array_equal(s.astype(np.int64) - 127, j)
    np.testing.assert_array_equal(quant.dequantize(q, s, SQ, fmt), x)


def _bits(v):
    # exact: e4m3 / e5m2 grid values times powers of two are bf16 values
    b = codec.f64_to_bf16(v)
    assert np.array_equal(bf16_to_f64(b), v)
    return b


def test_forward_exact_inputs_equal_plain_product():
    rng = np.random.default_rng(5)
    M, K, N = 64, 96, 64
    x, _ = _exact_blocks(rng, M, K, E4M3, -4, 4)
    w, _ = _exact_blocks(rng, K, N, E4M3, -9, -5)
    f = forward.gemm_ln_forward(_bits(x), _bits(w), recipe="mx32_sq", eps=1e-5)
    np.testing.assert_array_equal(f["z"], x @ w)   # every partial sum is exact in fp64
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x @ w), (N,), eps=float(np.float32(1e-5)))
    np.testing.assert_allclose(f["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_exact_inputs_equal_plain_products():
    rng = np.random.default_rng(6)
    M, K, N = 96, 64, 128
    x, _ = _exact_blocks(rng, M, K, E4M3, -3, 3)
    w, _ = _exact_blocks(rng, K, N, E4M3, -9, -6)
    dy, _ = _exact_blocks(rng, M, N, E5M2, -20, -14)
    o = backward.gemm_ln_backward_sq(_bits(x), _bits(w), _bits(dy), no_ln=True)
    np.testing.assert_array_equal(o["dx"], dy @ w.T)
    np.testing.assert_array_equal(o["dw"], x.T @ dy)
    np.testing.assert_array_equal(o["dbias"], dy.sum(axis=0))
    # the codes the backward uses are the forward's: one quantization per tensor
    qx, sx = quant.quantize(x, SQ, E4M3)
    np.testing.assert_array_equal(o["q_x"], qx)
    np.testing.assert_array_equal(o["s_x"], sx)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_error_within_half_spacing(fmt):
    # RNE to a grid with m mantissa bits: |err| <= 2^-(m+1) * 2^floor(log2|t|)
    # for a scaled value t in the normal range of the format
    rng = np.random.default_rng(7)
    x = _f32(rng, (128, 128)) * np.exp(2 * rng.standard_normal((128, 1)))
    q, s = quant.quantize(x, SQ, fmt)
    d = quant.dequantize(q, s, SQ, fmt)
    sc = np.repeat(np.repeat(codec.decode_e8m0(s), 32, axis=0), 32, axis=1)
    t = np.abs(x) / sc
    normal = t >= 2.0 ** fmt.emin
    ulp_half = 2.0 ** (np.floor(np.log2(np.where(normal, t, 1.0))) - fmt.mbits - 1) * sc
    assert np.all(np.abs(d - x)[normal] <= ulp_half[normal])
    assert normal.mean() > 0.9


def test_layernorm_backward_square_matches_autograd():
    # the square recipe's dZ is the same LayerNorm backward, taken through
    # torch autograd on the oracle's own forward values
    rng = np.random.default_rng(8)
    M, K, N = 64, 64, 96
    xb = codec.f64_to_bf16(_f32(rng, (M, K)))
    wb = codec.f64_to_bf16(_f32(rng, (K, N), 1 / 8))
    dyb = codec.f64_to_bf16(_f32(rng, (M, N), 0.01))
    gb = codec.f64_to_bf16(1.0 + _f32(rng, (N,), 0.1))
    o = backward.gemm_ln_backward_sq(xb, wb, dyb, gamma_bits=gb)
    f = forward.gemm_ln_forward(xb, wb, gamma_bits=gb, recipe="mx32_sq")
    z = torch.from_numpy(f["z"]).requires_grad_(True)
    y = torch.nn.functional.layer_norm(z, (N,), weight=torch.from_numpy(bf16_to_f64(gb)),
                                       eps=float(np.float32(1e-5)))
    y.backward(torch.from_numpy(bf16_to_f64(dyb)))
    np.testing.assert_allclose(o["dz"], z.grad.numpy(), rtol=1e-9, atol=1e-12)
