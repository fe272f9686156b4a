"""loka_gemm_fp8_bwd on the GPU against the oracle (training step on the
16384 x 512 x 512 outlier workload).

Literal reading (dY is dZ, no LayerNorm): dZ is an exact input, so the e5m2
codes and scales are bit-exact and dX, dW, dbias are checked to tolerance.

LayerNorm reading: the kernel computes dZ in fp32 and the oracle in fp64.
The e5m2 codes and scales must equal, bit for bit, the oracle quantizer run
on the kernel's own fp32 dZ (which the kernel writes).  Against the fp64 dZ,
a code whose exact value sits within the fp32 error of a rounding midpoint
may legitimately round either way: that comparison checks what is unique --
every code away from a midpoint must match -- and bounds dX and dW by the
tolerance plus, for each possibly-flipped code, one e5m2 spacing times its
weight (all bounds computed from oracle data only).

Tolerances:
  dZ (fp32):  |dz - dz_ref| <= TAU * max(|dz_ref|, rms_row(dz_ref)), TAU = 1e-3
  dX (bf16):  2 ulp_bf16 + 1e-3 * rms_row(dx_ref) + MFMA term (+ flip bound)
  dW (fp32):  1e-3 * rms(dw_ref) + MFMA term (+ flip bound)
  dgamma, dbeta, dbias (fp32 sums over 16384 rows): 1e-3 of sum |terms|
The MFMA term is 2^-14 * sum |a*b| over the contraction: the gfx950 FP8
MFMA adds its products in a fixed-point window about 13 bits below the
largest product of each group of 8 (measured: at most 2.3e-5 * sum |a*b|
per 128-deep instruction on random e4m3 codes), a known "fast accumulation"
error that grows with the contraction length (16384 rows for dW).
"""

import numpy as np
import pytest
import torch

from oracle import backward, codec, forward, quant
from synth.workloads import forward_case, outlier_case
from tests.gpu_helpers import bf16_dev, bf16_ulp, host, unpack_packed

pytestmark = pytest.mark.gpu

TAU = 1e-3
MFMA_WINDOW = 2.0 ** -14
E5 = codec.E5M2


def run_gpu(lib, c, no_ln, w_packed=False):
    """One backward call with every optional output; w_packed: both weights
    quantized straight into the fragment-interleaved layouts."""
    x, w, dy = bf16_dev(c["x"]), bf16_dev(c["w"]), bf16_dev(c["dy"])
    bias, gamma, beta = bf16_dev(c["bias"]), bf16_dev(c["gamma"]), bf16_dev(c["beta"])
    qw, sw, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="col", transpose_out=True)
    qwr, swr, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="row", transpose_out="packed_rows" if w_packed else False)
    ctx = None
    if not no_ln:
        f = lib.loka_gemm_fp8_ln(x, qw, sw, bias, gamma, beta, want_stats=True, want_qx=True)
        if w_packed:  # the backward's copy of the forward weight, packed (any N)
            qw, _, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="col", transpose_out="packed")
        ctx = {"qx": f["qx"], "sx": f["sx"], "mean": f["mean"], "rstd": f["rstd"], "qw": qw, "sw": sw}
    out = lib.loka_gemm_fp8_bwd(dy, x, qwr, swr, ctx=ctx, bias=bias, gamma=gamma, no_ln=no_ln, want_dz=True,
                                want_dz_codes=True, w_packed=w_packed, want_col_codes=True)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def check_col_codes(g, x_bits):
    """The wgrad operands, bit for bit: X's column codes and scales against
    the oracle quantizer on X; dZ's against the oracle quantizer on the
    kernel's own fp32 dZ (the precision the quantizer is defined on)."""
    M, K = x_bits.shape
    N = g["dz"].shape[1]
    q_x, s_x = quant.quantize(codec.bf16_to_f64(x_bits), quant.COL, codec.E4M3)
    np.testing.assert_array_equal(unpack_packed(g["xc_codes"], K, M).T, q_x)
    np.testing.assert_array_equal(g["xc_scales"].view(np.uint32), s_x.astype(np.float32).view(np.uint32))
    q_d, s_d = quant.quantize(g["dz"].astype(np.float64), quant.COL, E5)
    np.testing.assert_array_equal(unpack_packed(g["dzc_codes"], N, M).T, q_d)
    np.testing.assert_array_equal(g["dzc_scales"].view(np.uint32), s_d.astype(np.float32).view(np.uint32))


def spacing_e5m2(t):
    """Distance between the two e5m2 grid points around |t| (t in code units)."""
    vals, _ = codec.fp8_grid(E5)
    a = np.minimum(np.abs(t), E5.fmax)
    j = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    return vals[j] - vals[j - 1], (vals[j] + vals[j - 1]) / 2


def ambiguous(t_ref, width):
    """Elements whose code is not unique given the kernel's fp32 dZ: the
    exact scaled value lies within `width` of an e5m2 rounding midpoint, or
    within `width` of zero (the sign may differ).  Returns the mask and the
    largest difference of decoded codes each element may show."""
    gap, mid = spacing_e5m2(t_ref)
    near_mid = np.abs(np.abs(t_ref) - mid) <= width
    near_zero = np.abs(t_ref) <= width
    allowed = np.where(near_zero, 2 * (np.abs(t_ref) + width) + gap, gap)
    return near_mid | near_zero, allowed


def mfma_term_dx(o):
    dzq = np.abs(codec.decode_fp8(o["q_dz"], E5)) * o["s_dz"].astype(np.float64)[:, None]
    wq = np.abs(codec.decode_fp8(o["q_wr"], codec.E4M3)) * o["s_wr"].astype(np.float64)[:, None]
    return MFMA_WINDOW * (dzq @ wq.T)


def mfma_term_dw(o):
    xq = np.abs(codec.decode_fp8(o["q_xc"], codec.E4M3)) * o["s_xc"].astype(np.float64)[None, :]
    dzq = np.abs(codec.decode_fp8(o["q_dzc"], E5)) * o["s_dzc"].astype(np.float64)[None, :]
    return MFMA_WINDOW * (xq.T @ dzq)


def check_dx(g, o, dz_ref, x_w, flip_rows=None):
    dx = codec.bf16_to_f64(g["dx"])
    dx_ref = o["dx"]
    rms = np.sqrt((dx_ref ** 2).mean(axis=1, keepdims=True))
    tol = 2 * bf16_ulp(dx_ref) + 1e-3 * rms + mfma_term_dx(o)
    if flip_rows is not None:
        tol = tol + flip_rows
    err = np.abs(dx - dx_ref)
    bad = err > tol
    assert not bad.any(), f"dX: {int(bad.sum())} entries outside tolerance; worst {np.max(err / tol):.3f} x tol"
    return float(np.max(err / rms))


def check_dw(g, o, flip=None):
    dw = g["dw"].astype(np.float64)
    rms = np.sqrt((o["dw"] ** 2).mean())
    tol = 1e-3 * rms + mfma_term_dw(o) + (0 if flip is None else flip)
    err = np.abs(dw - o["dw"])
    assert np.all(err <= tol), f"dW: worst {np.max(err / tol):.3f} x tol"
    return float(err.max() / rms)


def check_colsum(got, ref, terms_abs, name):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= 1e-3 * terms_abs + 1e-30), f"{name}: worst {np.max(err / terms_abs):.3e}"


def test_literal_reading_full_size(lib):
    c = outlier_case(dy=True)
    g = run_gpu(lib, c, no_ln=True)
    o = backward.gemm_ln_backward(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"], no_ln=True)
    np.testing.assert_array_equal(g["dz"], o["dz"].astype(np.float32))
    np.testing.assert_array_equal(g["dz_codes"], o["q_dz"])
    np.testing.assert_array_equal(g["dz_scales"].view(np.uint32), o["s_dz"].astype(np.float32).view(np.uint32))
    # dZ = dY exactly: the column codes equal the oracle's wgrad operands too
    check_col_codes(g, c["x"])
    np.testing.assert_array_equal(unpack_packed(g["dzc_codes"], c["N"], c["M"]).T, o["q_dzc"])
    ex = check_dx(g, o, o["dz"], None)
    ew = check_dw(g, o)
    dy = codec.bf16_to_f64(c["dy"])
    check_colsum(g["dbias"], o["dbias"], np.abs(dy).sum(axis=0), "dbias")
    print(f"literal: dX err/rms {ex:.2e}  dW err/rms {ew:.2e}")


@pytest.mark.parametrize("M,K,N", [(16384, 512, 512), (1040, 192, 320), (64, 64, 64), (144, 1024, 256), (96, 256, 1024)])
def test_layernorm_reading(lib, M, K, N):
    if M == 16384:
        c = outlier_case(dy=True)
    else:
        c = forward_case(M, K, N, seed=M + K, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1, dy_var=1e-3)
    g = run_gpu(lib, c, no_ln=False)
    o = backward.gemm_ln_backward(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"])
    dz_ref = o["dz"]
    rms_row = np.sqrt((dz_ref ** 2).mean(axis=1, keepdims=True))
    dz_tol = TAU * np.maximum(np.abs(dz_ref), rms_row)
    dz_err = np.abs(g["dz"].astype(np.float64) - dz_ref)
    assert np.all(dz_err <= dz_tol), f"dZ: worst {np.max(dz_err / dz_tol):.3f} x tol"

    # the dgrad operand is the quantization of the kernel's own fp32 dZ: the
    # oracle quantizer on that dZ must give the same codes and scales, bit for bit
    q_own, s_own = quant.quantize(g["dz"].astype(np.float64), quant.ROW, E5)
    np.testing.assert_array_equal(g["dz_codes"], q_own)
    np.testing.assert_array_equal(g["dz_scales"].view(np.uint32), s_own.astype(np.float32).view(np.uint32))
    check_col_codes(g, c["x"])

    # against the fp64 dZ: codes unique away from midpoints
    s_ref = o["s_dz"].astype(np.float64)
    np.testing.assert_allclose(g["dz_scales"], s_ref, rtol=2 * TAU)
    t_ref = dz_ref / s_ref[:, None]
    width = (dz_tol + np.abs(dz_ref) * 2 * TAU) / s_ref[:, None]
    amb, gap = ambiguous(t_ref, width)
    differ = g["dz_codes"] != o["q_dz"]
    assert not np.any(differ & ~amb), f"{int((differ & ~amb).sum())} dZ codes differ away from a midpoint"
    dec_g = codec.decode_fp8(g["dz_codes"], E5)
    dec_o = codec.decode_fp8(o["q_dz"], E5)
    assert np.all(np.abs(dec_g - dec_o)[differ] <= gap[differ] * (1 + 1e-12))
    # dX: flip bound per (m, k) = sum over ambiguous n of gap * s_dz * |w_q(k, n)| * s_w(k), plus scale drift
    wq = codec.decode_fp8(o["q_wr"], codec.E4M3) * o["s_wr"].astype(np.float64)[:, None]  # [K, N]
    flip = ((amb * gap) * s_ref[:, None]) @ np.abs(wq).T * (1 + 2 * TAU) + 2 * TAU * np.abs(o["dx"])
    ex = check_dx(g, o, dz_ref, None, flip_rows=flip)

    # wgrad: column codes of dZ are internal; bound their possible flips the same way
    dzc_s = o["s_dzc"].astype(np.float64)
    tcol = dz_ref / dzc_s[None, :]
    col_rms = np.sqrt((dz_ref ** 2).mean(axis=0, keepdims=True))
    wtol = (TAU * np.maximum(np.abs(dz_ref), np.maximum(rms_row, col_rms)) + np.abs(dz_ref) * 2 * TAU) / dzc_s[None, :]
    amb_c, gap_c = ambiguous(tcol, wtol)
    xq = codec.decode_fp8(o["q_xc"], codec.E4M3) * o["s_xc"].astype(np.float64)[None, :]  # [M, K]
    flip_w = np.abs(xq).T @ (amb_c * gap_c * dzc_s[None, :]) * (1 + 2 * TAU) + 2 * TAU * np.abs(o["dw"])
    ew = check_dw(g, o, flip_w)

    dy = codec.bf16_to_f64(c["dy"])
    fwd = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"])
    yhat = (fwd["z"] - fwd["mean"][:, None]) * fwd["rstd"][:, None]
    check_colsum(g["dgamma"], o["dgamma"], np.abs(dy * yhat).sum(axis=0), "dgamma")
    check_colsum(g["dbeta"], o["dbeta"], np.abs(dy).sum(axis=0), "dbeta")
    check_colsum(g["dbias"], o["dbias"], np.abs(dz_ref).sum(axis=0), "dbias")
    print(f"LN {M}x{K}x{N}: dZ worst {np.max(dz_err / dz_tol):.3f} x tol, {int(differ.sum())} row-code flips "
          f"of {int(amb.sum())} ambiguous; dX err/rms {ex:.2e}; dW err/rms {ew:.2e}")


@pytest.mark.parametrize("M,K,N", [(16384, 512, 512), (1040, 192, 320), (96, 256, 1024)])
def test_packed_weights_bit_identical(lib, M, K, N):
    """LOKA_BWD_W_PACKED (both weights quantized straight into the
    interleaved layouts) gives the same bits as the row-major call."""
    c = outlier_case(dy=True) if M == 16384 else forward_case(M, K, N, seed=M + N, x_dist="student_t3_outliers",
                                                               gamma_var=0.1, beta_var=0.1, dy_var=1e-3)
    a = run_gpu(lib, c, no_ln=False)
    b = run_gpu(lib, c, no_ln=False, w_packed=True)
    assert set(a) == set(b)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_backward_deterministic(lib):
    c = forward_case(2048, 256, 256, seed=3, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1, dy_var=1e-3)
    a = run_gpu(lib, c, no_ln=False)
    b = run_gpu(lib, c, no_ln=False)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
