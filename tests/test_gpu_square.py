"""The square-block MX32 recipe on the GPU against the oracle ([GEM] "Low
Precision Flash Attention", Block-wise Quantization: one E8M0 scale per
32 x 32 block, quantized once and read by every GEMM).

Forward: X and W quantized once with loka_quant_fp8(mode="mx32_sq") (codes
and scales bit-exact against the oracle), then loka_gemm_fp8_ln with
x_mode="mx32_sq" taking X's codes.  The full-size case is the benchmark's
16384 x 512 x 512 outlier workload with the packed weight; the oracle
computes sampled whole 32-row blocks (a block's codes depend only on its own
rows).  Z and Y use the forward tests' tolerances."""

import numpy as np
import pytest
import torch

from oracle import forward, quant
from oracle.codec import E4M3
from synth.workloads import forward_case, outlier_case
from tests.gpu_helpers import bf16_dev, check_y, check_z, host, row_sigma

pytestmark = pytest.mark.gpu


def sample_blocks(M, n, seed=0):
    """Row indices of the first and last 32-row blocks plus n seeded blocks."""
    nb = M // 32
    rng = np.random.default_rng(seed)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, size=min(n, nb), replace=False)]))
    return (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)


def run_square(lib, c, packed=True, no_bias=False):
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    qx, sx, _ = lib.loka_quant_fp8(x, fmt="e4m3", mode="mx32_sq")
    qw, sw, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="mx32_sq", transpose_out="packed" if packed else True)
    vec = dict(bias=None if no_bias else bf16_dev(c["bias"]), gamma=bf16_dev(c["gamma"]), beta=bf16_dev(c["beta"]))
    out = lib.loka_gemm_fp8_ln(qx, qw, sw, x_mode="mx32_sq", x_scales=sx, w_packed=packed, want_z=True,
                               want_stats=True, **vec)
    plain = lib.loka_gemm_fp8_ln(qx, qw, sw, x_mode="mx32_sq", x_scales=sx, w_packed=packed, **vec)
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    res["qx"], res["sx"], res["sw"] = host(qx), host(sx), host(sw)
    np.testing.assert_array_equal(host(plain["y"]), res["y"], err_msg="Y without the optional outputs")
    return res


def compare(g, c, rows, label, no_bias=False):
    xs = c["x"][rows]
    o = forward.gemm_ln_forward(xs, c["w"], None if no_bias else c["bias"], c["gamma"], c["beta"],
                                recipe="mx32_sq")
    np.testing.assert_array_equal(g["qx"][rows], o["qx"], err_msg=f"{label}: X codes")
    np.testing.assert_array_equal(g["sx"][rows[::32] // 32], o["sx"], err_msg=f"{label}: X scales")
    np.testing.assert_array_equal(g["sw"], o["sw"], err_msg=f"{label}: W scales")
    sigma = row_sigma(o["z"])
    ez = check_z(g["z"][rows], o["z"], sigma, label)
    ey = check_y(g["y"][rows], o["y"], label)
    np.testing.assert_allclose(g["mean"][rows], o["mean"], rtol=0, atol=1e-3 * sigma.max())
    np.testing.assert_allclose(g["rstd"][rows], o["rstd"], rtol=2e-3)
    print(f"{label}: Z err {ez:.2e}  Y max abs err {ey:.2e}")


def test_square_forward_full_size(lib):
    c = outlier_case()
    g = run_square(lib, c, packed=True)
    compare(g, c, sample_blocks(c["M"], 40), "square 16384x512x512")


@pytest.mark.parametrize("packed", [True, False])
# K = 512 with M % 16 == 0 takes the staged run (codes straight into LDS):
# (1024, 512, 512) one tile per workgroup, (2048, 512, 256) 256 columns,
# (12288, 512, 512) three tiles per workgroup
@pytest.mark.parametrize("M,K,N", [(96, 160, 192), (64, 1024, 128), (32, 64, 64), (320, 640, 384),
                                   (1024, 512, 512), (224, 96, 256), (2048, 512, 256), (12288, 512, 512)])
def test_square_forward_shapes(lib, M, K, N, packed):
    c = forward_case(M, K, N, seed=M + 3 * K + N, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    g = run_square(lib, c, packed=packed, no_bias=(M == 96))
    compare(g, c, np.arange(M), f"square {M}x{K}x{N}", no_bias=(M == 96))


def test_square_forward_rejects_unsupported(lib):
    from fp8_precision_gemm_amd import LokaError
    x = torch.zeros((48, 64), dtype=torch.uint8, device="cuda")
    qw = torch.zeros((64, 64), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((2, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises((LokaError, ValueError)):
        lib.loka_gemm_fp8_ln(x, qw, sw, x_mode="mx32_sq", x_scales=torch.zeros((1, 2), dtype=torch.uint8,
                                                                                  device="cuda"))


# ---- backward ---------------------------------------------------------------
# The square-block backward (flag LOKA_BWD_MX32_SQ) takes the forward's codes
# as they are and quantizes dZ once in 32 x 32 e5m2 blocks.  Literal reading
# (dY is dZ): the codes and block scales are bit-exact and dX, dW, dbias are
# checked to the backward tests' tolerances.  LayerNorm reading: the kernel's
# dZ is fp32 against the oracle's fp64, so a code within that error of an
# e5m2 midpoint (or a block whose max-abs is that close to a power of two) may
# round either way; those are masked and bounded as in test_gpu_backward.py.

from oracle import backward, codec  # noqa: E402
from tests.gpu_helpers import bf16_ulp  # noqa: E402
from tests.test_gpu_backward import ambiguous, check_colsum  # noqa: E402

TAU = 1e-3
MFMA_WINDOW = 2.0 ** -14
E5 = codec.E5M2


def run_square_bwd(lib, c, no_ln, fast_check=True):
    x, w, dy = bf16_dev(c["x"]), bf16_dev(c["w"]), bf16_dev(c["dy"])
    bias, gamma, beta = bf16_dev(c["bias"]), bf16_dev(c["gamma"]), bf16_dev(c["beta"])
    qx, sx, _ = lib.loka_quant_fp8(x, fmt="e4m3", mode="mx32_sq")
    qw, sw, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="mx32_sq", transpose_out=True)
    ctx = {"qx": qx, "sx": sx, "qw": qw, "sw": sw}
    if not no_ln:
        f = lib.loka_gemm_fp8_ln(qx, qw, sw, bias, gamma, beta, x_mode="mx32_sq", x_scales=sx, want_stats=True)
        ctx["mean"], ctx["rstd"] = f["mean"], f["rstd"]
    out = lib.loka_gemm_fp8_bwd(dy, None, None, None, ctx=ctx, bias=bias, gamma=gamma, no_ln=no_ln, want_dz=True,
                                want_dz_codes=True, square=True)
    fast = None
    if fast_check:  # without the optional outputs: the configuration the benchmark times
        fast = lib.loka_gemm_fp8_bwd(dy, None, None, None, ctx=ctx, bias=bias, gamma=gamma, no_ln=no_ln,
                                     square=True)
    packed = None
    if fast_check:  # the weights quantized straight into the packed layouts: no rearrangement in the call
        qwp, _, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="mx32_sq", transpose_out="packed")
        qwr, _, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode="mx32_sq", transpose_out="packed_rows")
        packed = lib.loka_gemm_fp8_bwd(dy, None, qwr, None, ctx=dict(ctx, qw=qwp), bias=bias, gamma=gamma,
                                       no_ln=no_ln, square=True, w_packed=True)
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    if fast is not None:
        for k in ("dx", "dw", "dbias"):
            np.testing.assert_array_equal(host(fast[k]), res[k], err_msg=f"{k} without the optional outputs")
    if packed is not None:
        for k in packed:
            np.testing.assert_array_equal(host(packed[k]), res[k], err_msg=f"{k} with packed weights")
    return res


def _deq(q, s, fmt):
    return quant.dequantize(q, s, quant.MX32_SQ, fmt)


def check_dx_sq(g, o, flip=None):
    dx = codec.bf16_to_f64(g["dx"])
    rms = np.sqrt((o["dx"] ** 2).mean(axis=1, keepdims=True))
    term = MFMA_WINDOW * (np.abs(_deq(o["q_dz"], o["s_dz"], E5)) @ np.abs(_deq(o["q_w"], o["s_w"], E4M3)).T)
    tol = 2 * bf16_ulp(o["dx"]) + 1e-3 * rms + term + (0 if flip is None else flip)
    err = np.abs(dx - o["dx"])
    assert np.all(err <= tol), f"dX: {int((err > tol).sum())} outside tolerance; worst {np.max(err / tol):.3f} x tol"
    return float(np.max(err / rms))


def check_dw_sq(g, o, flip=None):
    rms = np.sqrt((o["dw"] ** 2).mean())
    term = MFMA_WINDOW * (np.abs(_deq(o["q_x"], o["s_x"], E4M3)).T @ np.abs(_deq(o["q_dz"], o["s_dz"], E5)))
    tol = 1e-3 * rms + term + (0 if flip is None else flip)
    err = np.abs(g["dw"].astype(np.float64) - o["dw"])
    assert np.all(err <= tol), f"dW: worst {np.max(err / tol):.3f} x tol"
    return float(err.max() / rms)


def test_square_backward_literal_full_size(lib):
    c = outlier_case(dy=True)
    g = run_square_bwd(lib, c, no_ln=True)
    o = backward.gemm_ln_backward_sq(c["x"], c["w"], c["dy"], no_ln=True)
    np.testing.assert_array_equal(g["dz"], o["dz"].astype(np.float32))
    np.testing.assert_array_equal(g["dz_codes"], o["q_dz"])
    np.testing.assert_array_equal(g["dz_scales"], o["s_dz"])
    ex = check_dx_sq(g, o)
    ew = check_dw_sq(g, o)
    check_colsum(g["dbias"], o["dbias"], np.abs(codec.bf16_to_f64(c["dy"])).sum(axis=0), "dbias")
    print(f"square literal: dX err/rms {ex:.2e}  dW err/rms {ew:.2e}")


@pytest.mark.parametrize("M,K,N", [(16384, 512, 512), (1056, 192, 320), (64, 64, 64), (96, 512, 128),
                                   (160, 256, 448)])
def test_square_backward_layernorm(lib, M, K, N):
    if M == 16384:
        c = outlier_case(dy=True)
    else:
        c = forward_case(M, K, N, seed=M + 2 * K + N, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1,
                         dy_var=1e-3)
    g = run_square_bwd(lib, c, no_ln=False, fast_check=(M != 16384))
    o = backward.gemm_ln_backward_sq(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"])
    dz_ref = o["dz"]
    rms_row = np.sqrt((dz_ref ** 2).mean(axis=1, keepdims=True))
    dz_tol = TAU * np.maximum(np.abs(dz_ref), rms_row)
    dz_err = np.abs(g["dz"].astype(np.float64) - dz_ref)
    assert np.all(dz_err <= dz_tol), f"dZ: worst {np.max(dz_err / dz_tol):.3f} x tol"

    # the kernel's own fp32 dZ, quantized by the oracle in 32 x 32 blocks: the
    # same codes and scales, bit for bit
    q_own, s_own = quant.quantize(g["dz"].astype(np.float64), quant.MX32_SQ, E5)
    np.testing.assert_array_equal(g["dz_codes"], q_own)
    np.testing.assert_array_equal(g["dz_scales"], s_own)

    # against the fp64 dZ: block scales unique unless the block max-abs is
    # within the dZ error of a power of two
    am = quant.amax(dz_ref, quant.MX32_SQ)
    am_tol = quant.amax(dz_tol, quant.MX32_SQ)
    lo, hi = np.floor(np.log2(np.maximum(am - am_tol, 1e-300))), np.floor(np.log2(am + am_tol))
    amb_s = lo != hi
    sdiff = g["dz_scales"] != o["s_dz"]
    assert not np.any(sdiff & ~amb_s), f"{int((sdiff & ~amb_s).sum())} block scales differ away from a boundary"
    assert np.all(np.abs(g["dz_scales"].astype(int) - o["s_dz"].astype(int)) <= 1)
    # codes: unique away from midpoints within blocks of equal scale
    e_ref = np.repeat(np.repeat(codec.decode_e8m0(o["s_dz"]), 32, axis=0), 32, axis=1)
    t_ref = dz_ref / e_ref
    amb, gap = ambiguous(t_ref, (dz_tol + 2 * TAU * np.abs(dz_ref)) / e_ref)
    blk_amb = np.repeat(np.repeat(sdiff, 32, axis=0), 32, axis=1)
    differ = g["dz_codes"] != o["q_dz"]
    assert not np.any(differ & ~amb & ~blk_amb), f"{int((differ & ~amb & ~blk_amb).sum())} dZ codes differ"
    # bound of a flipped value (decoded difference), a flipped block: both scales' rounding
    flip_v = np.where(blk_amb, 0.5 * np.abs(dz_ref) + 2.0 * e_ref * gap, amb * gap * e_ref)
    wq = np.abs(_deq(o["q_w"], o["s_w"], E4M3))       # [K, N]
    xq = np.abs(_deq(o["q_x"], o["s_x"], E4M3))       # [M, K]
    ex = check_dx_sq(g, o, flip_v @ wq.T * (1 + 2 * TAU) + 2 * TAU * np.abs(o["dx"]))
    ew = check_dw_sq(g, o, xq.T @ flip_v * (1 + 2 * TAU) + 2 * TAU * np.abs(o["dw"]))
    dy = codec.bf16_to_f64(c["dy"])
    fwd = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe="mx32_sq")
    yhat = (fwd["z"] - fwd["mean"][:, None]) * fwd["rstd"][:, None]
    check_colsum(g["dgamma"], o["dgamma"], np.abs(dy * yhat).sum(axis=0), "dgamma")
    check_colsum(g["dbeta"], o["dbeta"], np.abs(dy).sum(axis=0), "dbeta")
    check_colsum(g["dbias"], o["dbias"], np.abs(dz_ref).sum(axis=0), "dbias")
    print(f"square LN {M}x{K}x{N}: dZ worst {np.max(dz_err / dz_tol):.3f} x tol, {int(differ.sum())} code flips "
          f"of {int(amb.sum())} ambiguous, {int(sdiff.sum())} scale flips; dX err/rms {ex:.2e}; dW err/rms {ew:.2e}")


def test_square_backward_rejects_unsupported(lib):
    from fp8_precision_gemm_amd import LokaError
    c = forward_case(64, 64, 640, seed=1, dy_var=1e-3)
    with pytest.raises(LokaError):  # N > 512 is outside the square-block backward
        run_square_bwd(lib, c, no_ln=True, fast_check=False)


# ---- Y leaving in 32 x 32 blocks (the next layer's square-block input) -------
# With want_y_square the LayerNorm epilogue also writes Y's e4m3 codes and
# E8M0 block scales.  They must be bit-identical to quantizing the stored Y
# with loka_quant_fp8 (the definition of the output), Y itself unchanged, and
# against the oracle (forward.square_quantized_output of the oracle's Y) the
# decoded values must agree within Y's tolerance plus one e4m3 spacing.

@pytest.mark.parametrize("x_mode,M,K,N", [("row", 16384, 512, 512), ("row", 96, 160, 256), ("tensor", 224, 256, 512),
                                          ("mx32_row", 64, 1024, 256), ("mx32_sq", 320, 512, 512)])
def test_fused_y_square_output(lib, x_mode, M, K, N):
    c = outlier_case() if M == 16384 else forward_case(M, K, N, seed=M + K, x_dist="student_t3_outliers",
                                                       gamma_var=0.1, beta_var=0.1)
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    wmode = {"row": "col", "tensor": "tensor", "mx32_row": "mx32_col", "mx32_sq": "mx32_sq"}[x_mode]
    qw, sw, _ = lib.loka_quant_fp8(w, mode=wmode, transpose_out="packed")
    vec = dict(bias=bf16_dev(c["bias"]), gamma=bf16_dev(c["gamma"]), beta=bf16_dev(c["beta"]), x_mode=x_mode,
               w_packed=True)
    xin = x
    if x_mode == "mx32_sq":
        xin, sx, _ = lib.loka_quant_fp8(x, mode="mx32_sq")
        vec["x_scales"] = sx
    out = lib.loka_gemm_fp8_ln(xin, qw, sw, want_y_square=True, **vec)
    plain = lib.loka_gemm_fp8_ln(xin, qw, sw, **vec)
    qy, sy, _ = lib.loka_quant_fp8(out["y"], mode="mx32_sq")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["y"]), host(plain["y"]), err_msg="Y changed")
    np.testing.assert_array_equal(host(out["y_codes"]), host(qy), err_msg="codes differ from quantizing Y")
    np.testing.assert_array_equal(host(out["y_scales"]), host(sy), err_msg="scales differ from quantizing Y")
    rows = sample_blocks(M, 24) if M == 16384 else np.arange(M)
    recipe = {"row": "row", "tensor": "tensor", "mx32_row": "mx32", "mx32_sq": "mx32_sq"}[x_mode]
    o = forward.gemm_ln_forward(c["x"][rows], c["w"], c["bias"], c["gamma"], c["beta"], recipe=recipe)
    qo, so = forward.square_quantized_output(o["y_bits"])
    got = quant.dequantize(host(out["y_codes"])[rows], host(out["y_scales"])[rows[::32] // 32], quant.MX32_SQ, E4M3)
    want = quant.dequantize(qo, so, quant.MX32_SQ, E4M3)
    blk = np.repeat(np.repeat(np.exp2(so.astype(np.float64) - 127), 32, axis=0), 32, axis=1)
    y_err = np.abs(codec.bf16_to_f64(host(out["y"])[rows]) - o["y"])
    # one e4m3 spacing at the value (relative 2^-3), the subnormal spacing of
    # the block (2^-9 of its scale) and the Y deviation, doubled for a scale
    # that may differ by one
    tol = 2 * (0.125 * np.abs(want) + 2.0 ** -9 * 448 * blk / 256 + y_err) + 1e-30
    assert np.all(np.abs(got - want) <= tol), f"worst {np.max(np.abs(got - want) / tol):.3f} x tol"


def test_fused_y_square_feeds_the_next_layer(lib):
    c1 = forward_case(256, 256, 512, seed=21, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    c2 = forward_case(256, 512, 256, seed=22, gamma_var=0.1, beta_var=0.1)
    qw1, sw1, _ = lib.loka_quant_fp8(bf16_dev(c1["w"]), mode="col", transpose_out="packed")
    l1 = lib.loka_gemm_fp8_ln(bf16_dev(c1["x"]), qw1, sw1, bf16_dev(c1["bias"]), bf16_dev(c1["gamma"]),
                              bf16_dev(c1["beta"]), w_packed=True, want_y_square=True)
    qw2, sw2, _ = lib.loka_quant_fp8(bf16_dev(c2["w"]), mode="mx32_sq", transpose_out="packed")
    vec2 = dict(bias=bf16_dev(c2["bias"]), gamma=bf16_dev(c2["gamma"]), beta=bf16_dev(c2["beta"]), x_mode="mx32_sq",
                w_packed=True)
    fused = lib.loka_gemm_fp8_ln(l1["y_codes"], qw2, sw2, x_scales=l1["y_scales"], **vec2)
    qy, sy, _ = lib.loka_quant_fp8(l1["y"], mode="mx32_sq")
    sep = lib.loka_gemm_fp8_ln(qy, qw2, sw2, x_scales=sy, **vec2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(fused["y"]), host(sep["y"]))


def test_fused_y_square_rejects_unsupported(lib):
    from fp8_precision_gemm_amd import LokaError
    c = forward_case(64, 128, 384, seed=2)
    qw, sw, _ = lib.loka_quant_fp8(bf16_dev(c["w"]), mode="col", transpose_out=True)
    with pytest.raises(LokaError):  # N = 384: not 256 or 512
        lib.loka_gemm_fp8_ln(bf16_dev(c["x"]), qw, sw, want_y_square=True)
