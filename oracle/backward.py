"""Backward of the block (LayerNorm backward, e5m2 dZ, dgrad, wgrad), fp64.

Test infrastructure only (see the package docstring).

Sources:
  * [LoKA] section III-C (Trainer Integration): the low-precision linear is a
    drop-in for a standard Linear with its own autograd function routing the
    forward and the backward separately, so the backward is the exact
    gradient of the forward's definition;
  * [LoKA] section III-C and Table VI: rowwise recipes for the backward GEMMs
    (the "RW" recipe, with "RW GW HP" keeping wgrad in high precision as the
    alternative);
  * [GEM] "Mixed Ultra-Low-Precision Training": e5m2-range gradients,
    scale factors along each GEMM's own contraction (K) dimension.

Reading R8 (the training-step configuration names dY, dX = dY.W^T and
dW = X^T.dY "plus LayerNorm backward" without saying where the LayerNorm
sits): dY is the gradient at the LayerNorm output Y; the LayerNorm backward
turns it into dZ, the gradient at the GEMM output; dZ is what both GEMMs
consume.  Per row m, with yhat = (z - mu) * rstd and g = dY * gamma:
    dZ     = rstd * (g - mean_n g - yhat * mean_n (g * yhat))
    dgamma = sum_m dY * yhat,   dbeta = sum_m dY,   dbias = sum_m dZ
dZ is rounded to fp32 (the precision the quantizer is defined on) and:
  * dgrad: dX = dequant( q_row(dZ, e5m2) . q_row(W, e4m3)^T ), where the
    rows of W[K,N] are its k index, so W's scale is per k, amax over n;
  * wgrad: dW = dequant( q_col(X, e4m3)^T . q_col(dZ, e5m2) ), scales per
    column of X (per k) and of dZ (per n), amax over the M rows -- both
    operands scaled along the contraction;
  * dW stays fp32-or-wider (returned in fp64 here), dX is rounded to bf16.
The literal reading (dY already is dZ, no LayerNorm) is `no_ln=True`.

Square-block recipe ([GEM] "Low Precision Flash Attention", Block-wise
Quantization: 32 x 32 blocks make the quantization transpose-invariant, so
each tensor is quantized once and serves every GEMM that reads it):
X, W and dZ are each quantized once in 32 x 32 blocks (reading R3b; e4m3 for
X and W, e5m2 for dZ), the forward with those X and W codes, and
  * dgrad: dX = dequant(q_sq(dZ)) . dequant(q_sq(W))^T,
  * wgrad: dW = dequant(q_sq(X))^T . dequant(q_sq(dZ)),
with the same codes and scales the forward and dgrad used (no requantization
along the other dimension).
"""

import numpy as np

from .codec import E4M3, E5M2, bf16_to_f64, decode_fp8, f32, f64_to_bf16
from .forward import gemm_ln_forward, reference_forward, _vec
from .quant import quantize, dequantize, ROW, COL, MX32_SQ


def layernorm_backward(dy, z, mu, rstd, gamma):
    """Exact fp64 LayerNorm backward for y = gamma*(z-mu)*rstd + beta with
    rstd = 1/sqrt(var + eps): returns (dz, dgamma, dbeta)."""
    yhat = (z - mu[:, None]) * rstd[:, None]
    g = dy * gamma[None, :]
    mg = g.mean(axis=1)
    mgy = (g * yhat).mean(axis=1)
    dz = rstd[:, None] * (g - mg[:, None] - yhat * mgy[:, None])
    return dz, (dy * yhat).sum(axis=0), dy.sum(axis=0)


def dgrad(dz32, w):
    """dX = dequant(q_row(dZ) . q_row(W)^T): dz32 [M,N] fp32-exact, w [K,N]."""
    q_dz, s_dz = quantize(dz32, ROW, E5M2)
    q_w, s_w = quantize(w, ROW, E4M3)
    acc = decode_fp8(q_dz, E5M2) @ decode_fp8(q_w, E4M3).T
    dx = acc * np.asarray(s_dz, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :]
    return dx, q_dz, s_dz, q_w, s_w


def wgrad(x, dz32):
    """dW = dequant(q_col(X)^T . q_col(dZ)): x [M,K], dz32 [M,N]."""
    q_x, s_x = quantize(x, COL, E4M3)
    q_dz, s_dz = quantize(dz32, COL, E5M2)
    acc = decode_fp8(q_x, E4M3).T @ decode_fp8(q_dz, E5M2)
    dw = acc * np.asarray(s_x, np.float64)[:, None] * np.asarray(s_dz, np.float64)[None, :]
    return dw, q_x, s_x, q_dz, s_dz


def gemm_ln_backward(x_bits, w_bits, dy_bits, bias_bits=None, gamma_bits=None, beta_bits=None,
                     eps=1e-5, no_ln=False):
    """Backward of the rowwise-recipe forward for bf16 inputs.

    Returns a dict with dz (fp64), dz32 (its fp32 rounding), the e5m2 row
    codes/scales of dz32, dx (fp64) and dx_bits (bf16), dw (fp64), dgamma,
    dbeta, dbias (fp64; dgamma/dbeta are None when no_ln)."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    dy = bf16_to_f64(dy_bits)
    N = w.shape[1]
    if no_ln:
        dz, dgamma, dbeta = dy, None, None
    else:
        fwd = gemm_ln_forward(x_bits, w_bits, bias_bits, gamma_bits, beta_bits, eps, recipe="row")
        dz, dgamma, dbeta = layernorm_backward(dy, fwd["z"], fwd["mean"], fwd["rstd"],
                                               _vec(gamma_bits, N, 1.0))
    dz32 = f32(dz).astype(np.float64)
    dx, q_dz, s_dz, q_wr, s_wr = dgrad(dz32, w)
    dw, q_xc, s_xc, q_dzc, s_dzc = wgrad(x, dz32)
    return {
        "dz": dz, "dz32": dz32, "q_dz": q_dz, "s_dz": s_dz, "q_wr": q_wr, "s_wr": s_wr,
        "dx": dx, "dx_bits": f64_to_bf16(dx), "dw": dw,
        "q_xc": q_xc, "s_xc": s_xc, "q_dzc": q_dzc, "s_dzc": s_dzc,
        "dgamma": dgamma, "dbeta": dbeta, "dbias": dz.sum(axis=0),
    }


def gemm_ln_backward_sq(x_bits, w_bits, dy_bits, bias_bits=None, gamma_bits=None, beta_bits=None,
                        eps=1e-5, no_ln=False):
    """Backward of the square-block forward (recipe "mx32_sq") for bf16
    inputs x[M,K], w[K,N], dy[M,N] (M, K, N multiples of 32).

    Returns a dict with dz (fp64), dz32, the square e5m2 codes/scales of dz32
    (q_dz [M,N], s_dz [M/32,N/32]), the forward's square codes/scales of X
    and W, dx (fp64) and dx_bits (bf16), dw (fp64), dgamma, dbeta, dbias."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    dy = bf16_to_f64(dy_bits)
    N = w.shape[1]
    q_x, s_x = quantize(x, MX32_SQ, E4M3)
    q_w, s_w = quantize(w, MX32_SQ, E4M3)
    if no_ln:
        dz, dgamma, dbeta = dy, None, None
    else:
        fwd = gemm_ln_forward(x_bits, w_bits, bias_bits, gamma_bits, beta_bits, eps, recipe="mx32_sq")
        dz, dgamma, dbeta = layernorm_backward(dy, fwd["z"], fwd["mean"], fwd["rstd"],
                                               _vec(gamma_bits, N, 1.0))
    dz32 = f32(dz).astype(np.float64)
    q_dz, s_dz = quantize(dz32, MX32_SQ, E5M2)
    dzq = dequantize(q_dz, s_dz, MX32_SQ, E5M2)
    dx = dzq @ dequantize(q_w, s_w, MX32_SQ, E4M3).T
    dw = dequantize(q_x, s_x, MX32_SQ, E4M3).T @ dzq
    return {
        "dz": dz, "dz32": dz32, "q_dz": q_dz, "s_dz": s_dz, "q_x": q_x, "s_x": s_x, "q_w": q_w, "s_w": s_w,
        "dx": dx, "dx_bits": f64_to_bf16(dx), "dw": dw,
        "dgamma": dgamma, "dbeta": dbeta, "dbias": dz.sum(axis=0),
    }


def reference_backward(x_bits, w_bits, dy_bits, bias_bits=None, gamma_bits=None, beta_bits=None, eps=1e-5):
    """The unquantized bf16 reference of the backward: the exact fp64
    gradients of sum(dY * Y) for Y = LayerNorm(X W + b) on the bf16 inputs
    taken exactly (what the backward's quantization error is measured
    against, reading R10).  Returns dz, dx = dZ W^T, dw = X^T dZ."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    dy = bf16_to_f64(dy_bits)
    N = w.shape[1]
    ref = reference_forward(x_bits, w_bits, bias_bits, gamma_bits, beta_bits, eps)
    dz, _, _ = layernorm_backward(dy, ref["z"], ref["mean"], ref["rstd"], _vec(gamma_bits, N, 1.0))
    return {"dz": dz, "dx": dz @ w.T, "dw": x.T @ dz}
