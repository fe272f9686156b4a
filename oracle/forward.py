"""Forward of the block: Y = LayerNorm(dequant(q(X) . q(W)) + b), in fp64.

Test infrastructure only (see the package docstring).

Sources:
  * [LoKA] section I and section III-B: the dominant recommendation-model
    pattern is a small GEMM followed immediately by a normalization layer;
    LayerNorm must run in higher precision (mean cancellation), so the GEMM
    output is dequantized before it.
  * [LoKA] section III-B2 (Block-wise Normalization): the normalization
    runs on (Wx + b) while the output tile is on chip; in Case 1 (large
    batch, small N) the whole feature row is in one block and the result
    equals the standard normalization.  This is that standard
    normalization over the full row.
  * [LoKA] section III-B1 (No Bias): a missing bias is a first-class mode.
  * [GEM] "Low Precision Flash Attention": block scales along K (MX path);
    its Block-wise Quantization gives the square-block recipe "mx32_sq",
    X[M,K] and W[K,N] each with one E8M0 scale per 32 x 32 block.

Steps (the plain definition; the GPU kernel is a faster evaluation of it):
  1. quantize X per recipe (tensor / row / mx32 along K) and W per recipe
     (tensor / per output column over K / mx32 along K), e4m3;
  2. A = sum_k code_x[m,k] * code_w[k,n] in fp64 -- exact for e4m3 with
     K <= 1024 (every partial sum is a multiple of 2**-18 below 2**28);
  3. Z = A * s_x[m] * s_w[n] + b[n] (MX: the E8M0 scales multiply each
     32-wide K block before the sum);
  4. mu = mean_n Z, v = mean_n (Z - mu)**2 (population variance, two
     passes), y = gamma * (Z - mu) / sqrt(v + eps) + beta;
  5. Y = RNE-bf16(y).
The BlockNorm + Hard Swish variant ([LoKA] section III-B2 Fig. 7d and
section III-B3) replaces step 4 by y = h(Z / sqrt(mean_block Z^2 + eps)) over
fixed blocks of features, h the Hard Swish.
"""

import numpy as np

from .codec import E4M3, bf16_to_f64, decode_fp8, decode_e8m0, f64_to_bf16
from .quant import quantize, dequantize, TENSOR, ROW, COL, MX32_ROW, MX32_COL, MX32_SQ

RECIPES = {
    # recipe name -> (mode for X[M,K], mode for W[K,N])
    "tensor": (TENSOR, TENSOR),
    "row": (ROW, COL),
    "mx32": (MX32_ROW, MX32_COL),
    "mx32_sq": (MX32_SQ, MX32_SQ),
}


def _vec(bits, n, default):
    if bits is None:
        return np.full(n, default, dtype=np.float64)
    return bf16_to_f64(bits)


def layernorm(z, gamma, beta, eps):
    """fp64 LayerNorm over the last axis: returns (y, mu, rstd)."""
    mu = z.mean(axis=1)
    d = z - mu[:, None]
    v = (d * d).mean(axis=1)
    rstd = 1.0 / np.sqrt(v + eps)
    y = gamma[None, :] * d * rstd[:, None] + beta[None, :]
    return y, mu, rstd


def quantized_product(x, w, recipe, fmt_x=E4M3, fmt_w=E4M3):
    """Steps 1-3 without the bias: (Z_no_bias, qx, sx, qw, sw) for x[M,K],
    w[K,N] given as fp32-exact float64 arrays."""
    mode_x, mode_w = RECIPES[recipe]
    qx, sx = quantize(x, mode_x, fmt_x)
    qw, sw = quantize(w, mode_w, fmt_w)
    dx = decode_fp8(qx, fmt_x)
    dw = decode_fp8(qw, fmt_w)
    if recipe == "mx32":
        ex = np.repeat(decode_e8m0(sx), 32, axis=1)          # [M, K]
        ew = np.repeat(decode_e8m0(sw), 32, axis=1).T        # [K, N]
        z = (dx * ex) @ (dw * ew)
    elif recipe == "mx32_sq":
        z = dequantize(qx, sx, MX32_SQ, fmt_x) @ dequantize(qw, sw, MX32_SQ, fmt_w)
    else:
        acc = dx @ dw
        sxb = np.float64(sx[0]) if mode_x == TENSOR else np.asarray(sx, np.float64)[:, None]
        swb = np.float64(sw[0]) if mode_w == TENSOR else np.asarray(sw, np.float64)[None, :]
        z = acc * sxb * swb
    return z, qx, sx, qw, sw


def gemm_ln_forward(x_bits, w_bits, bias_bits=None, gamma_bits=None, beta_bits=None,
                    eps=1e-5, recipe="row"):
    """The block's forward on bf16 bit patterns x[M,K], w[K,N].

    bias/gamma/beta are bf16 bit patterns of length N or None (None means
    0 / 1 / 0).  eps is taken at fp32 precision, as the library receives it.
    Returns a dict with y_bits (bf16 [M,N]), y (fp64 before rounding),
    z (fp64 pre-norm output), mean, rstd, and the quantized operands
    qx, sx, qw, sw (codes in the arrays' own [M,K] / [K,N] layouts)."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    M, K = x.shape
    K2, N = w.shape
    assert K == K2
    bias = _vec(bias_bits, N, 0.0)
    gamma = _vec(gamma_bits, N, 1.0)
    beta = _vec(beta_bits, N, 0.0)
    eps = float(np.float32(eps))
    z, qx, sx, qw, sw = quantized_product(x, w, recipe)
    z = z + bias[None, :]
    y, mu, rstd = layernorm(z, gamma, beta, eps)
    return {
        "y_bits": f64_to_bf16(y), "y": y, "z": z, "mean": mu, "rstd": rstd,
        "qx": qx, "sx": sx, "qw": qw, "sw": sw,
    }


def hard_swish(v):
    """[LoKA] section III-B3 (Hard Swish): h(v) = v * ReLU6(v + 3) / 6 with
    ReLU6(u) = min(max(u, 0), 6): zero at and below -3, the identity at and
    above 3, piecewise quadratic between."""
    return v * np.minimum(np.maximum(v + 3.0, 0.0), 6.0) / 6.0


def block_rmsnorm(z, block, eps):
    """[LoKA] section III-B2 (BlockNorm, Fig. 7d): root-mean-square
    normalization over fixed blocks of `block` consecutive features, each
    block's statistic computed on its own (an unparameterized grouped
    RMSNorm).  z [M, N] with N a multiple of block; returns (yhat, rinv),
    yhat = z / sqrt(mean_block(z^2) + eps) and rinv [M, N/block] the
    blocks' 1 / sqrt(mean(z^2) + eps)."""
    M, N = z.shape
    assert N % block == 0
    zb = z.reshape(M, N // block, block)
    rinv = 1.0 / np.sqrt((zb * zb).mean(axis=2) + eps)
    return (zb * rinv[:, :, None]).reshape(M, N), rinv


def gemm_blocknorm_hswish_forward(x_bits, w_bits, bias_bits=None, eps=1e-5, recipe="row", block=256):
    """The BlockNorm + Hard Swish variant of the block ([LoKA] section
    III-B2 and III-B3, the "LoKA Mods" epilogue): steps 1-3 and the bias as
    in gemm_ln_forward, then y = h(BlockNorm(Z)) per block of `block`
    features (no affine parameters), Y = RNE-bf16(y).  Returns y_bits, y,
    z, rinv and the quantized operands."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    N = w.shape[1]
    eps = float(np.float32(eps))
    z, qx, sx, qw, sw = quantized_product(x, w, recipe)
    z = z + _vec(bias_bits, N, 0.0)[None, :]
    yhat, rinv = block_rmsnorm(z, block, eps)
    y = hard_swish(yhat)
    return {"y_bits": f64_to_bf16(y), "y": y, "z": z, "rinv": rinv, "qx": qx, "sx": sx, "qw": qw, "sw": sw}


def square_quantized_output(y_bits):
    """The block's output Y quantized in 32 x 32 blocks, e4m3 (reading R16:
    the next layer's square-block input, its quantization fused into the
    normalization that produces Y -- [GEM] "Handling Quantization
    Overhead", PreNorm fusion): the codes and scales of the bf16 Y."""
    return quantize(bf16_to_f64(y_bits), MX32_SQ, E4M3)


def reference_forward(x_bits, w_bits, bias_bits=None, gamma_bits=None, beta_bits=None, eps=1e-5):
    """The unquantized bf16 reference: the same block on the bf16 inputs taken
    exactly in fp64 (what the quantization error is measured against)."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    N = w.shape[1]
    z = x @ w + _vec(bias_bits, N, 0.0)[None, :]
    y, mu, rstd = layernorm(z, _vec(gamma_bits, N, 1.0), _vec(beta_bits, N, 0.0), float(np.float32(eps)))
    return {"z": z, "y": y, "mean": mu, "rstd": rstd}
