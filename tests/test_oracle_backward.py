"""Pins for the oracle's backward (LayerNorm backward, dgrad, wgrad).

Pinned against:
  * central finite differences of the fp64 LayerNorm forward (dZ, dgamma,
    dbeta) on small shapes;
  * the exact per-row identities sum_n dZ = 0 and
    sum_n dZ*yhat = rstd * N * mean(g*yhat) * eps / (v + eps);
  * lossless special cases for dgrad (rows of dZ on the e5m2 grid, rows of W
    on the e4m3 grid, maxima FMAX * 2**j) and wgrad (the same per column):
    the result must equal the plain products of the raw inputs, which fixes
    each operand's orientation, scale axis and format;
  * the literal reading (no LayerNorm): dZ == dY.
"""

import numpy as np

from oracle import backward, codec, forward
from synth.workloads import to_bf16_bits, forward_case


def _ln(z, gamma, beta, eps):
    y, _, _ = forward.layernorm(z, gamma, beta, eps)
    return y


def test_layernorm_backward_finite_differences():
    rng = np.random.default_rng(0)
    M, N = 3, 17
    z = rng.standard_normal((M, N)) * 3 + 1
    gamma = rng.standard_normal(N)
    beta = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    eps = 0.3   # large eps so that the eps terms are visible
    _, mu, rstd = forward.layernorm(z, gamma, beta, eps)
    dz, dgamma, dbeta = backward.layernorm_backward(dy, z, mu, rstd, gamma)
    h = 1e-6
    L = lambda zz, gg, bb: np.sum(dy * _ln(zz, gg, bb, eps))
    fd = np.zeros_like(z)
    for i in range(M):
        for j in range(N):
            e = np.zeros_like(z)
            e[i, j] = h
            fd[i, j] = (L(z + e, gamma, beta) - L(z - e, gamma, beta)) / (2 * h)
    np.testing.assert_allclose(dz, fd, rtol=1e-6, atol=1e-8)
    fdg = np.array([(L(z, gamma + h * (np.arange(N) == j), beta) - L(z, gamma - h * (np.arange(N) == j), beta)) / (2 * h)
                    for j in range(N)])
    np.testing.assert_allclose(dgamma, fdg, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dbeta, dy.sum(axis=0), rtol=1e-14)


def test_layernorm_backward_identities():
    rng = np.random.default_rng(1)
    M, N = 50, 64
    z = rng.standard_normal((M, N)) * rng.uniform(0.01, 10, size=(M, 1))
    gamma = 1 + 0.3 * rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    eps = 1e-2
    _, mu, rstd = forward.layernorm(z, gamma, np.zeros(N), eps)
    dz, _, _ = backward.layernorm_backward(dy, z, mu, rstd, gamma)
    yhat = (z - mu[:, None]) * rstd[:, None]
    g = dy * gamma
    v = ((z - mu[:, None]) ** 2).mean(axis=1)
    scale = np.abs(dz).sum(axis=1)
    np.testing.assert_allclose(dz.sum(axis=1) / scale, 0, atol=1e-14)
    expect = rstd * N * (g * yhat).mean(axis=1) * eps / (v + eps)
    np.testing.assert_allclose((dz * yhat).sum(axis=1), expect, rtol=1e-9, atol=1e-12 * scale.max())


def _on_grid(rng, shape, fmt, max_axis):
    vals, _ = codec.fp8_grid(fmt)
    x = rng.choice(np.concatenate([vals, -vals]), size=shape)
    if max_axis == 1:   # every row holds +-FMAX
        x[np.arange(shape[0]), rng.integers(0, shape[1], shape[0])] = fmt.fmax
    else:               # every column holds +-FMAX
        x[rng.integers(0, shape[0], shape[1]), np.arange(shape[1])] = -fmt.fmax
    return x


def test_dgrad_lossless():
    """dZ rows on the e5m2 grid (row max 57344 * 2**j), W rows (its k index)
    on the e4m3 grid (row max 448 * 2**i): dX = dZ . W^T exactly."""
    rng = np.random.default_rng(2)
    M, K, N = 40, 24, 32
    dz = np.ldexp(_on_grid(rng, (M, N), codec.E5M2, 1), rng.integers(-30, -10, M)[:, None])
    w = np.ldexp(_on_grid(rng, (K, N), codec.E4M3, 1), rng.integers(-12, -4, K)[:, None])
    dx, *_ = backward.dgrad(dz, w)
    np.testing.assert_array_equal(dx, dz @ w.T)


def test_wgrad_lossless():
    """Columns of X on the e4m3 grid and columns of dZ on the e5m2 grid with
    column maxima FMAX * 2**j: dW = X^T . dZ exactly."""
    rng = np.random.default_rng(3)
    M, K, N = 64, 24, 40
    x = np.ldexp(_on_grid(rng, (M, K), codec.E4M3, 0), rng.integers(-8, 2, K)[None, :])
    dz = np.ldexp(_on_grid(rng, (M, N), codec.E5M2, 0), rng.integers(-30, -10, N)[None, :])
    dw, *_ = backward.wgrad(x, dz)
    np.testing.assert_allclose(dw, x.T @ dz, rtol=1e-15, atol=0)


def test_literal_reading_no_layernorm():
    c = forward_case(32, 64, 48, seed=4, dy_var=1e-3)
    out = backward.gemm_ln_backward(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"], no_ln=True)
    np.testing.assert_array_equal(out["dz"], codec.bf16_to_f64(c["dy"]))
    np.testing.assert_array_equal(out["dbias"], codec.bf16_to_f64(c["dy"]).sum(axis=0))
    assert out["dgamma"] is None


def test_full_backward_consistency():
    """The full backward's pieces agree with the separately pinned parts and
    its dX/dW approximate the unquantized gradients."""
    c = forward_case(64, 96, 80, seed=5, gamma_var=0.1, beta_var=0.1, dy_var=1e-3)
    out = backward.gemm_ln_backward(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"])
    x, w = codec.bf16_to_f64(c["x"]), codec.bf16_to_f64(c["w"])
    np.testing.assert_array_equal(out["dz32"], out["dz"].astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(out["dbias"], out["dz"].sum(axis=0), rtol=1e-15)
    np.testing.assert_allclose(out["dbeta"], codec.bf16_to_f64(c["dy"]).sum(axis=0), rtol=1e-15)
    dx_plain = out["dz"] @ w.T
    dw_plain = x.T @ out["dz"]
    assert np.abs(out["dx"] - dx_plain).max() < 0.2 * np.abs(dx_plain).max()
    assert np.abs(out["dw"] - dw_plain).max() < 0.2 * np.abs(dw_plain).max()
    np.testing.assert_array_equal(out["dx_bits"], codec.f64_to_bf16(out["dx"]))


def test_reference_backward_finite_differences():
    """The unquantized reference backward against central differences of the
    plain fp64 loss L(X, W, b) = sum(dY * LayerNorm(X W + b)) -- a function
    written here from the definition, not from the oracle."""
    rng = np.random.default_rng(21)
    M, K, N = 3, 4, 5
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((K, N))
    b = rng.standard_normal(N)
    g = 1 + 0.3 * rng.standard_normal(N)
    be = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    xb, wb, bb, gb, beb, dyb = (to_bf16_bits(a) for a in (x, w, b, g, be, dy))
    x, w, b, g, be, dy = (codec.bf16_to_f64(a) for a in (xb, wb, bb, gb, beb, dyb))
    eps = float(np.float32(1e-5))

    def loss(xx, ww):
        z = xx @ ww + b[None, :]
        mu = z.mean(axis=1, keepdims=True)
        var = ((z - mu) ** 2).mean(axis=1, keepdims=True)
        return np.sum(dy * (g * (z - mu) / np.sqrt(var + eps) + be))

    ref = backward.reference_backward(xb, wb, dyb, bb, gb, beb)
    h = 1e-6
    for arr, grad in ((x, ref["dx"]), (w, ref["dw"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(x, w)
            arr[idx] = old - h
            lm = loss(x, w)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7)
