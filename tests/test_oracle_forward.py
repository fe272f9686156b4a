"""Pins for the oracle's forward (quantize -> GEMM -> dequant + bias -> LN).

Pinned against:
  * exact integer arithmetic: e4m3 codes times 2**9 are integers, so the
    fp64 code GEMM must equal an int64 GEMM bit for bit (K <= 1024);
  * exact rationals on tiny shapes;
  * lossless special cases: inputs on the FP8 grid whose group maxima are
    FMAX * 2**j quantize exactly, so Z must equal the plain X.W + b of the
    unquantized inputs (this fixes the scale application, the operand
    orientation and the bias, for every recipe);
  * LayerNorm invariants (zero mean, variance v/(v+eps), constant rows,
    affinity in gamma/beta, power-of-two row rescaling);
  * the MERE definition on out = ref * (1 + delta).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, forward, grouped, mere, quant
from synth.workloads import to_bf16_bits, forward_case

E4 = codec.E4M3


def _grid_values(rng, shape, fmt, fill_max=True, axis=1):
    vals, _ = codec.fp8_grid(fmt)
    vals = vals[vals > 0]
    x = rng.choice(np.concatenate([vals, -vals, [0.0]]), size=shape)
    if fill_max:
        if axis == 1:
            x[:, rng.integers(0, shape[1])] = fmt.fmax
        else:
            x[rng.integers(0, shape[0]), :] = -fmt.fmax
    return x


def test_integer_exact_gemm():
    """fp64 GEMM of decoded e4m3 codes == int64 GEMM of codes * 2**9."""
    rng = np.random.default_rng(0)
    M, K, N = 64, 1024, 48
    cx = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 256, size=(K, N)).astype(np.uint8)
    cx[(cx & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    cw[(cw & 0x7F) == 0x7F] = 0x7E
    dx = codec.decode_fp8(cx, E4)
    dw = codec.decode_fp8(cw, E4)
    ix = (dx * 512).astype(np.int64)
    iw = (dw * 512).astype(np.int64)
    assert np.all(ix == dx * 512) and np.all(iw == dw * 512)
    exact = (ix @ iw)
    np.testing.assert_array_equal(dx @ dw, exact.astype(np.float64) / 2.0 ** 18)


@pytest.mark.parametrize("recipe", ["tensor", "row"])
def test_lossless_grid_inputs_give_plain_product(recipe):
    """X rows (row recipe) or X as a whole (tensor recipe) on the e4m3 grid
    with max magnitude 448 * 2**j, W likewise per column: quantization is
    exact, so Z = X.W + b computed on the raw inputs."""
    rng = np.random.default_rng(1)
    M, K, N = 48, 64, 40
    x = _grid_values(rng, (M, K), E4)
    w = _grid_values(rng, (K, N), E4, axis=0)
    if recipe == "row":
        jx = rng.integers(-12, 6, size=M)
        jw = rng.integers(-12, 6, size=N)
    else:
        jx = np.full(M, -3)
        jw = np.full(N, -7)
    x = np.ldexp(x, jx[:, None])
    w = np.ldexp(w, jw[None, :])
    xb, wb = to_bf16_bits(x), to_bf16_bits(w)
    assert np.all(codec.bf16_to_f64(xb) == x) and np.all(codec.bf16_to_f64(wb) == w)
    bias = to_bf16_bits(rng.standard_normal(N))
    out = forward.gemm_ln_forward(xb, wb, bias, recipe=recipe)
    zref = x @ w + codec.bf16_to_f64(bias)[None, :]
    np.testing.assert_array_equal(out["z"], zref)
    # W is not symmetric in any sense here: the transposed product differs
    assert not np.allclose(x @ w, (x[:, :N] @ w[:N, :]) if K != N else x @ w.T)


def test_lossless_mx_blocks():
    """Each 32-block of X (along K) and of W's columns (along K) holds e4m3
    grid values times a per-block power of two with the block maximum in
    [256, 448] * 2**e: the MX scales recover the blocks exactly and Z is the
    plain product."""
    rng = np.random.default_rng(2)
    M, K, N = 32, 128, 24
    vals, _ = codec.fp8_grid(E4)
    big = vals[(vals >= 256)]
    x = _grid_values(rng, (M, K), E4, fill_max=False)
    w = _grid_values(rng, (K, N), E4, fill_max=False)
    for b in range(K // 32):
        x[:, 32 * b + rng.integers(0, 32)] = rng.choice(big, M)
        w[32 * b + rng.integers(0, 32), :] = -rng.choice(big, N)
    x = np.minimum(np.abs(x), 448) * np.sign(x)
    ex = rng.integers(-20, 4, size=(M, K // 32))
    ew = rng.integers(-20, 4, size=(N, K // 32))
    x = np.ldexp(x, np.repeat(ex, 32, axis=1))
    w = np.ldexp(w, np.repeat(ew, 32, axis=1).T)
    xb, wb = to_bf16_bits(x), to_bf16_bits(w)
    assert np.all(codec.bf16_to_f64(xb) == x) and np.all(codec.bf16_to_f64(wb) == w)
    out = forward.gemm_ln_forward(xb, wb, None, recipe="mx32")
    np.testing.assert_array_equal(out["sx"].astype(np.int64) - 127 - 0, ex)  # block maxima in [256,448]: e = exponent - 8
    np.testing.assert_allclose(out["z"], x @ w, rtol=1e-15, atol=0)


def test_tiny_shapes_exact_rationals():
    """Z of tiny random problems against exact rational arithmetic on the
    oracle's own codes and scales (pins the summation and the scale
    order), and the codes against exact-rational RNE decisions."""
    rng = np.random.default_rng(3)
    for M, K, N in [(1, 1, 1), (3, 5, 2), (8, 8, 8), (2, 7, 5)]:
        c = forward_case(M, K, N, seed=int(rng.integers(1 << 30)))
        out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe="row")
        dx = codec.decode_fp8(out["qx"], E4)
        dw = codec.decode_fp8(out["qw"], E4)
        b = codec.bf16_to_f64(c["bias"])
        for m in range(M):
            for n in range(N):
                acc = sum(Fraction(dx[m, k]) * Fraction(dw[k, n]) for k in range(K))
                z = acc * Fraction(float(out["sx"][m])) * Fraction(float(out["sw"][n])) + Fraction(b[n])
                assert abs(Fraction(out["z"][m, n]) - z) <= abs(z) * Fraction(1, 1 << 50) + Fraction(1, 1 << 80)


def test_error_bound_random_inputs():
    """|Z - (X.W + b)| is bounded by the quantization error bounds of both
    operands: sum_k |dx||w| + |x||dw| + |dx||dw| with |dx| <= s_x*gap/2."""
    c = forward_case(96, 256, 80, seed=4, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    x, w = codec.bf16_to_f64(c["x"]), codec.bf16_to_f64(c["w"])
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe="row")
    zref = x @ w + codec.bf16_to_f64(c["bias"])[None, :]
    # half spacing of e4m3 relative to the value: 2**-4 (normals); absolute floor s * 2**-10
    ex = np.abs(x) * 2.0 ** -4 + out["sx"][:, None].astype(np.float64) * 2.0 ** -10
    ew = np.abs(w) * 2.0 ** -4 + out["sw"][None, :].astype(np.float64) * 2.0 ** -10
    bound = ex @ np.abs(w) + np.abs(x) @ ew + ex @ ew
    assert np.all(np.abs(out["z"] - zref) <= bound * 1.0001)
    # and the quantized result is genuinely different from the plain one
    assert np.abs(out["z"] - zref).max() > 0


def test_layernorm_invariants():
    c = forward_case(64, 128, 96, seed=5, gamma_var=None, beta_var=None)
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], None, None, eps=1e-5, recipe="row")
    y, z = out["y"], out["z"]
    eps = float(np.float32(1e-5))
    v = ((z - z.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), v / (v + eps), rtol=1e-12)
    np.testing.assert_allclose(out["rstd"], 1 / np.sqrt(v + eps), rtol=1e-14)
    # rounding to bf16 is the last step
    np.testing.assert_array_equal(out["y_bits"], codec.f64_to_bf16(y))


def test_layernorm_constant_row_and_affinity():
    M, K, N = 4, 32, 64
    x = np.zeros((M, K))
    x[0] = 1.0
    c = forward_case(M, K, N, seed=6)
    beta = to_bf16_bits(np.linspace(-1, 1, N))
    gamma = to_bf16_bits(np.linspace(0.5, 2, N))
    # zero input and no bias: Z == 0, so y == beta exactly
    out = forward.gemm_ln_forward(to_bf16_bits(x * 0), c["w"], None, gamma, beta)
    np.testing.assert_array_equal(out["y"], np.tile(codec.bf16_to_f64(beta), (M, 1)))
    # affine in gamma and beta
    g2 = to_bf16_bits(2 * codec.bf16_to_f64(gamma))
    o1 = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], gamma, None)
    o2 = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], g2, beta)
    np.testing.assert_allclose(o2["y"], 2 * o1["y"] + codec.bf16_to_f64(beta)[None, :], rtol=0, atol=1e-12)


def test_power_of_two_rescaling_changes_only_eps():
    """Row m scaled by 2**j (row recipe, no bias): codes are unchanged, Z
    scales by 2**j, and y equals the unscaled y computed with eps * 4**-j."""
    c = forward_case(16, 64, 48, seed=7)
    x = codec.bf16_to_f64(c["x"])
    j = np.arange(16) - 8
    xs = to_bf16_bits(np.ldexp(x, j[:, None]))
    o1 = forward.gemm_ln_forward(c["x"], c["w"], None, recipe="row")
    o2 = forward.gemm_ln_forward(xs, c["w"], None, recipe="row")
    np.testing.assert_array_equal(o1["qx"], o2["qx"])
    np.testing.assert_array_equal(np.ldexp(o1["z"], j[:, None]), o2["z"])
    eps = float(np.float32(1e-5))
    y1, _, _ = forward.layernorm(o1["z"], np.ones(48), np.zeros(48), 0.0)
    y2, _, _ = forward.layernorm(o2["z"], np.ones(48), np.zeros(48), 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)
    # with eps the rescaled rows see an effectively rescaled epsilon
    for m in range(16):
        ym, _, _ = forward.layernorm(o1["z"][m:m + 1], np.ones(48), np.zeros(48), eps * 4.0 ** (-j[m]))
        np.testing.assert_allclose(ym[0], o2["y"][m], rtol=1e-12, atol=1e-12)


def test_mere_definition():
    rng = np.random.default_rng(8)
    ref = rng.standard_normal((50, 40))
    ref[0, 0] = 0.0
    for delta in (0.0, 1e-3, 0.25):
        v, n = mere.mere(ref * (1 + delta), ref)
        assert n == ref.size - 1
        assert abs(v - delta) <= 1e-15 + delta * 1e-12
    v, n = mere.mere(ref * (1 - 0.5), ref)
    assert abs(v - 0.5) < 1e-15


def test_grouped_is_list_of_singles():
    gs = [forward_case(32, k, n, seed=k + n) for k, n in [(128, 192), (64, 32)]]
    outs = grouped.grouped_forward(gs)
    for g, o in zip(gs, outs):
        s = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        np.testing.assert_array_equal(o["y_bits"], s["y_bits"])


def test_reference_forward_quantization_error_is_small():
    """The quantized block against the unquantized bf16 reference: MERE of Y
    is of the order of e4m3's relative precision, not zero, not large."""
    c = forward_case(128, 256, 128, seed=9, gamma_var=0.1, beta_var=0.1)
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"])
    ref = forward.reference_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"])
    mz, _ = mere.mere(out["z"], ref["z"])
    # MERE is dominated by outputs near zero (the pages report values around
    # 0.4-0.5 for FP8 libraries); against each row's spread the error is small
    assert 1e-3 < mz < 1.0
    sigma = np.sqrt(ref["z"].var(axis=1))
    rel_row = np.abs(out["z"] - ref["z"]) / sigma[:, None]
    assert 1e-4 < rel_row.max() < 0.2


def test_reference_forward_exact_rationals():
    """The unquantized reference against exact rational arithmetic on a tiny
    problem with bias, gamma and beta: Z = X.W + b entry by entry (the
    products and sums of these bf16 values are exact in fp64, so Z must
    match bit for bit), then the mean and population variance exactly, and
    y = gamma (z - mean) / sqrt(v + eps) + beta with one final square root.
    A dropped bias, a transposed W (the shape is square and W asymmetric) or
    a mean over the wrong axis fails."""
    rng = np.random.default_rng(11)
    M, K, N = 3, 6, 6
    x = np.ldexp(rng.integers(-255, 256, size=(M, K)), rng.integers(-6, -3, size=(M, K))).astype(np.float64)
    w = np.ldexp(rng.integers(-255, 256, size=(K, N)), rng.integers(-9, -6, size=(K, N))).astype(np.float64)
    assert not np.allclose(w, w.T)
    b = np.ldexp(rng.integers(-255, 256, size=N), -8).astype(np.float64)
    g = np.ldexp(rng.integers(64, 256, size=N), -7).astype(np.float64)
    be = np.ldexp(rng.integers(-128, 128, size=N), -7).astype(np.float64)
    xb, wb, bb, gb, beb = (to_bf16_bits(a) for a in (x, w, b, g, be))
    for a, ab in ((x, xb), (w, wb), (b, bb), (g, gb), (be, beb)):
        assert np.all(codec.bf16_to_f64(ab) == a)
    ref = forward.reference_forward(xb, wb, bb, gb, beb)
    eps = Fraction(float(np.float32(1e-5)))
    for m in range(M):
        z = [sum(Fraction(x[m, k]) * Fraction(w[k, n]) for k in range(K)) + Fraction(b[n]) for n in range(N)]
        for n in range(N):
            assert Fraction(ref["z"][m, n]) == z[n]
        mu = sum(z) / N
        v = sum((zz - mu) ** 2 for zz in z) / N
        rstd = 1.0 / np.sqrt(float(v + eps))
        assert abs(ref["mean"][m] - float(mu)) <= 1e-15 * max(abs(float(mu)), 1e-30)
        for n in range(N):
            y = float(Fraction(g[n]) * (z[n] - mu)) * rstd + be[n]
            assert abs(ref["y"][m, n] - y) <= 1e-13 * (abs(y) + 1)


@pytest.mark.parametrize("recipe", ["tensor", "row", "mx32"])
def test_reference_equals_quantized_on_lossless_inputs(recipe):
    """Inputs on the e4m3 grid whose group maxima are 448 * 2**j quantize
    exactly, so the quantized block and the unquantized reference are the
    same computation: Z and Y equal bit for bit, and the MERE of both is 0
    over every nonzero entry."""
    rng = np.random.default_rng(12)
    M, K, N = 40, 96, 48
    x = _grid_values(rng, (M, K), E4)
    w = _grid_values(rng, (K, N), E4, axis=0)
    if recipe == "mx32":
        for blk in range(K // 32):
            x[:, 32 * blk] = 448.0
            w[32 * blk, :] = -448.0
        x = np.ldexp(x, np.repeat(rng.integers(-10, 3, size=(M, K // 32)), 32, axis=1))
        w = np.ldexp(w, np.repeat(rng.integers(-10, 3, size=(N, K // 32)), 32, axis=1).T)
    elif recipe == "row":
        x = np.ldexp(x, rng.integers(-10, 3, size=M)[:, None])
        w = np.ldexp(w, rng.integers(-10, 3, size=N)[None, :])
    else:
        x, w = np.ldexp(x, -2), np.ldexp(w, -6)
    xb, wb = to_bf16_bits(x), to_bf16_bits(w)
    assert np.all(codec.bf16_to_f64(xb) == x) and np.all(codec.bf16_to_f64(wb) == w)
    c = forward_case(M, K, N, seed=13, gamma_var=0.1, beta_var=0.1)
    out = forward.gemm_ln_forward(xb, wb, c["bias"], c["gamma"], c["beta"], recipe=recipe)
    ref = forward.reference_forward(xb, wb, c["bias"], c["gamma"], c["beta"])
    np.testing.assert_array_equal(out["z"], ref["z"])
    np.testing.assert_array_equal(out["y"], ref["y"])
    for a, r in ((out["z"], ref["z"]), (out["y"], ref["y"])):
        v, n = mere.mere(a, r)
        assert v == 0.0 and n == int((r != 0).sum()) and n > 0
