"""Property tests over random small problems (hypothesis, derandomized, a
fixed example budget, no example database).

The pages' lesson ([LoKA] section II-C and Table V) is that ordinary normal
inputs hide real faults, so the strategies draw shapes, recipes, value
scales over many binades, heavy-tailed and outlier distributions.

CPU (the oracle against what fixes it independently of its code):
  * Z of every recipe lies within the quantization error bound of both
    operands around the exact X.W + b (half an e4m3 spacing per operand,
    relative 2^-4 for normals, plus the subnormal floor, plus the MX
    clipping of values in (448, 512) 2^e);
  * scaling X by a power of two scales the row / MX32 recipe's scales by
    the same power and leaves the codes and the normalized output alone
    (up to eps);
  * the LayerNorm output has zero mean and variance v/(v+eps) per row.
GPU: the fused forward against the oracle for every drawn case: X codes and
scales bit for bit, Z and Y to the stated tolerances."""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import codec, forward, quant
from synth.workloads import to_bf16_bits

RECIPES = ("tensor", "row", "mx32")
SETTINGS = dict(derandomize=True, database=None, deadline=None, print_blob=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@st.composite
def problems(draw, max_m=96, max_k=512, max_n=512):
    recipe = draw(st.sampled_from(RECIPES))
    M = draw(st.integers(1, max_m))
    K = 32 * draw(st.integers(1, max_k // 32)) if recipe == "mx32" else 16 * draw(st.integers(1, max_k // 16))
    N = 64 * draw(st.integers(1, max_n // 64))
    dist = draw(st.sampled_from(("normal", "t3_outliers", "lognormal_rows", "sparse")))
    xexp = draw(st.integers(-24, 24))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    with_bias = draw(st.booleans())
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((M, K))
    elif dist == "t3_outliers":
        x = rng.standard_t(3, size=(M, K))
        x[:, rng.permutation(K)[:max(1, K // 100)]] *= 50.0
    elif dist == "lognormal_rows":
        x = np.exp(rng.standard_normal((M, 1)) * 2.0) * rng.standard_normal((M, K))
    else:
        x = rng.standard_normal((M, K)) * (rng.random((M, K)) < 0.05)
    x = np.ldexp(x, xexp)
    w = rng.standard_normal((K, N)) / np.sqrt(K)
    bias = to_bf16_bits(0.1 * rng.standard_normal(N)) if with_bias else None
    gamma = to_bf16_bits(1.0 + 0.3 * rng.standard_normal(N))
    beta = to_bf16_bits(0.3 * rng.standard_normal(N))
    return {"recipe": recipe, "M": M, "K": K, "N": N, "x": to_bf16_bits(x), "w": to_bf16_bits(w),
            "bias": bias, "gamma": gamma, "beta": beta, "dist": dist}


def _half_spacing(v, s):
    """Half the e4m3 spacing around v / s, in units of v: relative 2^-4 for
    normals, absolute 2^-10 * s below the normal range."""
    return np.abs(v) * 2.0 ** -4 + np.asarray(s, np.float64) * 2.0 ** -10


@settings(max_examples=60, **SETTINGS)
@given(problems())
def test_oracle_z_within_quantization_bound(c):
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe=c["recipe"])
    x, w = codec.bf16_to_f64(c["x"]), codec.bf16_to_f64(c["w"])
    b = 0.0 if c["bias"] is None else codec.bf16_to_f64(c["bias"])[None, :]
    zref = x @ w + b
    if c["recipe"] == "mx32":
        # E8M0 scale 2^e per block: half spacing relative 2^-4, floor 2^-10 2^e,
        # plus the MX clipping of values in (448, 512) 2^e down to 448 2^e
        sx = np.repeat(codec.decode_e8m0(out["sx"]), 32, axis=1)
        sw = np.repeat(codec.decode_e8m0(out["sw"]), 32, axis=1).T
        ex = _half_spacing(x, sx) + np.maximum(np.abs(x) - 448.0 * sx, 0.0)
        ew = _half_spacing(w, sw) + np.maximum(np.abs(w) - 448.0 * sw, 0.0)
    else:
        if c["recipe"] == "row":
            sx = np.asarray(out["sx"], np.float64)[:, None]
            sw = np.asarray(out["sw"], np.float64)[None, :]
        else:
            sx, sw = float(out["sx"][0]), float(out["sw"][0])
        ex = _half_spacing(x, sx)
        ew = _half_spacing(w, sw)
    bound = ex @ np.abs(w) + np.abs(x) @ ew + ex @ ew
    err = np.abs(out["z"] - zref)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-300), float(np.max(err / np.maximum(bound, 1e-300)))


@settings(max_examples=40, **SETTINGS)
@given(problems(), st.integers(-12, 12))
def test_oracle_power_of_two_rescaling(c, j):
    if c["recipe"] == "tensor" or c["bias"] is not None:
        c = dict(c, recipe="row", bias=None)
    x = codec.bf16_to_f64(c["x"])
    xs = to_bf16_bits(np.ldexp(x, j))
    if not np.array_equal(codec.bf16_to_f64(xs), np.ldexp(x, j)):
        return  # the rescaled X left the bf16 range: not a valid case
    o1 = forward.gemm_ln_forward(c["x"], c["w"], None, c["gamma"], c["beta"], eps=0.0, recipe=c["recipe"])
    o2 = forward.gemm_ln_forward(xs, c["w"], None, c["gamma"], c["beta"], eps=0.0, recipe=c["recipe"])
    np.testing.assert_array_equal(o1["qx"], o2["qx"])
    np.testing.assert_array_equal(np.ldexp(o1["z"], j), o2["z"])
    np.testing.assert_allclose(o1["y"], o2["y"], rtol=1e-12, atol=1e-12)


@settings(max_examples=60, **SETTINGS)
@given(problems())
def test_oracle_layernorm_moments(c):
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], None, None, recipe=c["recipe"])
    z = out["z"]
    v = ((z - z.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    eps = float(np.float32(1e-5))
    y = out["y"]
    scale = np.maximum(np.abs(z).max(axis=1), 1e-300) * out["rstd"]
    assert np.all(np.abs(y.mean(axis=1)) <= 1e-12 * (1 + scale))
    np.testing.assert_allclose((y ** 2).mean(axis=1), v / (v + eps), rtol=1e-9, atol=1e-12)


# ---- GPU parity over the same strategy ----------------------------------------------

@pytest.mark.gpu
@settings(max_examples=40, **SETTINGS)
@given(problems(max_m=300, max_k=1024, max_n=1024))
def test_gpu_forward_property(c):
    import torch
    from tests.conftest import gpu_available
    if not gpu_available():
        pytest.skip("no GPU visible")
    import fp8_precision_gemm_amd as lk
    from tests.gpu_helpers import bf16_dev, check_y, check_z, host, row_sigma
    x_mode = {"tensor": "tensor", "row": "row", "mx32": "mx32_row"}[c["recipe"]]
    w_mode = {"tensor": "tensor", "row": "col", "mx32": "mx32_col"}[c["recipe"]]
    qw, sw, _ = lk.loka_quant_fp8(bf16_dev(c["w"]), mode=w_mode, transpose_out=True)
    g = lk.loka_gemm_fp8_ln(bf16_dev(c["x"]), qw, sw, bf16_dev(c["bias"]), bf16_dev(c["gamma"]),
                            bf16_dev(c["beta"]), x_mode=x_mode, want_z=True, want_qx=True)
    torch.cuda.synchronize()
    o = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe=c["recipe"])
    label = f"{c['recipe']} {c['M']}x{c['K']}x{c['N']} {c['dist']}"
    np.testing.assert_array_equal(host(g["qx"]), o["qx"], err_msg=f"{label}: X codes")
    if c["recipe"] == "mx32":
        np.testing.assert_array_equal(host(g["sx"]), o["sx"], err_msg=f"{label}: X scales")
    else:
        np.testing.assert_array_equal(host(g["sx"]).view(np.uint32), np.asarray(o["sx"], np.float32).view(np.uint32),
                                      err_msg=f"{label}: X scales")
    check_z(host(g["z"]), o["z"], row_sigma(o["z"]), label)
    check_y(host(g["y"]), o["y"], label)
