"""loka_gemm_fp8_ln on the GPU against the oracle.

Full-size cases use the three forward workloads (tensor recipe 512x256x256,
rowwise 16384x512x512 on outlier activations, MX 65536x1024x256 on
log-normal rows) in the launch configuration the benchmark times, and every
row is checked: X codes and scales bit for bit, Z, Y, mean and rstd (the
oracle takes the rows in blocks, which changes nothing: rows are independent
under the row and MX recipes).  Smaller cases
span several tiles with ragged M, K not a multiple of 128, No-Bias and
default gamma/beta, and degenerate rows."""

import numpy as np
import pytest
import torch

from oracle import codec, forward, quant
from synth.workloads import forward_case, mx_case, outlier_case, tensor_case, to_bf16_bits
from tests.gpu_helpers import bf16_dev, check_y, check_z, host, oracle_forward_blocks, row_sigma

pytestmark = pytest.mark.gpu

W_MODE = {"tensor": "tensor", "row": "col", "mx32_row": "mx32_col"}
RECIPE = {"tensor": "tensor", "row": "row", "mx32_row": "mx32"}


def run_gpu(lib, c, x_mode, eps=1e-5, no_bias=False, no_affine=False, packed=False):
    """One forward with every optional output.  packed: the weight in the
    packed layout (the benchmark's configuration), and a second call without
    the optional outputs (the kernel variant the benchmark times) whose Y
    must be bit-identical."""
    x = bf16_dev(c["x"])
    w = bf16_dev(c["w"])
    qw, sw, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode=W_MODE[x_mode], transpose_out=True)
    vec = dict(bias=None if no_bias else bf16_dev(c["bias"]), gamma=None if no_affine else bf16_dev(c["gamma"]),
               beta=None if no_affine else bf16_dev(c["beta"]), eps=eps, x_mode=x_mode)
    wq = qw
    if packed:
        wq, sw2, _ = lib.loka_quant_fp8(w, fmt="e4m3", mode=W_MODE[x_mode], transpose_out="packed")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(sw2), host(sw))
    out = lib.loka_gemm_fp8_ln(x, wq, sw, want_z=True, want_stats=True, want_qx=True, w_packed=packed, **vec)
    if packed:
        plain = lib.loka_gemm_fp8_ln(x, wq, sw, w_packed=True, **vec)
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    res["qw"], res["sw"] = host(qw), host(sw)
    if packed:
        np.testing.assert_array_equal(host(plain["y"]), res["y"], err_msg="Y without the optional outputs")
    return res


def oracle_rows(c, x_mode, rows, eps=1e-5, no_bias=False, no_affine=False):
    xs = c["x"][rows] if rows is not None else c["x"]
    return forward.gemm_ln_forward(xs, c["w"], None if no_bias else c["bias"],
                                   None if no_affine else c["gamma"], None if no_affine else c["beta"],
                                   eps=eps, recipe=RECIPE[x_mode])


def compare(g, o, rows, x_mode, label):
    sel = slice(None) if rows is None else rows
    np.testing.assert_array_equal(g["qx"][sel], o["qx"], err_msg=f"{label}: X codes")
    if x_mode == "row":
        np.testing.assert_array_equal(g["sx"][sel].view(np.uint32), o["sx"].astype(np.float32).view(np.uint32))
    elif x_mode == "mx32_row":
        np.testing.assert_array_equal(g["sx"][sel], o["sx"])
    else:
        np.testing.assert_array_equal(g["sx"].view(np.uint32), o["sx"].astype(np.float32).view(np.uint32))
    # the weight's codes (transposed) and scales
    np.testing.assert_array_equal(g["qw"].T, o["qw"], err_msg=f"{label}: W codes")
    if x_mode == "mx32_row":
        np.testing.assert_array_equal(g["sw"], o["sw"])
    else:
        np.testing.assert_array_equal(g["sw"].view(np.uint32), o["sw"].astype(np.float32).view(np.uint32))
    sigma = row_sigma(o["z"])
    ez = check_z(g["z"][sel], o["z"], sigma, label)
    ey = check_y(g["y"][sel], o["y"], label)
    np.testing.assert_allclose(g["mean"][sel], o["mean"], rtol=0, atol=1e-3 * sigma.max())
    np.testing.assert_allclose(g["rstd"][sel], o["rstd"], rtol=2e-3)
    print(f"{label}: Z err {ez:.2e}  Y max abs err {ey:.2e}")
    return ez


def test_tensor_recipe_full(lib):
    c = tensor_case()
    g = run_gpu(lib, c, "tensor", packed=True)
    o = oracle_rows(c, "tensor", None)
    compare(g, o, None, "tensor", "tensor 512x256x256")


def test_rowwise_outliers_full_size(lib):
    c = outlier_case()
    g = run_gpu(lib, c, "row", packed=True)
    o = oracle_forward_blocks(forward.gemm_ln_forward, c["x"], c["w"], c["bias"], c["gamma"], c["beta"],
                              recipe="row")
    compare(g, o, None, "row", "row 16384x512x512 (every row)")


def test_mx_full_size(lib):
    c = mx_case()
    g = run_gpu(lib, c, "mx32_row", packed=True)
    o = oracle_forward_blocks(forward.gemm_ln_forward, c["x"], c["w"], c["bias"], c["gamma"], c["beta"],
                              recipe="mx32")
    compare(g, o, None, "mx32_row", "mx 65536x1024x256 (every row)")


@pytest.mark.parametrize("x_mode", ["tensor", "row", "mx32_row"])
@pytest.mark.parametrize("M,K,N", [(1000, 192, 192), (130, 160, 384), (64, 1024, 128), (1, 64, 64),
                                   (257, 2048, 128), (200, 512, 1024)])
def test_ragged_shapes(lib, x_mode, M, K, N):
    c = forward_case(M, K, N, seed=M + K + N, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    g = run_gpu(lib, c, x_mode)
    o = oracle_rows(c, x_mode, None)
    compare(g, o, None, x_mode, f"{x_mode} {M}x{K}x{N}")


@pytest.mark.parametrize("M", [256, 272])
def test_tensor_scale_either_side_of_the_small_x_path(lib, M):
    """Tensorwise X at 1024 columns: 256 rows (16 workgroups x 2^18 elements =
    2^22) take the max inside the forward kernel, 272 rows use the partials
    pass.  Both give the oracle's scale and codes bit for bit."""
    c = forward_case(M, 1024, 256, seed=M, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    g = run_gpu(lib, c, "tensor", packed=True)
    o = oracle_rows(c, "tensor", None)
    compare(g, o, None, "tensor", f"tensor {M}x1024x256")


@pytest.mark.parametrize("x_mode", ["tensor", "row", "mx32_row"])
@pytest.mark.parametrize("M,K,N", [(1000, 192, 192), (130, 160, 384), (300, 256, 320), (77, 512, 512),
                                   (33, 1024, 128), (40, 640, 384), (16, 16, 64)])
def test_packed_weight_is_bit_identical(lib, x_mode, M, K, N):
    """The packed weight layout (loka_quant_fp8 transpose_out="packed" with
    w_packed=True) and the row-major layout (rearranged inside the call)
    give bit-identical outputs, with and without the optional outputs;
    N = 320 leaves the last wavefronts with fewer column tiles, K = 16 one
    partial chunk."""
    if x_mode == "mx32_row" and K % 32:
        pytest.skip("MX needs K % 32 == 0")
    c = forward_case(M, K, N, seed=3 * M + K + N, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    a = run_gpu(lib, c, x_mode, packed=True)
    b = run_gpu(lib, c, x_mode, packed=False)
    for k in ("y", "z", "mean", "rstd", "qx", "sx"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{x_mode} {M}x{K}x{N}: {k}")
    if M * N <= 200000:
        compare(a, oracle_rows(c, x_mode, None), None, x_mode, f"packed {x_mode} {M}x{K}x{N}")


@pytest.mark.parametrize("x_mode", ["row", "mx32_row"])
def test_no_bias_default_affine_and_degenerate_rows(lib, x_mode):
    c = forward_case(192, 256, 256, seed=7)
    x = codec.bf16_to_f64(c["x"])
    x[3] = 0.0               # zero row: Z = 0 -> y = beta
    x[4] = 1.0               # constant row
    x[5] *= 2.0 ** -120      # tiny amax (r saturates / E8M0 clamps)
    x[6] *= 2.0 ** 100
    c["x"] = to_bf16_bits(x)
    g = run_gpu(lib, c, x_mode, no_bias=True, no_affine=True)
    o = oracle_rows(c, x_mode, None, no_bias=True, no_affine=True)
    compare(g, o, None, x_mode, f"{x_mode} no-bias")
    assert np.all(g["y"][3] == 0)


def test_power_of_two_row_rescaling_on_gpu(lib):
    """Rows scaled by 2**j, j >= 0, with no bias and eps = 0: the codes are
    identical, the row scales exactly 2**j times larger, Z exactly 2**j
    times larger and Y bit-identical -- on the GPU alone (every scaling by a
    power of two is exact in the kernel's fp32 arithmetic)."""
    c = forward_case(256, 512, 512, seed=11, x_dist="student_t3_outliers")
    x = codec.bf16_to_f64(c["x"])
    j = np.arange(256) % 17
    c2 = dict(c, x=to_bf16_bits(np.ldexp(x, j[:, None])))
    g1 = run_gpu(lib, c, "row", eps=0.0, no_bias=True)
    g2 = run_gpu(lib, c2, "row", eps=0.0, no_bias=True)
    np.testing.assert_array_equal(g1["qx"], g2["qx"])
    np.testing.assert_array_equal(np.ldexp(g1["sx"].astype(np.float64), j), g2["sx"].astype(np.float64))
    np.testing.assert_array_equal(np.ldexp(g1["z"].astype(np.float64), j[:, None]), g2["z"].astype(np.float64))
    np.testing.assert_array_equal(g1["y"], g2["y"])


def test_deterministic_and_stream_async(lib):
    c = outlier_case(M=4096)
    a = run_gpu(lib, c, "row")
    b = run_gpu(lib, c, "row")
    for k in ("y", "z", "qx", "sx", "mean", "rstd"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    # on a side stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x = bf16_dev(c["x"])
        qw, sw, _ = lib.loka_quant_fp8(bf16_dev(c["w"]), mode="col", transpose_out=True)
        out = lib.loka_gemm_fp8_ln(x, qw, sw, bf16_dev(c["bias"]), bf16_dev(c["gamma"]), bf16_dev(c["beta"]))
    s.synchronize()
    np.testing.assert_array_equal(host(out["y"]), a["y"])
