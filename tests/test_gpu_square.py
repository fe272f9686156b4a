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
@pytest.mark.parametrize("M,K,N", [(96, 160, 192), (64, 1024, 128), (32, 64, 64), (320, 640, 384),
                                   (1024, 512, 512), (224, 96, 256)])
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
