"""loka_gemm_fp8_ln with the BlockNorm + Hard Swish epilogue on the GPU
against the oracle's gemm_blocknorm_hswish_forward ([LoKA] section III-B2
Fig. 7d, section III-B3).  X codes and scales bit-exact, Z and Y within the
tolerances of the LayerNorm tests (see gpu_helpers).  Shapes cover one slab
(N = 256 or 512), several slabs of 256 and of 512 columns (N up to 4096,
beyond the LayerNorm's one-workgroup row), ragged M, K not a multiple of
128, No-Bias, degenerate rows, and the packed weight."""

import numpy as np
import pytest
import torch

from oracle import codec, forward
from synth.workloads import forward_case, to_bf16_bits
from tests.gpu_helpers import bf16_dev, check_y, check_z, host, sample_rows

pytestmark = pytest.mark.gpu


def run(lib, c, packed, no_bias=False, want_opt=True, eps=1e-5):
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    qw, sw, _ = lib.loka_quant_fp8(w, mode="col", transpose_out="packed" if packed else True)
    out = lib.loka_gemm_fp8_ln(x, qw, sw, bias=None if no_bias else bf16_dev(c["bias"]), eps=eps,
                               want_z=want_opt, want_qx=want_opt, w_packed=packed, epilogue="blocknorm_hswish")
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def rms_sigma(z, block=256):
    """Per-element scale of the block the element lies in: sqrt(mean z^2)
    (what the Z tolerance is relative to, as the row sigma for LayerNorm)."""
    M, N = z.shape
    zb = z.reshape(M, N // block, block)
    s = np.sqrt((zb * zb).mean(axis=2) + 1e-30)
    return np.repeat(s, block, axis=1)


def compare(g, o, rows, label):
    sel = slice(None) if rows is None else rows
    np.testing.assert_array_equal(g["qx"][sel], o["qx"], err_msg=f"{label}: X codes")
    np.testing.assert_array_equal(g["sx"][sel].view(np.uint32), o["sx"].astype(np.float32).view(np.uint32))
    zs = rms_sigma(o["z"])
    err = np.max(np.abs(g["z"][sel] - o["z"]) / np.maximum(np.abs(o["z"]), zs))
    assert err <= 1e-3, f"{label}: Z relative error {err:.3e}"
    ey = check_y(g["y"][sel], o["y"], label)
    print(f"{label}: Z err {err:.2e}  Y max abs err {ey:.2e}")


# (512, 256, 768) and (8192, 256, 1024) take the staged run (guard-free, at
# most four tiles per workgroup of each slab): 256-column slabs, and two
# 512-column slabs with exactly four tiles per workgroup
@pytest.mark.parametrize("M,K,N", [(1000, 192, 256), (130, 512, 512), (64, 1024, 256), (300, 256, 768),
                                   (77, 512, 1024), (33, 160, 2048), (48, 640, 1024), (16, 1024, 4096),
                                   (512, 256, 768), (8192, 256, 1024),
                                   # a full grid of 8 x slabs workgroups (each row group's slabs on one
                                   # XCD) with a ragged last tile: staged, staged, per-tile
                                   (4100, 256, 1024), (2000, 512, 4096), (4100, 512, 2048)])
def test_blocknorm_shapes(lib, M, K, N):
    c = forward_case(M, K, N, seed=M + 3 * K + N, x_dist="student_t3_outliers")
    g = run(lib, c, packed=True)
    o = forward.gemm_blocknorm_hswish_forward(c["x"], c["w"], c["bias"])
    compare(g, o, None, f"blocknorm {M}x{K}x{N}")
    # the row-major weight (rearranged in the call) gives the same bits, and
    # so does the kernel without the optional outputs
    r = run(lib, c, packed=False)
    for k in ("y", "z", "qx", "sx"):
        np.testing.assert_array_equal(r[k], g[k], err_msg=k)
    np.testing.assert_array_equal(run(lib, c, packed=True, want_opt=False)["y"], g["y"])


def test_blocknorm_no_bias_and_degenerate_rows(lib):
    c = forward_case(96, 256, 512, seed=21)
    x = codec.bf16_to_f64(c["x"])
    x[3] = 0.0             # zero row: every block is 0 -> y = h(0) = 0
    x[4] = 1.0             # constant row
    x[5] *= 2.0 ** -120    # tiny amax
    x[6] *= 2.0 ** 100     # squares overflow fp32 without the row rescale
    c["x"] = to_bf16_bits(x)
    g = run(lib, c, packed=True, no_bias=True)
    o = forward.gemm_blocknorm_hswish_forward(c["x"], c["w"], None)
    compare(g, o, None, "blocknorm no-bias degenerate")
    assert np.all(g["y"][3] == 0)


@pytest.mark.parametrize("M,K,N", [(16384, 512, 512), (4096, 512, 4096)])
def test_blocknorm_full_size_sampled(lib, M, K, N):
    """The benchmark's BlockNorm workload (the rowwise forward's shape) and a
    wide one (Case 2: N = 4096, eight 512-column slabs), in the launch
    configuration the benchmark times, checked on sampled rows."""
    c = forward_case(M, K, N, seed=7, x_dist="student_t3_outliers")
    g = run(lib, c, packed=True)
    rows = sample_rows(M, 256, seed=M + N)
    o = forward.gemm_blocknorm_hswish_forward(c["x"][rows], c["w"], c["bias"])
    compare(g, o, rows, f"blocknorm {M}x{K}x{N}")
    np.testing.assert_array_equal(run(lib, c, packed=True, want_opt=False)["y"], g["y"])
