"""loka_quant_fp8 on the GPU against the oracle: codes and scales bit-exact
for every scaling mode, format, source dtype and layout."""

import numpy as np
import pytest
import torch

from oracle import codec, quant
from synth.workloads import outlier_case, to_bf16_bits
from tests.gpu_helpers import bf16_dev, f32_dev, host, unpack_packed

pytestmark = pytest.mark.gpu

MODES = ["tensor", "row", "col", "mx32_row", "mx32_col", "mx32_sq"]
MX = ("mx32_row", "mx32_col", "mx32_sq")
FMTS = {"e4m3": codec.E4M3, "e5m2": codec.E5M2}


def all_bf16_matrix():
    """Every finite bf16 pattern once, as a [256, 256]-shaped block of rows
    ([255 * 256 + tail]); the non-finite patterns are replaced by zero."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_to_f64(bits)
    bits = np.where(np.isfinite(v), bits, 0).astype(np.uint16)
    return bits.reshape(256, 256)


def check_quant(lib, x_bits_or_f32, mode, fmt, transpose, src_f32=False, label=""):
    if src_f32:
        xt = f32_dev(x_bits_or_f32)
        xv = x_bits_or_f32.astype(np.float64)
    else:
        xt = bf16_dev(x_bits_or_f32)
        xv = codec.bf16_to_f64(x_bits_or_f32)
    codes, scales, amax = lib.loka_quant_fp8(xt, fmt=fmt, mode=mode, transpose_out=transpose,
                                             want_amax=mode in ("tensor", "row", "col"))
    torch.cuda.synchronize()
    ref_codes, ref_scales = quant.quantize(xv, mode, FMTS[fmt])
    got = host(codes)
    if transpose == "packed":
        rows, cols = ref_codes.shape
        assert tuple(codes.shape) == lib.packed_shape(rows, cols)
        got = unpack_packed(got, cols, rows).T
    elif transpose == "packed_rows":
        rows, cols = ref_codes.shape
        assert tuple(codes.shape) == lib.packed_shape(cols, rows)
        got = unpack_packed(got, rows, cols)
    elif transpose:
        got = got.T
    bad = np.nonzero(got != ref_codes)
    assert bad[0].size == 0, (f"{label} {mode}/{fmt}/T={transpose}: {bad[0].size} code mismatches, first at "
                              f"{bad[0][0], bad[1][0]}: gpu {got[bad[0][0], bad[1][0]]:#04x} "
                              f"ref {ref_codes[bad[0][0], bad[1][0]]:#04x} x={xv[bad[0][0], bad[1][0]]!r}")
    gs = host(scales)
    if mode in MX:
        np.testing.assert_array_equal(gs, ref_scales)
    else:
        np.testing.assert_array_equal(gs.view(np.uint32), ref_scales.astype(np.float32).view(np.uint32))
        np.testing.assert_array_equal(host(amax), quant.amax(xv, mode).astype(np.float32))


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("mode", MODES)
def test_every_bf16_value(lib, mode, fmt, transpose):
    check_quant(lib, all_bf16_matrix(), mode, fmt, transpose, label="all-bf16")


@pytest.mark.parametrize("mode", ["tensor", "col", "mx32_col", "mx32_sq"])
@pytest.mark.parametrize("rows,cols", [(256, 256), (144, 96), (32, 16), (640, 48), (96, 160)])
def test_packed_layout(lib, mode, rows, cols):
    """transpose_out="packed": the codes of src^T in the fragment-interleaved
    layout (rows not a multiple of 128 are padded with zero codes), the same
    codes and scales as the plain layouts."""
    if mode == "mx32_col" and rows % 32:
        pytest.skip("MX32_COL needs rows % 32 == 0")
    if mode == "mx32_sq" and (rows % 32 or cols % 32):
        pytest.skip("MX32_SQ needs rows and cols % 32 == 0")
    rng = np.random.default_rng(rows * 7 + cols)
    x = to_bf16_bits(rng.standard_t(3, size=(rows, cols)))
    check_quant(lib, x, mode, "e4m3", "packed", label=f"packed {rows}x{cols}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rows,cols", [(256, 256), (144, 96), (32, 16), (64, 336), (96, 160)])
def test_packed_rows_layout(lib, mode, rows, cols):
    """transpose_out="packed_rows": the codes of src itself in the
    fragment-interleaved layout (columns not a multiple of 128 padded with
    zero codes), the same codes and scales as the plain layout."""
    if mode in ("mx32_row", "mx32_sq") and cols % 32:
        pytest.skip("MX32_ROW and MX32_SQ need cols % 32 == 0")
    if mode in ("mx32_col", "mx32_sq") and rows % 32:
        pytest.skip("MX32_COL and MX32_SQ need rows % 32 == 0")
    rng = np.random.default_rng(rows * 5 + cols)
    x = to_bf16_bits(rng.standard_t(3, size=(rows, cols)))
    check_quant(lib, x, mode, "e5m2" if mode == "row" else "e4m3", "packed_rows", label=f"packed_rows {rows}x{cols}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("mode", MODES)
def test_fp32_source_with_ragged_edges(lib, mode, fmt):
    """fp32 input (the backward's dZ), rows not a multiple of the 64-row
    tile, heavy tails, zero rows/columns and subnormal-range values."""
    rng = np.random.default_rng(3)
    rows, cols = 96 + 32, 80 + 48  # 128 x 128 for MX; ragged against 64-tiles elsewhere below
    if mode not in MX:
        rows, cols = 100 + 12, 144
    x = (rng.standard_t(3, size=(rows, cols)) * np.exp(3 * rng.standard_normal((rows, 1)))).astype(np.float32)
    x[5] = 0.0
    x[:, 7] = 0.0
    x[9] *= np.float32(1e-38)
    x[10, :] = np.float32(-0.0)
    check_quant(lib, x, mode, fmt, transpose=False, src_f32=True, label="fp32")
    if rows % 16 == 0:
        check_quant(lib, x, mode, fmt, transpose=True, src_f32=True, label="fp32")


def test_outlier_activations_rowwise(lib):
    """The 16384 x 512 Student-t activations with outlier columns, rowwise
    e4m3 (the forward's X recipe), and its weight per column, transposed."""
    c = outlier_case()
    check_quant(lib, c["x"], "row", "e4m3", False, label="outlier X")
    check_quant(lib, c["w"], "col", "e4m3", True, label="outlier W")


def test_tiny_and_degenerate(lib):
    for rows, cols in [(1, 16), (16, 16), (3, 32), (64, 1024)]:
        x = to_bf16_bits(np.random.default_rng(rows).standard_normal((rows, cols)))
        for mode in ("tensor", "row", "col"):
            check_quant(lib, x, mode, "e4m3", False, label=f"{rows}x{cols}")
    z = np.zeros((32, 64), np.uint16)
    for mode in MODES:
        check_quant(lib, z, mode, "e4m3", True, label="zeros")


@pytest.mark.parametrize("rows", [1024, 1040])
@pytest.mark.parametrize("transpose", [False, True, "packed", "packed_rows"])
def test_column_scales_both_paths(lib, rows, transpose):
    """Column scaling of bf16 takes one launch per 64-column strip up to 1024
    rows and the partial-maxima pass beyond: both against the oracle, with
    a column that is all zeros and a column whose maximum sits in the last
    row."""
    rng = np.random.default_rng(rows)
    x = rng.standard_t(3, size=(rows, 208)) * np.exp(2 * rng.standard_normal((1, 208)))
    x[:, 17] = 0.0
    x[-1, 40] = 1e6
    check_quant(lib, to_bf16_bits(x), "col", "e4m3", transpose, label=f"col {rows}x208")


def test_deterministic(lib):
    c = outlier_case(M=2048)
    xt = bf16_dev(c["x"])
    a = [host(t) for t in lib.loka_quant_fp8(xt, fmt="e5m2", mode="col", transpose_out=True)[:2]]
    b = [host(t) for t in lib.loka_quant_fp8(xt, fmt="e5m2", mode="col", transpose_out=True)[:2]]
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(96, 160), (32, 32), (160, 96)])
def test_square_blocks_partial_tiles(lib, fmt, rows, cols):
    """MX32_SQ where the 32 x 32 blocks do not fill the 64 x 64 cast tiles,
    with one block per row band scaled far apart (every block its own scale)."""
    rng = np.random.default_rng(rows + 3 * cols)
    x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-30, 30, (rows // 32, cols // 32))).repeat(
        32, axis=0).repeat(32, axis=1)
    check_quant(lib, to_bf16_bits(x), "mx32_sq", fmt, False, label="square")
    check_quant(lib, to_bf16_bits(x), "mx32_sq", fmt, True, label="square")
