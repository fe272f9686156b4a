"""The allocation-free forward (loka_gemm_fp8_ln_noalloc) against
loka_gemm_fp8_ln: the same kernels with the workspace in the library's fixed
device scratch instead of a caller buffer, so every output must be identical
bit for bit.  Two calls in a row on one GPU, the second smaller than the
first, so that a stale scratch (the first call's rearranged weight or amax
partials) would show; the row-major weight and the tensor recipe are the
cases that use the scratch."""

import numpy as np
import pytest
import torch

import fp8_precision_gemm_amd as lk
from synth.workloads import forward_case
from tests.gpu_helpers import bf16_dev, host

pytestmark = pytest.mark.gpu


def _both(c, x_mode, wmode, want_qx=True):
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    vec = [bf16_dev(c[k]) for k in ("bias", "gamma", "beta")]
    qw, sw, _ = lk.loka_quant_fp8(w, mode=wmode, transpose_out=True)   # row-major [N, K] codes
    kw = dict(x_mode=x_mode, want_z=True, want_stats=True, want_qx=want_qx)
    ref = lk.loka_gemm_fp8_ln(x, qw, sw, *vec, **kw)
    got = lk.loka_gemm_fp8_ln_noalloc(x, qw, sw, *vec, **kw)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, label):
    assert ref.keys() == got.keys()
    for k in ref:
        a, b = host(ref[k]), host(got[k])
        assert a.shape == b.shape, (label, k)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{label}: {k} differs"


@pytest.mark.parametrize("x_mode,wmode", [("row", "col"), ("tensor", "tensor"), ("mx32_row", "mx32_col")])
def test_noalloc_equals_workspace_entry_two_calls(lib, x_mode, wmode):
    """First a 4096 x 512 x 512 call (256 KiB of rearranged weight; for the
    tensor recipe also the amax partials), then a smaller 1000 x 256 x 256
    call."""
    big = forward_case(4096, 512, 512, seed=41, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    small = forward_case(1000, 256, 256, seed=42, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    for label, c in (("first (4096x512x512)", big), ("second (1000x256x256)", small)):
        ref, got = _both(c, x_mode, wmode)
        _same(ref, got, f"{x_mode} {label}")


def test_noalloc_same_as_first_call_after_a_different_weight(lib):
    """The same small call before and after a call with another weight: the
    scratch is rewritten by every call, so both results are identical."""
    small = forward_case(1000, 256, 256, seed=43, gamma_var=0.1, beta_var=0.1)
    other = forward_case(512, 256, 256, seed=44, gamma_var=0.1, beta_var=0.1)
    _, g1 = _both(small, "row", "col")
    _both(other, "row", "col")
    _, g2 = _both(small, "row", "col")
    _same(g1, g2, "repeat")
