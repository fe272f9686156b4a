"""Pins of the oracle's BlockNorm + Hard Swish epilogue ([LoKA] section
III-B2 "Block-wise Normalization", Fig. 7d, and section III-B3 "Hard
Swish") against what fixes them independently of its code: the closed
form of h at its break points, PyTorch's own rms_norm and hardswish routines
(library implementations of the two textbook definitions), and the
invariants the definition implies (per-block scale invariance, unit mean
square, independence of the blocks).  A mistake in the block grouping
(axis, size, order), a dropped square root or eps, or a wrong constant in
h fails one of them."""

import numpy as np
import pytest
import torch

from oracle import forward
from oracle.codec import bf16_to_f64
from synth.workloads import forward_case

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def test_hard_swish_closed_form():
    v = np.array([-10.0, -4.0, -3.0, -1.5, -1.0, 0.0, 1.0, 2.0, 3.0, 5.0, 100.0])
    want = np.array([0.0, 0.0, 0.0, -0.375, -1.0 / 3.0, 0.0, 2.0 / 3.0, 10.0 / 6.0, 3.0, 5.0, 100.0])
    np.testing.assert_allclose(forward.hard_swish(v), want, rtol=0, atol=1e-15)
    # its minimum is -3/8 at -3/2; continuous at both break points
    g = np.linspace(-4, 4, 8001)
    h = forward.hard_swish(g)
    assert abs(h.min() + 0.375) < 1e-6 and abs(g[h.argmin()] + 1.5) < 1e-3
    for b in (-3.0, 3.0):
        assert abs(forward.hard_swish(np.array([b - 1e-9]))[0] - forward.hard_swish(np.array([b + 1e-9]))[0]) < 1e-8


def test_hard_swish_matches_library():
    v = np.random.default_rng(0).standard_normal(4096) * 4.0
    lib = torch.nn.functional.hardswish(torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(forward.hard_swish(v), lib, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("block", [64, 256, 512])
def test_block_rmsnorm_matches_library(block):
    rng = np.random.default_rng(block)
    z = rng.standard_normal((7, 1024)) * rng.uniform(0.1, 30.0, size=(7, 1)) + rng.uniform(-5, 5, size=(7, 1))
    eps = 1e-5
    got, rinv = forward.block_rmsnorm(z, block, eps)
    zt = torch.from_numpy(z).reshape(7, 1024 // block, block)
    lib = torch.nn.functional.rms_norm(zt, (block,), eps=eps).reshape(7, 1024).numpy()
    np.testing.assert_allclose(got, lib, rtol=1e-13, atol=1e-13)
    assert rinv.shape == (7, 1024 // block)


def test_block_rmsnorm_invariants():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((3, 768)) + 2.0
    y, _ = forward.block_rmsnorm(z, 256, 0.0)
    # each block has unit mean square (eps = 0)
    np.testing.assert_allclose((y.reshape(3, 3, 256) ** 2).mean(axis=2), 1.0, rtol=1e-13)
    # scaling one block by c > 0 leaves every output unchanged
    z2 = z.copy()
    z2[:, 256:512] *= 37.5
    y2, _ = forward.block_rmsnorm(z2, 256, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13)
    # changing one block leaves the others' outputs unchanged
    z3 = z.copy()
    z3[:, :256] = rng.standard_normal((3, 256)) * 9.0
    y3, _ = forward.block_rmsnorm(z3, 256, 1e-5)
    y1, _ = forward.block_rmsnorm(z, 256, 1e-5)
    np.testing.assert_array_equal(y3[:, 256:], y1[:, 256:])
    assert not np.allclose(y3[:, :256], y1[:, :256])
    # one block over the whole row: plain RMSNorm of the row
    yr, rinv = forward.block_rmsnorm(z, 768, 1e-5)
    np.testing.assert_allclose(yr, z / np.sqrt((z * z).mean(axis=1, keepdims=True) + 1e-5), rtol=1e-14)


def test_blocknorm_forward_composes_the_steps():
    c = forward_case(24, 128, 512, seed=9)
    o = forward.gemm_blocknorm_hswish_forward(c["x"], c["w"], c["bias"], eps=1e-5)
    ln = forward.gemm_ln_forward(c["x"], c["w"], c["bias"])
    # same quantized product and bias as the LayerNorm path
    np.testing.assert_array_equal(o["z"], ln["z"])
    zt = torch.from_numpy(o["z"]).reshape(24, 2, 256)
    want = torch.nn.functional.hardswish(torch.nn.functional.rms_norm(zt, (256,), eps=float(np.float32(1e-5))))
    np.testing.assert_allclose(o["y"], want.reshape(24, 512).numpy(), rtol=1e-13, atol=1e-13)
    # bf16 rounding of y
    np.testing.assert_allclose(bf16_to_f64(o["y_bits"]), o["y"], rtol=2.0 ** -8, atol=1e-30)
