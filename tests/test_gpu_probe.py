"""The Probe's statistics on the GPU against the oracle ([LoKA] section
III-A1): the batched mean/scatter merge, the matrix-normal flip-flop and the
two samplers, on the same bf16 inputs.

Tolerances (fp32 device arithmetic against fp64):
  mean:     1e-5 of the feature's scale (|mu| + std);
  scatter:  2e-5 * B * std_i * std_j (fp32 sums over B rows, in chunks);
  M, U, V:  1e-3 relative (Frobenius) after several updates: fp32 Cholesky
            factors and solves on well-conditioned factors;
  samples:  the Philox stream is integer-exact on both sides; the normals
            and the Z L^T products differ by fp32 rounding, so the bf16
            outputs agree to 2 ulp plus 1e-4 of the row's scale."""

import numpy as np
import pytest
import torch

import fp8_precision_gemm_amd as lk
from oracle import codec, probe
from synth.workloads import outlier_case, to_bf16_bits
from tests.gpu_helpers import bf16_dev, bf16_ulp, host

pytestmark = pytest.mark.gpu


def _batches(rng, sizes, K, offset):
    A = rng.standard_normal((K, K)) / np.sqrt(K) + np.eye(K)
    return [to_bf16_bits(offset + rng.standard_normal((b, K)) @ A) for b in sizes]


@pytest.mark.parametrize("K,sizes,offset", [(96, (300, 1, 77, 1024), 0.0), (64, (256, 512), 1e3)])
def test_input_merge(lib, K, sizes, offset):
    rng = np.random.default_rng(K)
    bs = _batches(rng, sizes, K, offset)
    state = None
    n, mu, S = 0, np.zeros(K), np.zeros((K, K))
    for b in bs:
        state = lk.loka_probe_input_update(bf16_dev(b), state)
        n, mu, S = probe.input_merge(n, mu, S, codec.bf16_to_f64(b))
    torch.cuda.synchronize()
    assert state["n"] == n
    sd = np.sqrt(np.diag(S) / (n - 1))
    np.testing.assert_allclose(host(state["mu"]), mu, rtol=0, atol=1e-5 * (np.abs(mu) + sd).max())
    tol = 2e-5 * n * np.outer(sd, sd) + 1e-5 * offset * n * np.outer(sd, sd) / max(sd.max(), 1e-30)
    err = np.abs(host(state["S"]).astype(np.float64) - S)
    assert np.all(err <= tol), f"scatter: worst {np.max(err / tol):.3f} x tol"


def test_input_merge_bench_activations(lib):
    """The 16384 x 512 outlier activations, as two batches."""
    c = outlier_case()
    x = c["x"]
    state = lk.loka_probe_input_update(bf16_dev(x[:6000]))
    state = lk.loka_probe_input_update(bf16_dev(x[6000:]), state)
    n, mu, S = probe.input_merge(0, np.zeros(512), np.zeros((512, 512)), codec.bf16_to_f64(x[:6000]))
    n, mu, S = probe.input_merge(n, mu, S, codec.bf16_to_f64(x[6000:]))
    torch.cuda.synchronize()
    sd = np.sqrt(np.diag(S) / (n - 1))
    np.testing.assert_allclose(host(state["mu"]), mu, rtol=0, atol=1e-5 * (np.abs(mu) + sd).max())
    err = np.abs(host(state["S"]).astype(np.float64) - S)
    assert np.all(err <= 2e-5 * n * np.outer(sd, sd)), f"worst {np.max(err / (2e-5 * n * np.outer(sd, sd))):.3f}"


@pytest.mark.parametrize("R,C", [(64, 48), (200, 136), (512, 512)])
def test_weight_flip_flop(lib, R, C):
    rng = np.random.default_rng(R + C)
    A = np.eye(R) + 0.3 * np.tril(rng.standard_normal((R, R))) / np.sqrt(R)
    Bm = np.eye(C) + 0.3 * np.tril(rng.standard_normal((C, C))) / np.sqrt(C)
    M0 = rng.standard_normal((R, C)) * 0.1
    Ws = [to_bf16_bits(M0 + 0.02 * A @ rng.standard_normal((R, C)) @ Bm.T) for _ in range(6)]
    state, ostate = None, None
    for W in Ws:
        state = lk.loka_probe_weight_update(bf16_dev(W), state, m=0.9)
        ostate = probe.weight_update(ostate, codec.bf16_to_f64(W), 0.9)
    torch.cuda.synchronize()
    for got, want, nm in zip((state["M"], state["U"], state["V"]), ostate, "MUV"):
        g = host(got).astype(np.float64)
        rel = np.linalg.norm(g - want) / np.linalg.norm(want)
        assert rel < 1e-3, f"{nm}: relative error {rel:.2e}"
    assert abs(np.trace(host(state["U"])) - R) < 1e-3 * R


def test_weight_zero_residual_closed_form(lib):
    """W equal to the tracked mean (both zero): U'' = m U, V'' = m V, then
    the symmetrization with eps I and the trace renormalization in closed
    form.  The diagonal spans four decades, so eps = 1e-6 trace / R moves the
    smallest entries by about 1e-3 (relative), far above fp32 rounding; the
    off-diagonal entries of U and V are asymmetric, so their average shows."""
    R, C, m = 96, 40, 0.9
    rng = np.random.default_rng(7)
    u = np.logspace(-2, 2, R)
    v = np.logspace(-1, 1, C)
    U0 = np.diag(u) + np.tril(rng.standard_normal((R, R)), -1) * 1e-3
    V0 = np.diag(v) + np.tril(rng.standard_normal((C, C)), -1) * 1e-3
    dev = torch.device("cuda")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    U0, V0 = U0.astype(np.float32).astype(np.float64), V0.astype(np.float32).astype(np.float64)
    state = {"M": f32(np.zeros((R, C))), "U": f32(U0), "V": f32(V0),
             "info": torch.zeros(2, dtype=torch.int32, device=dev)}
    W = np.zeros((R, C), dtype=np.uint16)           # bf16 zeros
    state = lk.loka_probe_weight_update(bf16_dev(W), state, m=m)
    torch.cuda.synchronize()
    eu, ev = 1e-6 * m * np.trace(U0) / R, 1e-6 * m * np.trace(V0) / C
    s = (m * np.trace(U0) + R * eu) / R
    U_hand = (m * (U0 + U0.T) / 2 + eu * np.eye(R)) / s
    V_hand = (m * (V0 + V0.T) / 2 + ev * np.eye(C)) * s
    for got, want, nm in ((state["U"], U_hand, "U"), (state["V"], V_hand, "V")):
        g = host(got).astype(np.float64)
        np.testing.assert_array_equal(g, g.T)
        tol = 4e-6 * np.abs(want) + 1e-9 * np.abs(want).max()   # fp32 EMA, average, trace sum
        err = np.abs(g - want)
        assert np.all(err <= tol), f"{nm}: worst {np.max(err / tol):.3f} x tol"
    np.testing.assert_array_equal(host(state["M"]), np.zeros((R, C), np.float32))


def _close_bf16(got_bits, want, label):
    g = codec.bf16_to_f64(got_bits)
    scale = np.sqrt((want ** 2).mean(axis=1, keepdims=True))
    tol = 2 * bf16_ulp(want) + 1e-4 * scale
    err = np.abs(g - want)
    assert np.all(err <= tol), f"{label}: worst {np.max(err / tol):.3f} x tol"


def test_sample_input(lib):
    rng = np.random.default_rng(3)
    K = 80
    b = _batches(rng, (2000,), K, 2.0)[0]
    state = lk.loka_probe_input_update(bf16_dev(b))
    n, mu, S = probe.input_merge(0, np.zeros(K), np.zeros((K, K)), codec.bf16_to_f64(b))
    out = host(lk.loka_probe_sample_input(state, 600, seed=17))
    want = probe.sample_input(n, host(state["mu"]).astype(np.float64), host(state["S"]).astype(np.float64), 600, 17)
    _close_bf16(out, want, "input sample")


def test_sample_weight(lib):
    rng = np.random.default_rng(4)
    R, C = 96, 64
    Ws = [to_bf16_bits(0.1 * rng.standard_normal((R, C))) for _ in range(3)]
    state = None
    for W in Ws:
        state = lk.loka_probe_weight_update(bf16_dev(W), state, m=0.8)
    out = host(lk.loka_probe_sample_weight(state, seed=5))
    M, U, V = (host(state[k]).astype(np.float64) for k in ("M", "U", "V"))
    _close_bf16(out, probe.sample_weight(M, U, V, 5), "weight sample")


def test_non_positive_definite_state_is_reported(lib):
    W = bf16_dev(to_bf16_bits(np.random.default_rng(6).standard_normal((32, 32))))
    state = lk.loka_probe_weight_update(W)
    state["V"].copy_(-torch.eye(32, device="cuda"))
    with pytest.raises(lk.LokaError):
        lk.loka_probe_weight_update(W, state)
