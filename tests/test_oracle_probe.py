"""Pins of the oracle's Probe statistics ([LoKA] section III-A1) against what
fixes them independently of its code:
  * Philox4x64-10 against NumPy's own Philox bit generator (a library
    implementation of the published generator), including a counter carry;
  * the normals against the standard normal distribution (moments and a
    Kolmogorov-Smirnov test with SciPy);
  * the batched mean/scatter merge against NumPy's mean and cov of all the
    batches at once, also with a mean far larger than the spread;
  * the flip-flop: trace renormalization, symmetry and definiteness, the
    Kronecker product unchanged by the renormalization, convergence to
    the true row and column covariances on matrix-normal samples, and a
    zero-residual update (W equal to the tracked mean) worked out by hand,
    which fixes the EMA, the symmetrization + eps I step and the trace
    renormalization in closed form;
  * the samplers against the moments of the distributions they sample.
A dropped merge term, a transposed factor or a wrong solve fails one."""

import numpy as np
import pytest
from scipy import stats

from oracle import probe


@pytest.mark.parametrize("key,counter", [((1, 2), (0, 0, 0, 0)), ((0xDEADBEEF, 7), (5, 0, 0, 0)),
                                         ((3, 0), ((1 << 64) - 1, 0, 0, 0)), ((0, 0), (9, 8, 7, 6))])
def test_philox_matches_numpy(key, counter):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(12)]
    c = list(counter)
    for blk in range(3):
        # NumPy advances the 256-bit counter before each block
        for i in range(4):
            c[i] = (c[i] + 1) & probe.M64
            if c[i] != 0:
                break
        assert probe.philox4x64_10(c, key) == raw[4 * blk:4 * blk + 4]


def test_normals_are_standard_normal():
    z = probe.normals(40000, seed=3)
    assert abs(z.mean()) < 4 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 4 * np.sqrt(2 / z.size)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # different seeds give different streams; a prefix is stable
    assert not np.allclose(probe.normals(100, 4), probe.normals(100, 3))
    np.testing.assert_array_equal(probe.normals(10, 3), z[:10])


@pytest.mark.parametrize("offset", [0.0, 1e4])
def test_input_merge_equals_one_shot(offset):
    rng = np.random.default_rng(0)
    A = rng.standard_normal((6, 6))
    batches = [offset + rng.standard_normal((b, 6)) @ A for b in (7, 1, 30, 12)]
    n, mu, S = 0, np.zeros(6), np.zeros((6, 6))
    for T in batches:
        n, mu, S = probe.input_merge(n, mu, S, T)
    allT = np.concatenate(batches)
    assert n == allT.shape[0]
    np.testing.assert_allclose(mu, allT.mean(axis=0), rtol=1e-12, atol=1e-12 * (1 + offset))
    np.testing.assert_allclose(probe.covariance(n, S), np.cov(allT.T, ddof=1), rtol=1e-9, atol=1e-9)


def _mn_sample(rng, M0, A, Bm):
    return M0 + A @ rng.standard_normal(M0.shape) @ Bm.T


def test_flip_flop_invariants_and_convergence():
    rng = np.random.default_rng(1)
    R, C = 6, 5
    A = np.tril(rng.standard_normal((R, R))) + 3 * np.eye(R)
    Bm = np.tril(rng.standard_normal((C, C))) + 2 * np.eye(C)
    U0, V0 = A @ A.T, Bm @ Bm.T
    M0 = rng.standard_normal((R, C))
    state = probe.weight_update(None, _mn_sample(rng, M0, A, Bm), 0.99)
    np.testing.assert_array_equal(state[1], np.eye(R))
    for it in range(6000):
        prev = state
        state = probe.weight_update(state, _mn_sample(rng, M0, A, Bm), 0.99)
        M, U, V = state
        if it < 5:
            assert abs(np.trace(U) - R) < 1e-9
            np.testing.assert_allclose(U, U.T, atol=1e-12)
            np.testing.assert_allclose(V, V.T, atol=1e-12)
            assert np.linalg.eigvalsh(U).min() > 0 and np.linalg.eigvalsh(V).min() > 0
    # identifiable up to a scale: compare U (x) V with U0 (x) V0
    K_est, K_true = np.kron(V, U), np.kron(V0, U0)
    err = np.linalg.norm(K_est - K_true) / np.linalg.norm(K_true)
    assert err < 0.15, err
    # M is an EMA of W: its noise has variance (1 - m) / (1 + m) of W's, whose
    # total is trace(U0) trace(V0)
    assert np.linalg.norm(M - M0) < 3 * np.sqrt(0.01 / 1.99 * np.trace(U0) * np.trace(V0))


def test_renormalization_keeps_the_kronecker_product():
    rng = np.random.default_rng(2)
    R, C = 4, 3
    state = probe.weight_update(None, rng.standard_normal((R, C)), 0.9)
    W = rng.standard_normal((R, C)) * 5
    M, U, V = probe.weight_update(state, W, 0.9)
    # the same update without the final rescaling, written from its parts
    Mo, Uo, Vo = state
    Mn = 0.9 * Mo + 0.1 * W
    Wc = W - Mn
    U1 = Wc @ np.linalg.inv(Vo + probe._eps(Vo) * np.eye(C)) @ Wc.T / C
    V1 = Wc.T @ np.linalg.inv(Uo + probe._eps(Uo) * np.eye(R)) @ Wc / R
    Uu, Vu = 0.9 * Uo + 0.1 * U1, 0.9 * Vo + 0.1 * V1
    Uu = (Uu + Uu.T) / 2 + 1e-6 * np.trace(Uu) / R * np.eye(R)
    Vu = (Vu + Vu.T) / 2 + 1e-6 * np.trace(Vu) / C * np.eye(C)
    np.testing.assert_allclose(np.kron(V, U), np.kron(Vu, Uu), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("m", [0.9, 0.99])
def test_zero_residual_update_closed_form(m):
    """W equal to the tracked mean: the mean stays, the centred residual and
    both per-update estimates vanish, so U'' = m U and V'' = m V.  With
    diagonal U = diag(u), V = diag(v) the pages' steps give by hand, with
    tu = sum(u), tv = sum(v):
        U <- m diag(u) + 1e-6 m tu / R I,   V <- m diag(v) + 1e-6 m tv / C I,
        s = m tu (1 + 1e-6) / R,            U <- U / s,  V <- s V.
    Dropping the eps I step moves every entry by about 1e-6 (relative); a
    missing renormalization leaves trace(U) = m R (1 + 1e-6)."""
    R, C = 5, 3
    u = np.array([0.5, 1.0, 2.0, 4.0, 0.25])
    v = np.array([3.0, 0.125, 1.5])
    W = np.zeros((R, C))     # m W + (1 - m) W == W exactly, so Wc == 0 exactly
    M, U, V = probe.weight_update((W.copy(), np.diag(u), np.diag(v)), W, m)
    tu, tv = u.sum(), v.sum()
    s = m * tu * (1 + 1e-6) / R
    U_hand = np.diag((m * u + 1e-6 * m * tu / R) / s)
    V_hand = np.diag((m * v + 1e-6 * m * tv / C) * s)
    np.testing.assert_array_equal(M, W)
    np.testing.assert_allclose(U, U_hand, rtol=1e-14, atol=0)
    np.testing.assert_allclose(V, V_hand, rtol=1e-14, atol=0)
    # the same without the regularization would be off by ~1e-6
    assert abs(U[0, 0] / (u[0] / (tu / R)) - 1) > 5e-8


def test_zero_residual_update_symmetrizes():
    """An asymmetric U or V (an EMA of round-off, say) leaves the update as
    the average of itself and its transpose plus eps I, then renormalized:
    with W equal to the mean, U <- (m (U + U^T) / 2 + eps I) / s where
    eps = 1e-6 m trace(U) / R and s = (m trace(U) + R eps) / R."""
    R, C, m = 3, 2, 0.9
    U0 = np.array([[2.0, 0.5, 0.0], [0.25, 1.0, 0.125], [0.0, 0.0, 3.0]])
    V0 = np.array([[1.0, 0.0], [0.5, 2.0]])
    W = np.zeros((R, C))
    _, U, V = probe.weight_update((W.copy(), U0, V0), W, m)
    eu = 1e-6 * m * 6.0 / R
    ev = 1e-6 * m * 3.0 / C
    s = (m * 6.0 + R * eu) / R
    U_hand = (m * np.array([[2.0, 0.375, 0.0], [0.375, 1.0, 0.0625], [0.0, 0.0625, 3.0]]) + eu * np.eye(R)) / s
    V_hand = (m * np.array([[1.0, 0.25], [0.25, 2.0]]) + ev * np.eye(C)) * s
    np.testing.assert_allclose(U, U_hand, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(V, V_hand, rtol=1e-14, atol=1e-16)
    np.testing.assert_array_equal(U, U.T)


def test_input_sampler_moments():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((5, 5))
    T = 3.0 + rng.standard_normal((4000, 5)) @ A
    n, mu, S = probe.input_merge(0, np.zeros(5), np.zeros((5, 5)), T)
    X = probe.sample_input(n, mu, S, 20000, seed=11)
    cov = probe.covariance(n, S)
    np.testing.assert_allclose(X.mean(axis=0), mu, atol=5 * np.sqrt(np.diag(cov).max() / 20000))
    np.testing.assert_allclose(np.cov(X.T), cov, rtol=0.05, atol=0.05 * np.abs(cov).max())


def test_weight_sampler_moments():
    rng = np.random.default_rng(5)
    R, C = 4, 3
    A = np.tril(rng.standard_normal((R, R))) + 2 * np.eye(R)
    Bm = np.tril(rng.standard_normal((C, C))) + 2 * np.eye(C)
    U, V = A @ A.T, Bm @ Bm.T
    M = rng.standard_normal((R, C))
    Ws = np.stack([probe.sample_weight(M, U, V, seed=s) - M for s in range(3000)])
    rows = np.einsum("sij,skj->ik", Ws, Ws) / len(Ws)   # E[(W-M)(W-M)^T] = tr(V) U
    cols = np.einsum("sji,sjk->ik", Ws, Ws) / len(Ws)   # E[(W-M)^T(W-M)] = tr(U) V
    np.testing.assert_allclose(rows, np.trace(V) * U, rtol=0.1, atol=0.1 * np.trace(V) * np.abs(U).max())
    np.testing.assert_allclose(cols, np.trace(U) * V, rtol=0.1, atol=0.1 * np.trace(U) * np.abs(V).max())
