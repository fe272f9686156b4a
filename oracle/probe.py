"""The Probe's statistics ([LoKA] section III-A1, "Online Distribution
Learning" and "Sampling learned distributions"), in fp64.

Test infrastructure only (see the package docstring).

  * Input tracker: a layer input T [B, K] per probed step; the summary is
    (n, mu, S) with S the unnormalized scatter matrix.  A batch with mean
    mu_b and scatter S_b merges as (Chan, Golub and LeVeque's pairwise
    update, the pages' equations):
        n' = n + B,  d = mu_b - mu,  mu' = mu + (B / n') d,
        S' = S + S_b + (n B / n') d d^T,
    and the covariance is S / (n - 1).
  * Weight tracker: W [R, C] ~ MN(M, U, V) with row covariance U [R, R] and
    column covariance V [C, C], kept by a Kronecker flip-flop with an EMA of
    momentum m.  Per update, with Wc = W - M:
        L_V L_V^T = V + eps_V I,  Wt = Wc L_V^-T,  U1 = Wt Wt^T / C,
        L_U L_U^T = U + eps_U I,  Wu = L_U^-1 Wc,  V1 = Wu^T Wu / R,
        U'' = m U + (1 - m) U1,  V'' = m V + (1 - m) V1,
        U <- (U'' + U''^T) / 2 + eps_U I,  V <- (V'' + V''^T) / 2 + eps_V I,
        s = trace(U) / R,  U <- U / s,  V <- s V.
    Linear solves with the Cholesky factors, never explicit inverses.
  * Sampler: T' = 1 mu^T + Z L^T with L L^T = cov + eps I;
    W' = M + L_U Z L_V^T.

Readings (reading R18), where the extracted text is silent:
  * the mean M is itself an EMA of W with the same momentum, updated
    before the centring; the first update only initializes (M = W, U = I_R,
    V = I_C), since its centred residual is zero;
  * both per-update estimates use the U and V from before the update
    (a simultaneous, not a sequential, flip-flop);
  * eps = 1e-6 trace(A) / dim(A) for each factor A (the pages give
    1e-6 trace(U) / M as the example), with A the matrix being regularized:
    the factor before the update for the two Cholesky factorizations, and
    the EMA result U'' or V'' for the symmetrization step;
  * the random draws Z are standard normal from Philox4x64-10 (Salmon,
    Moraes, Dror and Shaw, SC'11), counter (i, 0, 0, 0) for block i and key
    (seed, 0), each 64-bit output u giving the uniform (u >> 11) 2^-53 and
    pairs of uniforms (u1, u2) the Box-Muller normals
    sqrt(-2 ln(1 - u1)) cos(2 pi u2) and sqrt(-2 ln(1 - u1)) sin(2 pi u2),
    filled in row-major order.
"""

import numpy as np

M64 = (1 << 64) - 1
PHILOX_M0, PHILOX_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
PHILOX_W0, PHILOX_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def philox4x64_10(ctr, key):
    """One Philox4x64 block of 10 rounds: ctr 4 ints, key 2 ints (64-bit)."""
    c = [int(v) & M64 for v in ctr]
    k0, k1 = int(key[0]) & M64, int(key[1]) & M64
    for rnd in range(10):
        p0, p1 = PHILOX_M0 * c[0], PHILOX_M1 * c[2]
        hi0, lo0 = p0 >> 64, p0 & M64
        hi1, lo1 = p1 >> 64, p1 & M64
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        if rnd < 9:
            k0, k1 = (k0 + PHILOX_W0) & M64, (k1 + PHILOX_W1) & M64
    return c


def normals(count, seed):
    """count standard normals: block i (counter (i, 0, 0, 0), key (seed, 0))
    gives four 64-bit outputs, i.e. two uniform pairs, i.e. four normals."""
    out = np.empty(count)
    nblk = (count + 3) // 4
    for i in range(nblk):
        u = [(v >> 11) * 2.0 ** -53 for v in philox4x64_10((i, 0, 0, 0), (seed, 0))]
        for p in range(2):
            r = np.sqrt(-2.0 * np.log(1.0 - u[2 * p]))
            t = 2.0 * np.pi * u[2 * p + 1]
            for q, v in enumerate((r * np.cos(t), r * np.sin(t))):
                j = 4 * i + 2 * p + q
                if j < count:
                    out[j] = v
    return out


# ---- input tracker -----------------------------------------------------------

def input_merge(n, mu, S, T):
    """Merge batch T [B, K] (fp64 values) into the summary (n, mu [K], S [K, K])."""
    T = np.asarray(T, dtype=np.float64)
    B = T.shape[0]
    mu_b = T.mean(axis=0)
    C = T - mu_b[None, :]
    S_b = C.T @ C
    n_new = n + B
    d = mu_b - mu
    mu_new = mu + (B / n_new) * d
    S_new = S + S_b + (n * B / n_new) * np.outer(d, d)
    return n_new, mu_new, S_new


def covariance(n, S):
    return S / (n - 1)


# ---- weight tracker ----------------------------------------------------------

def _eps(A):
    return 1e-6 * np.trace(A) / A.shape[0]


def weight_update(state, W, m):
    """One flip-flop update of state (M, U, V) (None before the first) with
    W [R, C]; returns the new (M, U, V)."""
    W = np.asarray(W, dtype=np.float64)
    R, C = W.shape
    if state is None:
        return W.copy(), np.eye(R), np.eye(C)
    M, U, V = state
    M = m * M + (1 - m) * W
    Wc = W - M
    LV = np.linalg.cholesky(V + _eps(V) * np.eye(C))
    Wt = np.linalg.solve(LV, Wc.T).T          # Wc LV^-T: solve LV X^T = Wc^T
    U1 = Wt @ Wt.T / C
    LU = np.linalg.cholesky(U + _eps(U) * np.eye(R))
    Wu = np.linalg.solve(LU, Wc)              # LU^-1 Wc
    V1 = Wu.T @ Wu / R
    U2 = m * U + (1 - m) * U1
    V2 = m * V + (1 - m) * V1
    # symmetrize and regularize the EMA results, then fix the Kronecker
    # scale by the trace of U
    U = 0.5 * (U2 + U2.T) + _eps(U2) * np.eye(R)
    V = 0.5 * (V2 + V2.T) + _eps(V2) * np.eye(C)
    s = np.trace(U) / R
    return M, U / s, V * s


# ---- sampler -----------------------------------------------------------------

def sample_input(n, mu, S, B, seed):
    cov = covariance(n, S)
    K = cov.shape[0]
    L = np.linalg.cholesky(cov + _eps(cov) * np.eye(K))
    Z = normals(B * K, seed).reshape(B, K)
    return mu[None, :] + Z @ L.T


def sample_weight(M, U, V, seed):
    R, C = M.shape
    LU = np.linalg.cholesky(U + _eps(U) * np.eye(R))
    LV = np.linalg.cholesky(V + _eps(V) * np.eye(C))
    Z = normals(R * C, seed).reshape(R, C)
    return M + LU @ Z @ LV.T
