"""Seeded synthetic inputs for the FP8 GEMM + LayerNorm block.

This module draws random inputs and nothing else: it holds none of the
block's arithmetic (no quantization, GEMM or normalization), so the oracle
and the HIP library can both be fed from it.  Inputs are produced as bf16
bit patterns (numpy uint16): draws are float64 (NumPy PCG64), rounded to
fp32 and then to bf16, each rounding to nearest-even.

Distribution notation: N(mu, var) names the variance.  Per configuration:

  tensor-recipe case   X[512,256] ~ N(0,1); W[256,256] ~ N(0,1/256);
                       bias ~ N(0,0.01); gamma = 1, beta = 0
  outlier case         X[16384,512] ~ Student-t(3) with round(1% of K)
                       columns (chosen by a seeded permutation) scaled x50;
                       W[512,512] ~ N(0,1/512); bias ~ N(0,0.01);
                       gamma ~ N(1,0.1); beta ~ N(0,0.1)
  MX case              X[65536,1024] = exp(xi_m) * N(0,1), xi_m ~ N(0,1)
                       per row (log-normal row magnitude, sigma 1);
                       W[1024,256] ~ N(0,1/1024); bias ~ N(0,0.01);
                       gamma = 1, beta = 0
  training step        the outlier case plus dY[16384,512] ~ N(0,1e-3)
  grouped case         64 groups, M = 8192; K_g then N_g drawn with
                       rng.choice([128,192,256,384], 64); per group in order
                       X ~ N(0,1), W ~ N(0,1/K_g), bias ~ N(0,0.01);
                       gamma = 1, beta = 0

Draw order within a case: shapes, X, W, bias, gamma, beta, dY.  Seed 0.
The pages' own workloads (production recommendation-model traces) are not
available; these stand in for them, with the heavy tails and outlier
channels that the pages show ordinary N(0,1) tests miss.
"""

import numpy as np

GROUP_DIMS = (128, 192, 256, 384)


def to_bf16_bits(a):
    """float64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16."""
    u = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _normal(rng, shape, var):
    return rng.standard_normal(shape) * np.sqrt(var)


def draw_x(rng, M, K, dist):
    """X[M,K] as float64 draws for the named distribution."""
    if dist == "normal":
        return rng.standard_normal((M, K))
    if dist == "student_t3_outliers":
        x = rng.standard_t(3, size=(M, K))
        n_out = int(round(0.01 * K))
        cols = rng.permutation(K)[:n_out]
        x[:, cols] *= 50.0
        return x
    if dist == "lognormal_rows":
        mag = np.exp(rng.standard_normal(M))
        return mag[:, None] * rng.standard_normal((M, K))
    raise ValueError(dist)


def forward_case(M, K, N, seed=0, x_dist="normal", bias_var=0.01, gamma_var=None,
                 beta_var=None, with_bias=True, dy_var=None):
    """One forward (and optional backward) input set as bf16 bit patterns.

    gamma_var/beta_var None means gamma = 1, beta = 0 (still returned as
    explicit bf16 vectors).  with_bias False returns bias None (No Bias)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = draw_x(rng, M, K, x_dist)
    w = _normal(rng, (K, N), 1.0 / K)
    bias = _normal(rng, N, bias_var)
    gamma = np.ones(N) if gamma_var is None else 1.0 + _normal(rng, N, gamma_var)
    beta = np.zeros(N) if beta_var is None else _normal(rng, N, beta_var)
    case = {
        "M": M, "K": K, "N": N, "x": to_bf16_bits(x), "w": to_bf16_bits(w),
        "bias": to_bf16_bits(bias) if with_bias else None,
        "gamma": to_bf16_bits(gamma), "beta": to_bf16_bits(beta),
    }
    if dy_var is not None:
        case["dy"] = to_bf16_bits(_normal(rng, (M, N), dy_var))
    return case


def tensor_case(seed=0, M=512, K=256, N=256):
    """Per-tensor e4m3 forward, X[512,256] ~ N(0,1)."""
    return forward_case(M, K, N, seed, "normal")


def outlier_case(seed=0, M=16384, K=512, N=512, dy=False):
    """Rowwise-X / per-column-W forward on Student-t(3) with outlier columns."""
    return forward_case(M, K, N, seed, "student_t3_outliers", gamma_var=0.1, beta_var=0.1,
                        dy_var=1e-3 if dy else None)


def mx_case(seed=0, M=65536, K=1024, N=256):
    """MX32 forward on rows with log-normal magnitudes."""
    return forward_case(M, K, N, seed, "lognormal_rows")


def grouped_case(seed=0, groups=64, M=8192, dims=GROUP_DIMS):
    """Wide-ensemble grouped forward: per-group K and N drawn from `dims`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Ks = rng.choice(np.array(dims), groups)
    Ns = rng.choice(np.array(dims), groups)
    out = []
    for K, N in zip(Ks.tolist(), Ns.tolist()):
        x = rng.standard_normal((M, K))
        w = _normal(rng, (K, N), 1.0 / K)
        bias = _normal(rng, N, 0.01)
        out.append({"M": M, "K": K, "N": N, "x": to_bf16_bits(x), "w": to_bf16_bits(w),
                    "bias": to_bf16_bits(bias), "gamma": to_bf16_bits(np.ones(N)),
                    "beta": to_bf16_bits(np.zeros(N))})
    return out
