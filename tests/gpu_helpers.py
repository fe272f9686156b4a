"""Shared pieces of the GPU parity tests: tensor conversion and the
tolerance checks the block's parity is judged by.

Tolerances (each derived from the arithmetic, none tuned to pass):
  * FP8 codes, FP8 scales, E8M0 scales: bit-exact.
  * pre-norm Z (fp32): max_{m,n} |z - z_ref| / max(|z_ref|, sigma_m) <= 1e-3,
    sigma_m = sqrt(var_m + eps) the row's LayerNorm scale from the oracle.
    Elementwise relative error is undefined where z_ref crosses zero, and
    what reaches the output is the error relative to the row's scale.
  * bf16 Y: |y - y_ref| <= 2 ulp_bf16(y_ref) or <= 1e-2 absolute (y_ref is
    the single RNE rounding of the fp64 value; the kernel rounds from fp32).
"""

import numpy as np
import torch

from oracle import codec

DEV = "cuda"
Z_TOL = 1e-3


def bf16_dev(bits):
    """numpy bf16 bit patterns -> bf16 CUDA tensor (same bytes)."""
    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    """CUDA tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def unpack_packed(packed, R, C):
    """Codes in the fragment-interleaved ("packed") layout -> [R, C] row-major,
    plus the zero padding check.  The layout, as the header states it: one
    2 KiB block per 16 rows and 128-column chunk, block (rt, c) at
    (rt * nch + c) * 2048, byte 256 p + 16 i + b = element [16 rt + i][128 c + 16 p + b]."""
    nch = (C + 127) // 128
    flat = np.ascontiguousarray(packed).reshape(-1)
    assert flat.size == R * nch * 128, (flat.size, R, C)
    blocks = flat.reshape(R // 16, nch, 8, 16, 16)         # [rt, c, p, i, b]
    full = blocks.transpose(0, 3, 1, 2, 4).reshape(R, nch * 128)  # [rt, i, c, p, b]
    assert not full[:, C:].any(), "padding past the last column is not zero"
    return full[:, :C]


def bf16_ulp(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def check_y(y_bits_gpu, y_ref, label=""):
    """bf16 output check: within 2 ulp of the reference or 1e-2 absolute."""
    y = codec.bf16_to_f64(y_bits_gpu)
    err = np.abs(y - y_ref)
    ok = (err <= 2 * bf16_ulp(y_ref)) | (err <= 1e-2)
    if not ok.all():
        i = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(f"{label} Y mismatch at {i}: gpu {y[i]} ref {y_ref[i]} "
                             f"({int((~ok).sum())} of {ok.size} outside tolerance)")
    return float(err.max())


def z_metric(z_gpu, z_ref, sigma):
    """max |z - z_ref| / max(|z_ref|, sigma_row)."""
    den = np.maximum(np.abs(z_ref), sigma[:, None])
    return float(np.max(np.abs(z_gpu.astype(np.float64) - z_ref) / den))


def check_z(z_gpu, z_ref, sigma, label="", tol=Z_TOL):
    e = z_metric(z_gpu, z_ref, sigma)
    assert e <= tol, f"{label} pre-norm Z error {e:.3e} > {tol}"
    return e


def row_sigma(z_ref, eps=1e-5):
    v = ((z_ref - z_ref.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    return np.sqrt(v + float(np.float32(eps)))


def sample_rows(M, n, seed=0):
    """Sorted row indices: the first and last 64 rows plus a seeded sample."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(64, M))
    tail = np.arange(max(0, M - 64), M)
    mid = rng.choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


def oracle_forward_blocks(forward_fn, x_bits, *args, rows_per_block=4096, **kw):
    """The oracle forward of every row of X, taken in blocks of rows (rows are
    independent under the rowwise and MX recipes, so the result is the same
    as one call on all rows): the per-row outputs concatenated, the weight's
    codes and scales from the first block."""
    M = x_bits.shape[0]
    parts = [forward_fn(x_bits[lo:lo + rows_per_block], *args, **kw) for lo in range(0, M, rows_per_block)]
    out = dict(parts[0])
    for k in ("y_bits", "y", "z", "mean", "rstd", "qx", "sx"):
        out[k] = np.concatenate([p[k] for p in parts])
    return out
