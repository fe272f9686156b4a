"""Per-layer quantization-error report: the MERE of each workload's outputs
against the unquantized bf16 reference.

Test infrastructure only (see the package docstring).

Source: [LoKA] section II-C ("Error Analysis": the mean element-wise
relative error of a low-precision linear layer against a higher-precision
reference) and section III-A2 ("Offline Error Quantification": MERE and
speedup reported per linear layer, so layers whose error is too large can be
flagged).  Reading R10: MERE is taken over the entries whose reference is
nonzero and the count of those entries is reported with it; the reference is
the same block on the unquantized bf16 inputs taken exactly in fp64
(forward.reference_forward, backward.reference_backward).

Each workload is one "layer": the forward reports Z (the linear output the
pages define MERE on) and Y (after the LayerNorm); the training step also
reports dZ, dX and dW; the grouped workload reports every group.
"""

import numpy as np

from .backward import gemm_ln_backward, reference_backward
from .forward import gemm_ln_forward, reference_forward
from .mere import mere


def _pair(out, ref):
    v, n = mere(out, ref)
    return {"mere": v, "count": n}


def forward_error(x_bits, w_bits, bias_bits, gamma_bits, beta_bits, recipe, eps=1e-5, pmap=map, chunk_rows=None):
    """MERE of Z and Y of one forward against the bf16 reference.

    With the rowwise and MX recipes every row is quantized and normalized on
    its own, so the rows may be taken in blocks of chunk_rows (a multiple of
    32), each block through `pmap` (e.g. a thread pool's map); the outputs,
    and so the report, are the same as for the whole matrix.  The tensor
    recipe's scale spans all rows, so it always runs whole."""
    M = x_bits.shape[0]
    if chunk_rows is None or recipe not in ("row", "mx32") or M <= chunk_rows:
        spans = [(0, M)]
    else:
        assert chunk_rows % 32 == 0
        spans = [(lo, min(lo + chunk_rows, M)) for lo in range(0, M, chunk_rows)]

    def one(span):
        lo, hi = span
        out = gemm_ln_forward(x_bits[lo:hi], w_bits, bias_bits, gamma_bits, beta_bits, eps, recipe=recipe)
        ref = reference_forward(x_bits[lo:hi], w_bits, bias_bits, gamma_bits, beta_bits, eps)
        return out["z"], out["y"], ref["z"], ref["y"]

    parts = list(pmap(one, spans))
    z, y, zr, yr = (np.concatenate([p[i] for p in parts]) for i in range(4))
    return {"z": _pair(z, zr), "y": _pair(y, yr)}


def backward_error(x_bits, w_bits, dy_bits, bias_bits, gamma_bits, beta_bits, eps=1e-5):
    """MERE of dZ, dX and dW of the rowwise training step (reading R8)
    against the exact gradients of the unquantized block."""
    out = gemm_ln_backward(x_bits, w_bits, dy_bits, bias_bits, gamma_bits, beta_bits, eps)
    ref = reference_backward(x_bits, w_bits, dy_bits, bias_bits, gamma_bits, beta_bits, eps)
    return {k: _pair(out[k], ref[k]) for k in ("dz", "dx", "dw")}


def grouped_error(groups, eps=1e-5, pmap=map):
    """Per-group forward MERE (rowwise recipe) of a grouped workload, the
    groups through `pmap`."""
    return list(pmap(lambda g: forward_error(g["x"], g["w"], g.get("bias"), g.get("gamma"), g.get("beta"), "row",
                                             eps), groups))


def summarize(per_group):
    """Across groups: the mean and the largest MERE of Z and Y."""
    out = {}
    for k in ("z", "y"):
        v = np.array([g[k]["mere"] for g in per_group])
        out[k] = {"mean": float(v.mean()), "max": float(v.max()), "argmax": int(v.argmax())}
    return out
