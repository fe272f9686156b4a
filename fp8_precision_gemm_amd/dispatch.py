"""Dispatch: per-operation recipe selection ([LoKA] section III-C, "Library
and Recipe Selection"; the error measure is section II-C's MERE).

For one linear + LayerNorm operation, given its own bf16 operands, every
recipe of this library runs on them:

  * its error is the MERE of its Z against the fp32 reference X W + b on
    sampled rows (loka_mere_z);
  * its time is measured with HIP events around back-to-back launches on one
    stream.  For the square-block recipe the time includes quantizing X,
    since X arrives in bf16 here.

The high-precision path is timed the same way, or its time is given.  The
native loka_dispatch_select then applies the pages' rule: MERE below the
threshold, speedup above the factor, shortest time.  This module only
marshals arguments and times launches; every step of the recipes runs in the
library.
"""

import torch

from . import LokaError, loka_dispatch_select, loka_gemm_fp8_ln, loka_mere_z, loka_quant_fp8

# recipe -> (forward x_mode, weight quantization mode)
RECIPES = {
    "tensor": ("tensor", "tensor"),
    "row": ("row", "col"),
    "mx32": ("mx32_row", "mx32_col"),
    "mx32_sq": ("mx32_sq", "mx32_sq"),
}


def _time_us(fn, reps, warmup, stream):
    for _ in range(warmup):
        fn()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) * 1e3 / reps


def high_precision_us(x, w, bias=None, gamma=None, beta=None, eps=1e-5, reps=50, warmup=10, stream=None):
    """Time of the bf16 path the recipes are compared with: the framework's
    bf16 linear (a library GEMM) followed by its LayerNorm, on `stream`."""
    stream = stream or torch.cuda.current_stream()
    wt = w.t().contiguous()
    N = w.shape[1]

    def run():
        with torch.cuda.stream(stream):
            z = torch.nn.functional.linear(x, wt, bias)
            return torch.nn.functional.layer_norm(z, (N,), gamma, beta, eps)

    return _time_us(run, reps, warmup, stream)


def _prepare(name, x, w, bias, gamma, beta, eps, stream):
    """(launch without optional outputs, Z for the error) of one recipe, or
    None when the recipe does not take this shape."""
    x_mode, w_mode = RECIPES[name]
    M, K = x.shape
    if name in ("mx32", "mx32_sq") and K % 32:
        return None
    if name == "mx32_sq" and M % 32:
        return None
    # the packed weight layout first (the weight-resident shapes); else the
    # row-major layout, which every forward shape takes
    for layout in ("packed", True):
        try:
            qw, sw, _ = loka_quant_fp8(w, mode=w_mode, transpose_out=layout, stream=stream)
            kw = dict(x_mode=x_mode, w_packed=layout == "packed", stream=stream, eps=eps)
            if name == "mx32_sq":
                qx, sx, _ = loka_quant_fp8(x, mode="mx32_sq", stream=stream)
                z = loka_gemm_fp8_ln(qx, qw, sw, bias, gamma, beta, x_scales=sx, want_z=True, **kw)["z"]
                fwd, _ = loka_gemm_fp8_ln(qx, qw, sw, bias, gamma, beta, x_scales=sx, prepare=True, **kw)

                def launch(fwd=fwd, qx=qx, sx=sx):
                    loka_quant_fp8(x, mode="mx32_sq", codes=qx, scales=sx, stream=stream)
                    fwd()
                return launch, z
            z = loka_gemm_fp8_ln(x, qw, sw, bias, gamma, beta, want_z=True, **kw)["z"]
            fwd, _ = loka_gemm_fp8_ln(x, qw, sw, bias, gamma, beta, prepare=True, **kw)
            return fwd, z
        except LokaError as e:
            if e.status != 2:  # anything but "unsupported shape" is a real error
                raise
    return None


def dispatch(x, w, bias=None, gamma=None, beta=None, eps=1e-5, recipes=tuple(RECIPES), sample_rows=256, reps=50,
             warmup=10, mere_max=0.2, min_speedup=1.05, baseline_us=None, seed=0, stream=None):
    """Choose the recipe for one operation (x bf16 [M, K], w bf16 [K, N]).

    Returns {"choice": recipe name or "bf16", "table": [{"recipe", "us",
    "mere", "count"}...], "baseline_us": float, "skipped": [names]}."""
    stream = stream or torch.cuda.current_stream()
    M = x.shape[0]
    g = torch.Generator().manual_seed(seed)
    rows = torch.randperm(M, generator=g)[:min(sample_rows, M)].sort().values.to(torch.int64).cuda()
    table, skipped = [], []
    for name in recipes:
        prep = _prepare(name, x, w, bias, gamma, beta, eps, stream)
        if prep is None:
            skipped.append(name)
            continue
        launch, z = prep
        mere, count = loka_mere_z(x, w, z, rows, bias=bias, stream=stream)
        table.append({"recipe": name, "us": _time_us(launch, reps, warmup, stream), "mere": mere, "count": count})
    if baseline_us is None:
        baseline_us = high_precision_us(x, w, bias, gamma, beta, eps, reps, warmup, stream)
    idx = loka_dispatch_select([(r["us"], r["mere"]) for r in table], baseline_us, mere_max, min_speedup)
    return {"choice": table[idx]["recipe"] if idx >= 0 else "bf16", "table": table, "baseline_us": baseline_us,
            "skipped": skipped}
