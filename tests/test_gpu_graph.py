"""Entry points captured in a HIP graph: every replay equals the eager call
bit for bit (the timing loops replay such graphs).  Outputs are cleared
before each replay, replays are separated by eager calls of the same entry
point and by synchronizations, and every replay is checked, not only the
last.  The grouped entry point copies its group table to the device inside
the call, so its graph holds a host-to-device copy node as well."""

import numpy as np
import pytest
import torch

from synth.workloads import grouped_case, outlier_case
from tests.gpu_helpers import bf16_dev, host

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _flat(out):
    if isinstance(out, dict):
        return dict(out)
    return {f"{i}.{k}": v for i, o in enumerate(out) for k, v in o.items()}


def check_replays(make, eager_again):
    """make(stream) -> (launch, outputs) prepared on `stream`; the reference is
    launch()'s eager result on that stream."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn, out = make(s)
        fn()
    s.synchronize()
    out = _flat(out)
    ref = {k: host(v) for k, v in out.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    for rep in range(REPLAYS):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(host(out[k]), ref[k], err_msg=f"replay {rep}: {k}")
        eager_again()
        torch.cuda.synchronize()


def _forward_operands(lib, M):
    c = outlier_case(M=M, dy=True)
    d = {k: bf16_dev(c[k]) for k in ("x", "w", "dy", "bias", "gamma", "beta")}
    d["qw"], d["sw"], _ = lib.loka_quant_fp8(d["w"], mode="col", transpose_out="packed")
    return d


def test_forward_graph_replays_equal_eager(lib):
    d = _forward_operands(lib, 2048 + 48)  # a ragged last tile
    vec = (d["bias"], d["gamma"], d["beta"])
    kw = dict(w_packed=True, want_z=True, want_stats=True, want_qx=True)
    check_replays(lambda s: lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], *vec, stream=s, prepare=True, **kw),
                  lambda: lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], *vec, **kw))


def test_backward_graph_replays_equal_eager(lib):
    d = _forward_operands(lib, 2048)
    qwr, swr, _ = lib.loka_quant_fp8(d["w"], mode="row", transpose_out="packed_rows")
    f = lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], d["bias"], d["gamma"], d["beta"], w_packed=True,
                             want_stats=True, want_qx=True)
    ctx = {"qx": f["qx"], "sx": f["sx"], "mean": f["mean"], "rstd": f["rstd"], "qw": d["qw"], "sw": d["sw"]}
    kw = dict(ctx=ctx, bias=d["bias"], gamma=d["gamma"], want_dz=True, want_dz_codes=True, w_packed=True,
              want_col_codes=True)
    check_replays(lambda s: lib.loka_gemm_fp8_bwd(d["dy"], d["x"], qwr, swr, stream=s, prepare=True, **kw),
                  lambda: lib.loka_gemm_fp8_bwd(d["dy"], d["x"], qwr, swr, **kw))


def test_grouped_graph_replays_equal_eager(lib):
    groups = grouped_case(seed=3, groups=10, M=700)
    dg = []
    for g in groups:
        qw, sw, _ = lib.loka_quant_fp8(bf16_dev(g["w"]), mode="col", transpose_out=True)
        dg.append({"x": bf16_dev(g["x"]), "qw": qw, "sw": sw, "bias": bf16_dev(g["bias"]),
                   "gamma": bf16_dev(g["gamma"]), "beta": bf16_dev(g["beta"])})
    check_replays(lambda s: lib.loka_grouped_gemm_fp8_ln(dg, want_z=True, stream=s, prepare=True),
                  lambda: lib.loka_grouped_gemm_fp8_ln(dg, want_z=True))
