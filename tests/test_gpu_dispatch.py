"""The Dispatch runtime on the GPU ([LoKA] section III-C, "Library and Recipe
Selection", with section II-C's MERE as the error).

loka_mere_z is checked against closed forms (Z = Z_ref (1 + d) gives MERE d,
Z = Z_ref gives 0) with Z_ref from the oracle, and against the oracle's own
MERE of a recipe's output.  dispatch() is run on the 16384 x 512 x 512
outlier workload: its choice must be the oracle's rule applied to the table
it measured, and the table must show what the pages report for outlier
activations -- tensorwise scaling has a larger error than rowwise."""

import numpy as np
import pytest
import torch

import fp8_precision_gemm_amd as lk
from fp8_precision_gemm_amd.dispatch import dispatch
from oracle import dispatch as odispatch
from oracle import forward, mere
from synth.workloads import forward_case, outlier_case
from tests.gpu_helpers import bf16_dev, host

pytestmark = pytest.mark.gpu


def _rows(M, n, seed=0):
    return np.sort(np.random.default_rng(seed).choice(M, size=min(n, M), replace=False)).astype(np.int64)


@pytest.mark.parametrize("d", [0.0, 0.01, -0.25])
def test_mere_closed_form(lib, d):
    c = forward_case(1024, 256, 384, seed=5, x_dist="student_t3_outliers")
    ref = forward.reference_forward(c["x"], c["w"], c["bias"])["z"]
    z = torch.from_numpy((ref * (1.0 + d)).astype(np.float32)).cuda()
    rows = _rows(1024, 300)
    m, cnt = lk.loka_mere_z(bf16_dev(c["x"]), bf16_dev(c["w"]), z, torch.from_numpy(rows).cuda(),
                            bias=bf16_dev(c["bias"]))
    assert cnt == len(rows) * 384
    # the fp32 reference and the fp32 rounding of z_ref (1 + d) differ from
    # the exact values by a few ulp
    assert abs(m - abs(d)) <= 1e-5 + 1e-5 * abs(d), m


def test_mere_matches_oracle_row_recipe(lib):
    c = forward_case(2048, 512, 512, seed=11, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    qw, sw, _ = lib.loka_quant_fp8(w, mode="col", transpose_out=True)
    z = lib.loka_gemm_fp8_ln(x, qw, sw, bf16_dev(c["bias"]), want_z=True)["z"]
    rows = _rows(2048, 256, seed=2)
    m, cnt = lk.loka_mere_z(x, w, z, torch.from_numpy(rows).cuda(), bias=bf16_dev(c["bias"]))
    o = forward.gemm_ln_forward(c["x"][rows], c["w"], c["bias"], recipe="row")
    r = forward.reference_forward(c["x"][rows], c["w"], c["bias"])
    m_ref, cnt_ref = mere.mere(o["z"], r["z"])
    assert cnt == cnt_ref
    assert abs(m - m_ref) <= 0.02 * m_ref, (m, m_ref)


def test_mere_rejects_bad_rows(lib):
    c = forward_case(64, 64, 64, seed=1)
    z = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        lk.loka_mere_z(bf16_dev(c["x"]), bf16_dev(c["w"]), z, torch.tensor([0, 64], dtype=torch.int64).cuda())


def test_dispatch_outlier_workload(lib):
    c = outlier_case()
    x, w = bf16_dev(c["x"]), bf16_dev(c["w"])
    vec = [bf16_dev(c[k]) for k in ("bias", "gamma", "beta")]
    res = dispatch(x, w, *vec, reps=30, warmup=5)
    table = {r["recipe"]: r for r in res["table"]}
    print(res)
    assert set(table) == {"tensor", "row", "mx32", "mx32_sq"} and not res["skipped"]
    for r in res["table"]:
        assert 0.0 < r["mere"] < 1.0 and r["us"] > 0.0 and r["count"] > 0
    # outlier columns stretch a single tensor scale: tensorwise is the least accurate
    assert table["tensor"]["mere"] > table["row"]["mere"]
    want = odispatch.select([(r["us"], r["mere"]) for r in res["table"]], res["baseline_us"])
    got = [r["recipe"] for r in res["table"]].index(res["choice"]) if res["choice"] != "bf16" else -1
    assert got == want
    # a baseline no recipe beats by 5 % keeps the high-precision path
    slow = dispatch(x, w, *vec, reps=5, warmup=2, baseline_us=min(r["us"] for r in res["table"]))
    assert slow["choice"] == "bf16"
