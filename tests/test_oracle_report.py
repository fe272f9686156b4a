"""Pins for the oracle's per-layer error report ([LoKA] section II-C, MERE;
section III-A2, per-layer error quantification):
  * lossless inputs (e4m3-grid values whose group maxima are 448 * 2**j) give
    MERE 0 for Z and Y, over every nonzero reference entry;
  * the report's numbers are the MERE of the quantized forward's outputs
    against the unquantized reference, recomputed here from the definition
    (mean |out - ref| / |ref| over ref != 0);
  * quantization does change a random problem: the MERE is positive and
    bounded by e4m3's relative half-spacing times the row's conditioning;
  * the grouped report is the list of the groups' reports, and its summary
    the mean and the largest of them."""

import numpy as np

from oracle import codec, report
from synth.workloads import forward_case, grouped_case, to_bf16_bits


def test_lossless_report_is_zero():
    rng = np.random.default_rng(31)
    M, K, N = 24, 64, 32
    vals = np.array([1.0, 1.125, 1.25, 1.5, 1.75, 2.0, 3.0, 0.5, 0.25])
    x = rng.choice(np.concatenate([vals, -vals]), size=(M, K))
    x[:, 0] = 448.0
    w = rng.choice(np.concatenate([vals, -vals]), size=(K, N))
    w[0, :] = 448.0
    x = np.ldexp(x, rng.integers(-8, 2, size=M)[:, None])
    w = np.ldexp(w, rng.integers(-12, -6, size=N)[None, :])
    c = forward_case(M, K, N, seed=3, gamma_var=0.1, beta_var=0.1)
    r = report.forward_error(to_bf16_bits(x), to_bf16_bits(w), c["bias"], c["gamma"], c["beta"], "row")
    for k in ("z", "y"):
        assert r[k]["mere"] == 0.0 and r[k]["count"] > 0


def test_report_matches_definition_and_is_positive():
    c = forward_case(64, 128, 64, seed=5, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    r = report.forward_error(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], "row")
    # recompute from the definition on the same outputs
    from oracle import forward
    out = forward.gemm_ln_forward(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe="row")
    x, w, b = codec.bf16_to_f64(c["x"]), codec.bf16_to_f64(c["w"]), codec.bf16_to_f64(c["bias"])
    zref = x @ w + b[None, :]
    sel = zref != 0
    want = np.mean(np.abs(out["z"][sel] - zref[sel]) / np.abs(zref[sel]))
    assert abs(r["z"]["mere"] - want) <= 1e-15 * want and r["z"]["count"] == int(sel.sum())
    assert 1e-3 < r["z"]["mere"] < 1.0
    assert 1e-4 < r["y"]["mere"] < 1.0


def test_grouped_report_and_summary():
    gs = grouped_case(groups=3, M=16)
    per = report.grouped_error(gs)
    assert len(per) == 3
    for g, p in zip(gs, per):
        assert p == report.forward_error(g["x"], g["w"], g["bias"], g["gamma"], g["beta"], "row")
    s = report.summarize(per)
    zs = [p["z"]["mere"] for p in per]
    assert s["z"]["max"] == max(zs) and s["z"]["argmax"] == int(np.argmax(zs))
    assert abs(s["z"]["mean"] - np.mean(zs)) <= 1e-15


def test_backward_report_small():
    c = forward_case(64, 64, 64, seed=6, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1, dy_var=1e-3)
    r = report.backward_error(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"])
    for k in ("dz", "dx", "dw"):
        assert 0 < r[k]["mere"] < 10 and r[k]["count"] > 0


def test_row_blocks_give_the_same_report():
    """Rowwise and MX rows are independent: the report over row blocks equals
    the one over the whole matrix exactly; the tensor recipe ignores the
    blocking (its scale spans every row)."""
    c = forward_case(200, 64, 64, seed=8, x_dist="student_t3_outliers", gamma_var=0.1, beta_var=0.1)
    for recipe in ("row", "mx32", "tensor"):
        whole = report.forward_error(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe)
        blocks = report.forward_error(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe, chunk_rows=64)
        for k in ("z", "y"):
            assert whole[k]["count"] == blocks[k]["count"]
            assert abs(whole[k]["mere"] - blocks[k]["mere"]) <= 1e-15 * whole[k]["mere"]
