"""loka_grouped_gemm_fp8_ln on the GPU: the 64-group wide-ensemble workload
in one launch.  Every row of every group is checked against the oracle (Z
and Y), and every group's outputs must equal a single loka_gemm_fp8_ln call
bit for bit (same kernel body, same arithmetic order), whose X codes and
scales are checked bit for bit against the oracle's: the grouped entry
point has no codes output of its own."""

import numpy as np
import pytest
import torch

from oracle import forward
from synth.workloads import forward_case, grouped_case, to_bf16_bits
from tests.gpu_helpers import bf16_dev, check_y, check_z, host, row_sigma

pytestmark = pytest.mark.gpu


def prepare(lib, groups):
    dev_groups = []
    for g in groups:
        qw, sw, _ = lib.loka_quant_fp8(bf16_dev(g["w"]), mode="col", transpose_out=True)
        dev_groups.append({"x": bf16_dev(g["x"]), "qw": qw, "sw": sw, "bias": bf16_dev(g["bias"]),
                           "gamma": bf16_dev(g["gamma"]), "beta": bf16_dev(g["beta"])})
    return dev_groups


def test_grouped_full_workload(lib):
    groups = grouped_case()
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg, want_z=True)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (g, o) in enumerate(zip(groups, outs)):
        ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        label = f"group {i} (K={g['K']}, N={g['N']})"
        ez = check_z(host(o["z"]), ref["z"], row_sigma(ref["z"]), label)
        check_y(host(o["y"]), ref["y"], label)
        worst = max(worst, ez)
        # the same group as a single call: bitwise equal, and its X codes and scales the oracle's
        d = dg[i]
        s = lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], d["bias"], d["gamma"], d["beta"], want_z=True,
                                 want_qx=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(s["y"]), host(o["y"]), err_msg=label)
        np.testing.assert_array_equal(host(s["z"]), host(o["z"]), err_msg=label)
        np.testing.assert_array_equal(host(s["qx"]), ref["qx"], err_msg=f"{label}: X codes")
        np.testing.assert_array_equal(host(s["sx"]).view(np.uint32), ref["sx"].astype(np.float32).view(np.uint32),
                                      err_msg=f"{label}: X scales")
        np.testing.assert_array_equal(host(d["qw"]).T, ref["qw"], err_msg=f"{label}: W codes")
        np.testing.assert_array_equal(host(d["sw"]).view(np.uint32), ref["sw"].astype(np.float32).view(np.uint32),
                                      err_msg=f"{label}: W scales")
    print(f"grouped: 64 groups, every row, worst Z err {worst:.2e}")


def test_grouped_ragged_and_empty_groups(lib):
    groups = grouped_case(seed=5, groups=6, M=200)
    groups[2] = dict(groups[2], M=0, x=groups[2]["x"][:0])
    groups[4] = dict(groups[4], M=1, x=groups[4]["x"][:1])
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg, want_z=True)
    torch.cuda.synchronize()
    for i, (g, o) in enumerate(zip(groups, outs)):
        if g["x"].shape[0] == 0:
            assert o["y"].numel() == 0
            continue
        ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        check_z(host(o["z"]), ref["z"], row_sigma(ref["z"]), f"group {i}")
        check_y(host(o["y"]), ref["y"], f"group {i}")


def test_grouped_packed_weights_bit_identical(lib):
    """w_packed=True (every group's weight quantized straight into the packed
    layout) gives the same bits as row-major weights rearranged in the call."""
    groups = grouped_case(seed=9, groups=12, M=300)
    dg = prepare(lib, groups)
    dp = [dict(d, qw=lib.loka_quant_fp8(bf16_dev(g["w"]), mode="col", transpose_out="packed")[0])
          for d, g in zip(dg, groups)]
    a = lib.loka_grouped_gemm_fp8_ln(dg, want_z=True)
    b = lib.loka_grouped_gemm_fp8_ln(dp, want_z=True, w_packed=True)
    c = lib.loka_grouped_gemm_fp8_ln(dp, w_packed=True)
    torch.cuda.synchronize()
    for i in range(len(groups)):
        np.testing.assert_array_equal(host(a[i]["y"]), host(b[i]["y"]), err_msg=f"group {i}")
        np.testing.assert_array_equal(host(a[i]["z"]), host(b[i]["z"]), err_msg=f"group {i}")
        np.testing.assert_array_equal(host(a[i]["y"]), host(c[i]["y"]), err_msg=f"group {i} (no z)")


def test_grouped_many_groups_device_plan(lib):
    """More than 256 groups in one shape class: the launch plan is built on
    the device instead of being passed by value.  Every group (empty and
    ragged ones included) must equal a single call bit for bit, and a few
    are checked against the oracle."""
    groups = []
    for i in range(300):  # one shape class (K = N = 128), ragged and empty M
        m = (0, 1, 16, 17, 48)[i % 5]
        c = forward_case(max(m, 1), 128, 128, seed=1000 + i)
        groups.append(c if m > 0 else dict(c, M=0, x=c["x"][:0]))
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg, want_z=True)
    torch.cuda.synchronize()
    for i, (g, d, o) in enumerate(zip(groups, dg, outs)):
        if g["x"].shape[0] == 0:
            assert o["y"].numel() == 0
            continue
        s = lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], d["bias"], d["gamma"], d["beta"], want_z=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(s["y"]), host(o["y"]), err_msg=f"group {i}")
        np.testing.assert_array_equal(host(s["z"]), host(o["z"]), err_msg=f"group {i}")
        if i % 50 == 3:
            ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
            check_z(host(o["z"]), ref["z"], row_sigma(ref["z"]), f"group {i}")
            check_y(host(o["y"]), ref["y"], f"group {i}")


def _bitwise_like_single(lib, dg, outs, idx):
    for i in idx:
        d = dg[i]
        s = lib.loka_gemm_fp8_ln(d["x"], d["qw"], d["sw"], d["bias"], d["gamma"], d["beta"])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(s["y"]), host(outs[i]["y"]), err_msg=f"group {i}")


def test_grouped_y_only(lib):
    """Without Z (the launch the benchmark times): Y against the oracle and bit
    for bit against single calls without Z."""
    groups = grouped_case(seed=9, groups=12, M=1000)
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg)
    torch.cuda.synchronize()
    assert all("z" not in o for o in outs)
    for i, (g, o) in enumerate(zip(groups, outs)):
        ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        check_y(host(o["y"]), ref["y"], f"group {i} (K={g['K']}, N={g['N']})")
    _bitwise_like_single(lib, dg, outs, range(len(groups)))


def test_grouped_k_padding_after_nan_codes(lib):
    """Regression: code rows past K must hold zero codes in every code buffer
    of the launch.  A first launch with K = 256 and X all NaN leaves NaN codes
    in every byte of the code rows (each workgroup runs several tiles, so all
    of its buffers are used); a second launch with K = 192, whose rows are
    padded from byte 192 on, must then still equal the oracle and single
    calls (a stale NaN code times a zero weight would be NaN)."""
    poison = grouped_case(seed=21, groups=12, M=2048, dims=(256,))
    nan_bf16 = np.full_like(poison[0]["x"], 0x7FC0)
    for g in poison:
        g["x"] = nan_bf16
    lib.loka_grouped_gemm_fp8_ln(prepare(lib, poison))
    torch.cuda.synchronize()
    groups = grouped_case(seed=22, groups=12, M=2048, dims=(192,))
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg)
    torch.cuda.synchronize()
    for i, (g, o) in enumerate(zip(groups, outs)):
        ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        check_y(host(o["y"]), ref["y"], f"group {i} (K={g['K']}, N={g['N']})")
    _bitwise_like_single(lib, dg, outs, range(0, len(groups), 3))


@pytest.mark.parametrize("want_z", [False, True])
def test_grouped_with_wide_and_deep_groups(lib, want_z):
    """Groups with N = 512 or K > 512 in the mix (one launch per register
    shape class instead of the single launch): the same results."""
    groups = grouped_case(seed=13, groups=8, M=300)
    for i, (K, N) in zip((1, 4, 6), ((256, 512), (640, 128), (512, 512))):
        rng = np.random.default_rng(100 + i)
        groups[i] = dict(groups[i], K=K, N=N,
                         x=to_bf16_bits(rng.standard_normal((300, K))),
                         w=to_bf16_bits(rng.standard_normal((K, N)) / np.sqrt(K)),
                         bias=to_bf16_bits(0.1 * rng.standard_normal(N)),
                         gamma=to_bf16_bits(np.ones(N)), beta=to_bf16_bits(np.zeros(N)))
    dg = prepare(lib, groups)
    outs = lib.loka_grouped_gemm_fp8_ln(dg, want_z=want_z)
    torch.cuda.synchronize()
    for i, (g, o) in enumerate(zip(groups, outs)):
        ref = forward.gemm_ln_forward(g["x"], g["w"], g["bias"], g["gamma"], g["beta"])
        if want_z:
            check_z(host(o["z"]), ref["z"], row_sigma(ref["z"]), f"group {i}")
        check_y(host(o["y"]), ref["y"], f"group {i} (K={g['K']}, N={g['N']})")
    _bitwise_like_single(lib, dg, outs, range(len(groups)))
