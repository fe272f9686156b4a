"""The C ABI on the CPU: the library loads, exports every function that
include/loka_fp8.h declares, and rejects every invalid call before it
touches the GPU (no compute call is made here)."""

import ctypes
import os
import re
import subprocess

import pytest

import fp8_precision_gemm_amd as lk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loka_fp8.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lk.library_path):
        from fp8_precision_gemm_amd import build
        build.build()
    return lk.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loka_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("loka_quant_fp8", "loka_gemm_fp8_ln", "loka_gemm_fp8_bwd", "loka_grouped_gemm_fp8_ln"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lk.library_path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (loka_[a-z0-9_]+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_helpers(lib):
    assert lib.loka_abi_version() == 3
    for code, name in lk.STATUS.items():
        assert lib.loka_status_string(code).decode() == name


def test_struct_layouts_match_header():
    """Field order and count of the ctypes mirrors against the header's structs."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for cname, py in [("loka_quant_args", lk.QuantArgs), ("loka_fwd_args", lk.FwdArgs),
                      ("loka_bwd_args", lk.BwdArgs), ("loka_group_desc", lk.GroupDesc),
                      ("loka_grouped_args", lk.GroupedArgs)]:
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + cname + ";", text).group(1)
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if not decl:
                continue
            names = decl.split()[-1] if "," not in decl else None
            if names is None:  # "int64_t rows, cols, ld"
                first, *rest = decl.split(",")
                fields.append(first.split()[-1].lstrip("*"))
                fields += [r.strip().lstrip("*") for r in rest]
            else:
                fields.append(names.lstrip("*"))
        assert [f for f, _ in py._fields_] == fields, cname


FAKE = 0x100000  # an aligned, never-dereferenced address: validation fails first


def _fwd(**kw):
    a = lk.FwdArgs(M=128, N=256, K=256, x_mode=1, flags=0, eps=1e-5, x=FAKE, qw=FAKE, sw=FAKE, y=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _call(lib, fn, a):
    return getattr(lib, fn)(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=100), 2), (dict(N=2048), 2), (dict(N=0), 2), (dict(K=20), 2), (dict(K=4096), 2),
    (dict(M=-1), 1), (dict(x_mode=2), 1), (dict(x_mode=9), 1), (dict(flags=4), 1), (dict(flags=7), 1),
    # BlockNorm + Hard Swish (flag 2): row recipe, N % 256, K <= 1024, no gamma/beta/mean/rstd
    (dict(flags=2, x_mode=0), 2), (dict(flags=2, x_mode=3), 2), (dict(flags=2, N=320), 2), (dict(flags=2, N=8448), 2),
    (dict(flags=2, K=1040), 2), (dict(flags=2, gamma=FAKE), 1), (dict(flags=2, rstd=FAKE), 1),
    (dict(flags=2), 4), (dict(flags=2, N=4096, K=1024), 4),  # valid: stops at the missing relayout workspace
    (dict(flags=1, N=1024), 2),  # the packed weight layout exists only for the weight-resident shapes
    (dict(flags=1, N=512, K=1024), 2),
    (dict(eps=float("nan")), 1), (dict(eps=-1.0), 1),
    (dict(x=None), 1), (dict(qw=None), 1), (dict(sw=None), 1), (dict(y=None), 1),
    (dict(x=FAKE + 8), 3), (dict(bias=FAKE + 2), 3), (dict(z=FAKE + 4), 3),
    (dict(x_mode=3, K=48), 2),
    (dict(x_mode=0), 4),  # tensor recipe needs the amax workspace
    (dict(x_mode=1), 4),  # a row-major weight on a resident shape needs the relayout workspace
    (dict(x_mode=0, flags=1), 4),
])
def test_forward_validation(lib, kw, status):
    a = _fwd(**kw)
    assert _call(lib, "loka_gemm_fp8_ln", a) == status
    assert lib.loka_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(N=100), 2), (dict(M=-1), 1), (dict(x_mode=9), 1), (dict(flags=4), 1), (dict(x=None), 1),
    (dict(x=FAKE + 8), 3), (dict(eps=float("nan")), 1), (dict(flags=2, gamma=FAKE), 1),
    # a valid call whose workspace would exceed the fixed scratch: the row-major weight of a
    # 4096 x 512 BlockNorm needs 2 MiB rearranged
    (dict(flags=2, N=4096, K=512), 2),
])
def test_noalloc_validation(lib, kw, status):
    """The allocation-free forward validates exactly as loka_gemm_fp8_ln, then
    refuses calls whose workspace exceeds its fixed scratch (before any HIP
    call), and ignores the workspace fields."""
    a = _fwd(**kw)
    a.workspace, a.workspace_bytes = FAKE, 1 << 30
    assert _call(lib, "loka_gemm_fp8_ln_noalloc", a) == status
    msg = lib.loka_last_error().decode()
    assert msg
    if kw.get("N") == 4096:
        assert "scratch" in msg and str(1 << 20) in msg
        assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(a)) > (1 << 20)


def test_noalloc_empty_batch_is_a_noop(lib):
    assert _call(lib, "loka_gemm_fp8_ln_noalloc", _fwd(M=0, x=None, qw=None, sw=None, y=None)) == 0


def test_forward_empty_batch_is_a_noop(lib):
    assert _call(lib, "loka_gemm_fp8_ln", _fwd(M=0, x=None, qw=None, sw=None, y=None)) == 0


def test_forward_workspace_sizes(lib):
    a = _fwd(x_mode=0)
    need = lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(a))
    assert need > 0
    a.workspace = FAKE
    a.workspace_bytes = need - 4
    assert _call(lib, "loka_gemm_fp8_ln", a) == 4
    a.workspace = FAKE + 4
    a.workspace_bytes = need
    assert _call(lib, "loka_gemm_fp8_ln", a) == 3
    # row recipe: only the packed copy of a row-major weight (N * ceil(K/128) * 128 bytes) ...
    assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(_fwd(x_mode=1))) == 256 * 256
    assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(_fwd(x_mode=1, K=144))) == 256 * 256
    # ... none when the weight comes packed, or on shapes the resident kernel does not take
    assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(_fwd(x_mode=1, flags=1))) == 0
    assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(_fwd(x_mode=1, N=1024))) == 0
    packed = lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(_fwd(x_mode=0, flags=1)))
    assert 0 < packed < need


def _quant(**kw):
    a = lk.QuantArgs(rows=64, cols=64, ld=64, src_dtype=0, fmt=0, mode=1, transpose_out=0, src=FAKE, codes=FAKE,
                     scales=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), 1), (dict(ld=32), 1), (dict(src_dtype=2), 1), (dict(fmt=3), 1), (dict(mode=6), 1),
    (dict(transpose_out=4), 1), (dict(transpose_out=-1), 1), (dict(transpose_out=2, rows=40), 2),
    (dict(transpose_out=3, rows=40), 2),
    (dict(cols=40, ld=40), 2), (dict(mode=3, cols=48, ld=48), 2),
    (dict(mode=4, rows=48), 2), (dict(transpose_out=1, rows=40), 2), (dict(ld=68), 3),
    (dict(mode=5, rows=48), 2), (dict(mode=5, cols=48, ld=48), 2), (dict(mode=5, amax=FAKE), 1),
    (dict(src=None), 1), (dict(codes=None), 1), (dict(scales=None), 1), (dict(mode=3, amax=FAKE), 1),
    (dict(codes=FAKE + 1), 3), (dict(mode=0), 4), (dict(mode=2), 4),
])
def test_quant_validation(lib, kw, status):
    assert _call(lib, "loka_quant_fp8", _quant(**kw)) == status


def test_quant_empty_is_a_noop(lib):
    assert _call(lib, "loka_quant_fp8", _quant(rows=0, src=None, codes=None, scales=None)) == 0
    assert lib.loka_quant_workspace_size(ctypes.byref(_quant(mode=3))) == 0
    assert lib.loka_quant_workspace_size(ctypes.byref(_quant(mode=2))) > 0


def _bwd(**kw):
    a = lk.BwdArgs(M=128, N=256, K=256, flags=0, dy=FAKE, qx=FAKE, sx=FAKE, mean=FAKE, rstd=FAKE, qw=FAKE, sw=FAKE,
                   x=FAKE, qw_row=FAKE, sw_row=FAKE, dx=FAKE, dw=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(flags=8), 1), (dict(K=96), 2), (dict(K=2048), 2), (dict(M=24), 2), (dict(N=96), 2),
    # the column-code outputs belong to the ROW recipe; the square-block
    # recipe's packed weights need qw_row (the packed dgrad weight)
    (dict(flags=6), 4), (dict(flags=6, qw_row=None), 1), (dict(flags=2, xc_codes=FAKE), 1),
    (dict(flags=2, dzc_scales=FAKE), 1),
    (dict(xc_codes=FAKE + 1), 3), (dict(dzc_scales=FAKE + 2), 3),
    (dict(flags=4), 4), (dict(xc_codes=FAKE, xc_scales=FAKE, dzc_codes=FAKE, dzc_scales=FAKE), 4),
    # the square-block recipe: N, K <= 512, M % 32 == 0, the codes required, mean/rstd unless NO_LN
    (dict(flags=2, N=640), 2), (dict(flags=2, K=576), 2), (dict(flags=2, M=48), 2), (dict(flags=2, qx=None), 1),
    (dict(flags=2, sw=None), 1), (dict(flags=2, rstd=None), 1), (dict(flags=2, x=None, qw_row=None, sw_row=None), 4),
    (dict(flags=3, mean=None, rstd=None, x=None), 4),
    (dict(dy=None), 1), (dict(dw=None), 1), (dict(mean=None), 1), (dict(qx=None), 1),
    (dict(flags=1, dgamma=FAKE), 1), (dict(dz=FAKE + 4), 3),
    ({}, 4),  # the backward always needs its workspace
])
def test_backward_validation(lib, kw, status):
    assert _call(lib, "loka_gemm_fp8_bwd", _bwd(**kw)) == status


def test_square_backward_workspace_is_smaller(lib):
    # no fp32 dZ and no column maxima or scales: only the codes and block scales
    row = lib.loka_gemm_fp8_bwd_workspace_size(ctypes.byref(_bwd(M=16384, N=512, K=512)))
    sq = lib.loka_gemm_fp8_bwd_workspace_size(ctypes.byref(_bwd(M=16384, N=512, K=512, flags=2)))
    assert row - sq >= 16384 * 512 * 4


def test_backward_literal_reading_needs_no_context(lib):
    a = _bwd(flags=1, qx=None, sx=None, mean=None, rstd=None, qw=None, sw=None)
    assert _call(lib, "loka_gemm_fp8_bwd", a) == 4  # past the context checks, stops at the workspace


def test_grouped_validation(lib):
    descs = (lk.GroupDesc * 2)()
    descs[0] = lk.GroupDesc(M=64, N=128, K=128, x=FAKE, qw=FAKE, sw=FAKE, y=FAKE)
    descs[1] = lk.GroupDesc(M=64, N=96, K=128, x=FAKE, qw=FAKE, sw=FAKE, y=FAKE)
    a = lk.GroupedArgs(num_groups=2, x_mode=1, eps=1e-5, groups=descs)
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 2
    assert "group 1" in lib.loka_last_error().decode()
    descs[1].N = 128
    descs[1].y = FAKE + 2
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 3
    descs[1].y = FAKE
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 4
    plain = lib.loka_grouped_workspace_size(ctypes.byref(a))
    a.flags = 1  # packed weights: no relayout copies in the workspace
    assert lib.loka_grouped_workspace_size(ctypes.byref(a)) == plain - 2 * 128 * 128
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 4
    a.flags = 2
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 1
    a.flags = 0
    a.x_mode = 0
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 2
    a.x_mode = 1
    a.num_groups = 0
    assert lib.loka_grouped_gemm_fp8_ln(ctypes.byref(a), None) == 0


def test_product_path_refuses_without_library(monkeypatch, tmp_path):
    """No fallback: a missing library is an error, not a silent CPU path."""
    monkeypatch.setattr(lk, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lk, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        lk.library()


def test_probe_and_mere_validation(lib):
    """The Probe and MERE entry points check their arguments before any
    launch (no GPU work happens on these paths)."""
    a = lk.ProbeInputArgs(B=16, K=0, n_old=0, T=FAKE, mu=FAKE, S=FAKE)
    assert lib.loka_probe_input_update(ctypes.byref(a), None) == 2          # K out of range
    a.K = 64
    a.T = None
    assert lib.loka_probe_input_update(ctypes.byref(a), None) == 1          # missing input
    a.T = FAKE
    assert lib.loka_probe_input_update(ctypes.byref(a), None) == 4          # no workspace
    w = lk.ProbeWeightArgs(R=64, C=64, m=1.0, first=0, W=FAKE, M=FAKE, U=FAKE, V=FAKE, info=FAKE)
    assert lib.loka_probe_weight_update(ctypes.byref(w), None) == 1         # momentum must be < 1
    w.m = 0.9
    w.C = 4096
    assert lib.loka_probe_weight_update(ctypes.byref(w), None) == 2
    w.C = 64
    assert lib.loka_probe_weight_update(ctypes.byref(w), None) == 4
    w.first = 1
    assert lib.loka_probe_weight_workspace_size(ctypes.byref(w)) == 0       # initializing needs none
    si = lk.ProbeSampleInputArgs(B=8, K=32, n=1, mu=FAKE, S=FAKE, seed=1, out=FAKE, info=FAKE)
    assert lib.loka_probe_sample_input(ctypes.byref(si), None) == 1         # n >= 2 for a covariance
    sw = lk.ProbeSampleWeightArgs(R=32, C=32, M=FAKE, U=FAKE, V=FAKE, seed=1, out=FAKE, info=None)
    assert lib.loka_probe_sample_weight(ctypes.byref(sw), None) == 1
    m = lk.MereArgs(M=64, N=64, K=4096, S=8, x=FAKE, w=FAKE, z=FAKE, rows=FAKE, out=FAKE)
    assert lib.loka_mere_z(ctypes.byref(m), None) == 2                      # K > 2048
    m.K = 64
    m.S = 0
    assert lib.loka_mere_z(ctypes.byref(m), None) == 1
    m.S = 8
    assert lib.loka_mere_z(ctypes.byref(m), None) == 4
    assert lib.loka_mere_workspace_size(ctypes.byref(m)) == 8 * 3 * 8


def test_fused_y_square_validation(lib):
    a = _fwd(x_mode=1, N=256, K=256, M=128)
    a.y_codes = FAKE
    assert lib.loka_gemm_fp8_ln(ctypes.byref(a), None) == 1                 # y_scales missing
    a.y_scales = FAKE
    a.N = 384
    assert lib.loka_gemm_fp8_ln(ctypes.byref(a), None) == 2                 # N must be 256 or 512
    a.N = 256
    a.M = 144
    assert lib.loka_gemm_fp8_ln(ctypes.byref(a), None) == 2                 # M % 32


def test_hip_error_path_without_a_device(lib):
    """A call that passes validation reaches the HIP runtime; with no device
    its first runtime call fails, and the entry point reports LOKA_ERR_HIP
    with the failing call named (nothing is launched: the packed-weight
    forward's first HIP call asks for the current device)."""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a device is visible: this path needs a host without one")
    a = _fwd(x_mode=1, flags=1)  # row recipe, packed weight: no workspace needed
    assert lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(a)) == 0
    assert _call(lib, "loka_gemm_fp8_ln", a) == 5
    msg = lib.loka_last_error().decode()
    assert "loka_gemm_fp8_ln" in msg, msg
    assert lib.loka_status_string(5).decode() != ""


def test_validation_under_sanitizers(tmp_path):
    """api.cpp rebuilt with the address and undefined-behaviour sanitizers
    (host code only), linked with the library's other objects, and its
    validation paths driven through the C ABI by tests/abi_sanitized.cpp
    (also built with the sanitizers).  Any invalid access, overflow or
    undefined operation on these paths aborts the driver."""
    import shutil
    import subprocess
    from fp8_precision_gemm_amd import build as b
    objs = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "api.cpp"]
    clang = "/opt/rocm/llvm/bin/clang++"
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(clang):
        pytest.skip("needs the built objects and ROCm's clang")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    so = str(tmp_path / "liblokafp8_san.so")
    exe = str(tmp_path / "abi_sanitized")
    run = lambda cmd: subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    r = run([b.hipcc()] + b.FLAGS + san + ["-x", "hip", "-c", os.path.join(b.CSRC, "api.cpp"), "-o", api_o])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([b.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so, api_o] + objs + san)
    assert r.returncode == 0, r.stderr[-3000:]
    drv = os.path.join(os.path.dirname(__file__), "abi_sanitized.cpp")
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    r = run([clang, "-O1", "-g", "-std=c++17"] + host_san + [drv, "-o", exe, so, f"-Wl,-rpath,{tmp_path}",
                                                             "-L/opt/rocm/lib", "-lamdhip64"])
    assert r.returncode == 0, r.stderr[-3000:]
    import torch
    args = [exe] + (["nodevice"] if torch.cuda.device_count() == 0 else [])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run(args, capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "0 mismatch(es)" in r.stdout, r.stdout
