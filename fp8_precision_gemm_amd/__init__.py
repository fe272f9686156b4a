"""Python binding of liblokafp8.so (the FP8 GEMM + LayerNorm block for MI355X).

Argument marshalling only: every step of the block runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
functions carry the C ABI's names (see include/loka_fp8.h for the full
contract and the page passages each call follows).  If the library is not
built, importing works but every call raises: there is no fallback path.
"""

import ctypes
import os

import torch

__all__ = [
    "LokaError", "library", "library_path", "abi_version",
    "loka_quant_fp8", "loka_gemm_fp8_ln", "loka_gemm_fp8_bwd", "loka_grouped_gemm_fp8_ln",
    "loka_mere_z", "loka_dispatch_select", "loka_probe_input_update", "loka_probe_weight_update",
    "loka_probe_sample_input", "loka_probe_sample_weight",
    "QuantArgs", "FwdArgs", "BwdArgs", "GroupDesc", "GroupedArgs", "MereArgs", "DispatchCandidate",
    "E4M3", "E5M2", "MODES", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liblokafp8.so")

E4M3, E5M2 = 0, 1
FMTS = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
MODES = {"tensor": 0, "row": 1, "col": 2, "mx32_row": 3, "mx32_col": 4, "mx32_sq": 5}
STATUS = {0: "LOKA_OK", 1: "LOKA_ERR_INVALID_ARG", 2: "LOKA_ERR_UNSUPPORTED", 3: "LOKA_ERR_ALIGNMENT",
          4: "LOKA_ERR_WORKSPACE", 5: "LOKA_ERR_HIP"}
BWD_NO_LN = 1
BWD_MX32_SQ = 2
BWD_W_PACKED = 4
FWD_W_PACKED = 1
FWD_BLOCKNORM_HSWISH = 2
EPILOGUES = {"layernorm": 0, "blocknorm_hswish": FWD_BLOCKNORM_HSWISH}

c_i64, c_i32, c_f32, c_vp, c_sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class QuantArgs(ctypes.Structure):
    _fields_ = [("rows", c_i64), ("cols", c_i64), ("ld", c_i64), ("src_dtype", c_i32), ("fmt", c_i32),
                ("mode", c_i32), ("transpose_out", c_i32), ("src", c_vp), ("codes", c_vp), ("scales", c_vp),
                ("amax", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("M", c_i64), ("N", c_i64), ("K", c_i64), ("x_mode", c_i32), ("flags", c_i32), ("eps", c_f32),
                ("x", c_vp), ("qw", c_vp), ("sw", c_vp), ("bias", c_vp), ("gamma", c_vp), ("beta", c_vp),
                ("y", c_vp), ("z", c_vp), ("mean", c_vp), ("rstd", c_vp), ("qx_out", c_vp), ("sx_out", c_vp),
                ("workspace", c_vp), ("workspace_bytes", c_sz), ("x_scales", c_vp), ("y_codes", c_vp),
                ("y_scales", c_vp)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("M", c_i64), ("N", c_i64), ("K", c_i64), ("flags", c_i32), ("reserved", c_i32),
                ("dy", c_vp), ("qx", c_vp), ("sx", c_vp), ("mean", c_vp), ("rstd", c_vp), ("qw", c_vp),
                ("sw", c_vp), ("bias", c_vp), ("gamma", c_vp), ("x", c_vp), ("qw_row", c_vp), ("sw_row", c_vp),
                ("dx", c_vp), ("dw", c_vp), ("dgamma", c_vp), ("dbeta", c_vp), ("dbias", c_vp), ("dz", c_vp),
                ("dz_codes", c_vp), ("dz_scales", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz),
                ("xc_codes", c_vp), ("xc_scales", c_vp), ("dzc_codes", c_vp), ("dzc_scales", c_vp)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("M", c_i64), ("N", c_i64), ("K", c_i64), ("x", c_vp), ("qw", c_vp), ("sw", c_vp), ("bias", c_vp),
                ("gamma", c_vp), ("beta", c_vp), ("y", c_vp), ("z", c_vp)]


class GroupedArgs(ctypes.Structure):
    _fields_ = [("num_groups", c_i32), ("x_mode", c_i32), ("eps", c_f32), ("flags", c_i32),
                ("groups", ctypes.POINTER(GroupDesc)), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class MereArgs(ctypes.Structure):
    _fields_ = [("M", c_i64), ("N", c_i64), ("K", c_i64), ("S", c_i64), ("x", c_vp), ("w", c_vp), ("bias", c_vp),
                ("z", c_vp), ("rows", c_vp), ("out", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class DispatchCandidate(ctypes.Structure):
    _fields_ = [("us", ctypes.c_double), ("mere", ctypes.c_double)]


c_u64 = ctypes.c_uint64


class ProbeInputArgs(ctypes.Structure):
    _fields_ = [("B", c_i64), ("K", c_i64), ("n_old", c_i64), ("T", c_vp), ("mu", c_vp), ("S", c_vp),
                ("workspace", c_vp), ("workspace_bytes", c_sz)]


class ProbeWeightArgs(ctypes.Structure):
    _fields_ = [("R", c_i64), ("C", c_i64), ("m", c_f32), ("first", c_i32), ("W", c_vp), ("M", c_vp), ("U", c_vp),
                ("V", c_vp), ("info", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class ProbeSampleInputArgs(ctypes.Structure):
    _fields_ = [("B", c_i64), ("K", c_i64), ("n", c_i64), ("mu", c_vp), ("S", c_vp), ("seed", c_u64), ("out", c_vp),
                ("info", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class ProbeSampleWeightArgs(ctypes.Structure):
    _fields_ = [("R", c_i64), ("C", c_i64), ("M", c_vp), ("U", c_vp), ("V", c_vp), ("seed", c_u64), ("out", c_vp),
                ("info", c_vp), ("workspace", c_vp), ("workspace_bytes", c_sz)]


class LokaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


_lib = None


def library():
    """The loaded liblokafp8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m fp8_precision_gemm_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(library_path)
        for name, argt in [("loka_quant_fp8", QuantArgs), ("loka_gemm_fp8_ln", FwdArgs),
                           ("loka_gemm_fp8_ln_noalloc", FwdArgs),
                           ("loka_gemm_fp8_bwd", BwdArgs), ("loka_grouped_gemm_fp8_ln", GroupedArgs),
                           ("loka_mere_z", MereArgs), ("loka_probe_input_update", ProbeInputArgs),
                           ("loka_probe_weight_update", ProbeWeightArgs),
                           ("loka_probe_sample_input", ProbeSampleInputArgs),
                           ("loka_probe_sample_weight", ProbeSampleWeightArgs)]:
            f = getattr(lib, name)
            f.argtypes = [ctypes.POINTER(argt), c_vp]
            f.restype = c_i32
        for name, argt in [("loka_quant_workspace_size", QuantArgs), ("loka_gemm_fp8_ln_workspace_size", FwdArgs),
                           ("loka_gemm_fp8_bwd_workspace_size", BwdArgs), ("loka_grouped_workspace_size", GroupedArgs),
                           ("loka_mere_workspace_size", MereArgs),
                           ("loka_probe_input_workspace_size", ProbeInputArgs),
                           ("loka_probe_weight_workspace_size", ProbeWeightArgs),
                           ("loka_probe_sample_input_workspace_size", ProbeSampleInputArgs),
                           ("loka_probe_sample_weight_workspace_size", ProbeSampleWeightArgs)]:
            f = getattr(lib, name)
            f.argtypes = [ctypes.POINTER(argt)]
            f.restype = c_sz
        lib.loka_last_error.restype = ctypes.c_char_p
        lib.loka_status_string.restype = ctypes.c_char_p
        lib.loka_status_string.argtypes = [c_i32]
        lib.loka_abi_version.restype = c_i32
        lib.loka_dispatch_select.argtypes = [ctypes.POINTER(DispatchCandidate), c_i32, ctypes.c_double,
                                             ctypes.c_double, ctypes.c_double, ctypes.POINTER(c_i32)]
        lib.loka_dispatch_select.restype = c_i32
        _lib = lib
    return _lib


def abi_version():
    return library().loka_abi_version()


def _check(status):
    if status != 0:
        raise LokaError(status, library().loka_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes, device, given=None):
    if nbytes == 0:
        return None
    if given is not None:
        return given
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_shape(rows, cols):
    """Shape of the codes of a [rows, cols] source quantized with
    transpose_out="packed": cols rows of ceil(rows/128)*128 bytes (the
    fragment-interleaved layout; not row-major)."""
    return (cols, (rows + 127) // 128 * 128)


def loka_quant_fp8(src, fmt="e4m3", mode="row", transpose_out=False, codes=None, scales=None, amax=None,
                   want_amax=False, workspace=None, stream=None):
    """Quantize a 2-D bf16/fp32 CUDA tensor.  Returns (codes, scales, amax).

    transpose_out: False (codes [rows, cols]), True (codes of src^T, [cols,
    rows]), "packed" (codes of src^T in the fragment-interleaved layout
    that loka_gemm_fp8_ln(w_packed=True) reads; shape packed_shape(rows, cols))
    or "packed_rows" (codes of src itself in that layout, the dgrad weight
    of loka_gemm_fp8_bwd(w_packed=True); shape packed_shape(cols, rows))."""
    if src.dim() != 2 or src.stride(1) != 1:
        raise ValueError("src must be 2-D with unit column stride")
    rows, cols = src.shape
    m = MODES[mode]
    f = FMTS[fmt]
    dev = src.device
    trans = {"packed": 2, "packed_rows": 3}.get(transpose_out, 1 if transpose_out else 0)
    if codes is None:
        shape = {2: packed_shape(rows, cols), 3: packed_shape(cols, rows), 1: (cols, rows)}.get(trans, (rows, cols))
        codes = torch.empty(shape, dtype=torch.uint8, device=dev)
    if scales is None:
        if m == 0:
            scales = torch.empty(1, dtype=torch.float32, device=dev)
        elif m == 1:
            scales = torch.empty(rows, dtype=torch.float32, device=dev)
        elif m == 2:
            scales = torch.empty(cols, dtype=torch.float32, device=dev)
        elif m == 3:
            scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        elif m == 4:
            scales = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
        else:
            scales = torch.empty((rows // 32, cols // 32), dtype=torch.uint8, device=dev)
    if want_amax and amax is None and m <= 2:
        amax = torch.empty(scales.shape, dtype=torch.float32, device=dev)
    a = QuantArgs(rows=rows, cols=cols, ld=src.stride(0) if rows > 1 else cols,
                  src_dtype=0 if src.dtype == torch.bfloat16 else 1, fmt=f, mode=m,
                  transpose_out=trans, src=_ptr(src), codes=_ptr(codes), scales=_ptr(scales),
                  amax=_ptr(amax))
    if src.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("src must be bfloat16 or float32")
    lib = library()
    nb = lib.loka_quant_workspace_size(ctypes.byref(a))
    ws = _workspace(nb, dev, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = nb if ws is None else ws.numel()
    _check(lib.loka_quant_fp8(ctypes.byref(a), _stream(stream)))
    return codes, scales, amax


def _fwd_args(x, qw, sw, bias, gamma, beta, eps, x_mode, y, z, mean, rstd, qx_out, sx_out, w_packed=False,
              epilogue="layernorm", x_scales=None, y_codes=None, y_scales=None):
    M, K = x.shape
    N = qw.shape[0]
    flags = (FWD_W_PACKED if w_packed else 0) | EPILOGUES[epilogue]
    return FwdArgs(M=M, N=N, K=K, x_mode=MODES[x_mode], flags=flags, eps=eps, x=_ptr(x), qw=_ptr(qw), sw=_ptr(sw),
                   bias=_ptr(bias), gamma=_ptr(gamma), beta=_ptr(beta), y=_ptr(y), z=_ptr(z), mean=_ptr(mean),
                   rstd=_ptr(rstd), qx_out=_ptr(qx_out), sx_out=_ptr(sx_out), x_scales=_ptr(x_scales),
                   y_codes=_ptr(y_codes), y_scales=_ptr(y_scales))


def loka_gemm_fp8_ln(x, qw, sw, bias=None, gamma=None, beta=None, eps=1e-5, x_mode="row", y=None, want_z=False,
                     want_stats=False, want_qx=False, workspace=None, stream=None, prepare=False, w_packed=False,
                     epilogue="layernorm", x_scales=None, want_y_square=False, _noalloc=False):
    """Y = LayerNorm(dequant(q(X) . q(W)) + bias) for bf16 X [M, K] and the
    pre-quantized weight qw [N, K] (e4m3) with scales sw; with w_packed=True
    qw is in the packed layout (loka_quant_fp8(transpose_out="packed")).
    epilogue="blocknorm_hswish": Y = HardSwish(BlockNorm_256(Z)) instead
    (row recipe, no gamma/beta, no mean/rstd).
    x_mode="mx32_sq": x is X already quantized (uint8 e4m3 codes [M, K] from
    loka_quant_fp8(mode="mx32_sq")) and x_scales its E8M0 scales
    [M/32, K/32]; the weight is quantized with mode="mx32_sq" too.
    want_y_square: Y also as e4m3 codes [M, N] and E8M0 scales [M/32, N/32]
    in 32 x 32 blocks (out["y_codes"], out["y_scales"]): the next layer's
    x_mode="mx32_sq" input.

    Returns a dict with y and the requested optional outputs.  With
    prepare=True returns (launch, outputs) where launch() enqueues the call
    again with the same arguments (for timing loops)."""
    M, K = x.shape
    N = qw.shape[0]
    dev = x.device
    if x_mode == "mx32_sq":
        _need(x, torch.uint8, (M, K), "x")
        _need(x_scales, torch.uint8, (M // 32, K // 32), "x_scales")
    else:
        _need(x, torch.bfloat16, (M, K), "x")
    _need(qw, torch.uint8, packed_shape(K, N) if w_packed else (N, K), "qw")
    for v, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        if v is not None:
            _need(v, torch.bfloat16, (N,), nm)
    out = {"y": y if y is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)}
    if want_z:
        out["z"] = torch.empty((M, N), dtype=torch.float32, device=dev)
    if want_stats:
        out["mean"] = torch.empty(M, dtype=torch.float32, device=dev)
        out["rstd"] = torch.empty(M, dtype=torch.float32, device=dev)
    if want_qx:
        out["qx"] = torch.empty((M, K), dtype=torch.uint8, device=dev)
        if x_mode == "tensor":
            out["sx"] = torch.empty(1, dtype=torch.float32, device=dev)
        elif x_mode == "row":
            out["sx"] = torch.empty(M, dtype=torch.float32, device=dev)
        else:
            out["sx"] = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    if want_y_square:
        out["y_codes"] = torch.empty((M, N), dtype=torch.uint8, device=dev)
        out["y_scales"] = torch.empty((M // 32, N // 32), dtype=torch.uint8, device=dev)
    a = _fwd_args(x, qw, sw, bias, gamma, beta, eps, x_mode, out["y"], out.get("z"), out.get("mean"),
                  out.get("rstd"), out.get("qx"), out.get("sx"), w_packed, epilogue, x_scales, out.get("y_codes"),
                  out.get("y_scales"))
    lib = library()
    if _noalloc:
        ws = None
        a.workspace, a.workspace_bytes = None, 0
    else:
        nb = lib.loka_gemm_fp8_ln_workspace_size(ctypes.byref(a))
        ws = _workspace(nb, dev, workspace)
        a.workspace = _ptr(ws)
        a.workspace_bytes = nb if ws is None else ws.numel()
    keep = (x, qw, sw, bias, gamma, beta, ws, out, x_scales)
    st = _stream(stream)
    fn = lib.loka_gemm_fp8_ln_noalloc if _noalloc else lib.loka_gemm_fp8_ln
    ref = ctypes.byref(a)

    def launch():
        _check(fn(ref, st))
        return keep

    if prepare:
        return launch, out
    launch()
    return out


def loka_gemm_fp8_ln_noalloc(x, qw, sw, bias=None, gamma=None, beta=None, eps=1e-5, x_mode="row", y=None,
                             want_z=False, want_stats=False, want_qx=False, stream=None, prepare=False,
                             w_packed=False, epilogue="layernorm", x_scales=None, want_y_square=False):
    """loka_gemm_fp8_ln through the allocation-free entry point: the same
    arguments and outputs, no workspace (the library's fixed per-GPU device
    scratch serves instead; calls on one GPU must not overlap)."""
    return loka_gemm_fp8_ln(x, qw, sw, bias, gamma, beta, eps, x_mode, y, want_z, want_stats, want_qx, None,
                            stream, prepare, w_packed, epilogue, x_scales, want_y_square, _noalloc=True)


def loka_gemm_fp8_bwd(dy, x, qw_row, sw_row, ctx=None, bias=None, gamma=None, no_ln=False, want_dz=False,
                      want_dz_codes=False, want_dgamma=True, want_dbias=True, workspace=None, stream=None,
                      prepare=False, square=False, w_packed=False, want_col_codes=False):
    """Backward of loka_gemm_fp8_ln (row recipe).

    ctx: dict with qx [M,K] uint8, sx [M], mean [M], rstd [M], qw [N,K], sw [N]
    (the forward's qx/sx outputs, statistics and weight); unused with no_ln.
    w_packed=True (flag LOKA_BWD_W_PACKED): ctx["qw"] is the packed forward
    weight (packed_shape(K, N)) and qw_row the packed dgrad weight
    (loka_quant_fp8(w, mode="row", transpose_out="packed_rows"),
    packed_shape(N, K)).
    want_col_codes=True adds the wgrad operands: xc_codes (packed_shape(M, K))
    and xc_scales [K] of X per column (e4m3), dzc_codes (packed_shape(M, N))
    and dzc_scales [N] of dZ per column (e5m2).
    square=True: the backward of the square-block forward (x_mode="mx32_sq";
    flag LOKA_BWD_MX32_SQ): ctx holds X's codes qx [M,K] and scales sx
    [M/32,K/32], the weight's qw [N,K] and sw [K/32,N/32] (always required),
    and mean/rstd unless no_ln; x, qw_row and sw_row are unused (None).
    With square=True and w_packed=True, ctx["qw"] is
    loka_quant_fp8(w, mode="mx32_sq", transpose_out="packed") and qw_row is
    the same quantization with transpose_out="packed_rows".
    Returns a dict with dx, dw and the requested outputs."""
    M, N = dy.shape
    ctx = ctx or {}
    K = (ctx["qx"] if square else x).shape[1]
    dev = dy.device
    _need(dy, torch.bfloat16, (M, N), "dy")
    if square:
        _need(ctx["qx"], torch.uint8, (M, K), "qx")
        _need(ctx["sx"], torch.uint8, (M // 32, K // 32), "sx")
        _need(ctx["qw"], torch.uint8, packed_shape(K, N) if w_packed else (N, K), "qw")
        _need(ctx["sw"], torch.uint8, (K // 32, N // 32), "sw")
        if w_packed:
            _need(qw_row, torch.uint8, packed_shape(N, K), "qw_row")
    else:
        _need(x, torch.bfloat16, (M, K), "x")
        _need(qw_row, torch.uint8, packed_shape(N, K) if w_packed else (K, N), "qw_row")
        if w_packed and ctx.get("qw") is not None:
            _need(ctx["qw"], torch.uint8, packed_shape(K, N), "qw")
    out = {"dx": torch.empty((M, K), dtype=torch.bfloat16, device=dev),
           "dw": torch.empty((K, N), dtype=torch.float32, device=dev)}
    if want_dgamma and not no_ln:
        out["dgamma"] = torch.empty(N, dtype=torch.float32, device=dev)
        out["dbeta"] = torch.empty(N, dtype=torch.float32, device=dev)
    if want_dbias:
        out["dbias"] = torch.empty(N, dtype=torch.float32, device=dev)
    if want_dz:
        out["dz"] = torch.empty((M, N), dtype=torch.float32, device=dev)
    if want_dz_codes:
        out["dz_codes"] = torch.empty((M, N), dtype=torch.uint8, device=dev)
        out["dz_scales"] = (torch.empty((M // 32, N // 32), dtype=torch.uint8, device=dev) if square
                            else torch.empty(M, dtype=torch.float32, device=dev))
    if want_col_codes:
        out["xc_codes"] = torch.empty(packed_shape(M, K), dtype=torch.uint8, device=dev)
        out["xc_scales"] = torch.empty(K, dtype=torch.float32, device=dev)
        out["dzc_codes"] = torch.empty(packed_shape(M, N), dtype=torch.uint8, device=dev)
        out["dzc_scales"] = torch.empty(N, dtype=torch.float32, device=dev)
    flags = (BWD_NO_LN if no_ln else 0) | (BWD_MX32_SQ if square else 0) | (BWD_W_PACKED if w_packed else 0)
    a = BwdArgs(M=M, N=N, K=K, flags=flags, reserved=0, dy=_ptr(dy), qx=_ptr(ctx.get("qx")),
                sx=_ptr(ctx.get("sx")), mean=_ptr(ctx.get("mean")), rstd=_ptr(ctx.get("rstd")),
                qw=_ptr(ctx.get("qw")), sw=_ptr(ctx.get("sw")), bias=_ptr(bias), gamma=_ptr(gamma), x=_ptr(x),
                qw_row=_ptr(qw_row), sw_row=_ptr(sw_row), dx=_ptr(out["dx"]), dw=_ptr(out["dw"]),
                dgamma=_ptr(out.get("dgamma")), dbeta=_ptr(out.get("dbeta")), dbias=_ptr(out.get("dbias")),
                dz=_ptr(out.get("dz")), dz_codes=_ptr(out.get("dz_codes")), dz_scales=_ptr(out.get("dz_scales")),
                xc_codes=_ptr(out.get("xc_codes")), xc_scales=_ptr(out.get("xc_scales")),
                dzc_codes=_ptr(out.get("dzc_codes")), dzc_scales=_ptr(out.get("dzc_scales")))
    lib = library()
    nb = lib.loka_gemm_fp8_bwd_workspace_size(ctypes.byref(a))
    ws = _workspace(nb, dev, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = nb if ws is None else ws.numel()
    keep = (dy, x, qw_row, sw_row, ctx, bias, gamma, ws, out)
    st = _stream(stream)
    fn = lib.loka_gemm_fp8_bwd
    ref = ctypes.byref(a)

    def launch():
        _check(fn(ref, st))
        return keep

    if prepare:
        return launch, out
    launch()
    return out


def loka_grouped_gemm_fp8_ln(groups, eps=1e-5, want_z=False, workspace=None, stream=None, prepare=False,
                             w_packed=False):
    """groups: list of dicts with x [M,K] bf16, qw [N,K] uint8 (packed layout
    with w_packed=True), sw [N] fp32 and optional bias/gamma/beta bf16 [N].
    Returns one output dict per group."""
    outs, keep = [], []
    descs = (GroupDesc * max(1, len(groups)))()
    for i, g in enumerate(groups):
        x, qw = g["x"], g["qw"]
        M, K = x.shape
        N = qw.shape[0]
        _need(x, torch.bfloat16, (M, K), f"groups[{i}].x")
        _need(qw, torch.uint8, packed_shape(K, N) if w_packed else (N, K), f"groups[{i}].qw")
        o = {"y": torch.empty((M, N), dtype=torch.bfloat16, device=x.device)}
        if want_z:
            o["z"] = torch.empty((M, N), dtype=torch.float32, device=x.device)
        outs.append(o)
        keep.append((g, o))
        descs[i] = GroupDesc(M=M, N=N, K=K, x=_ptr(x), qw=_ptr(qw), sw=_ptr(g["sw"]), bias=_ptr(g.get("bias")),
                             gamma=_ptr(g.get("gamma")), beta=_ptr(g.get("beta")), y=_ptr(o["y"]), z=_ptr(o.get("z")))
    a = GroupedArgs(num_groups=len(groups), x_mode=MODES["row"], eps=eps, flags=FWD_W_PACKED if w_packed else 0,
                    groups=descs)
    lib = library()
    nb = lib.loka_grouped_workspace_size(ctypes.byref(a))
    dev = groups[0]["x"].device if groups else torch.device("cuda")
    ws = _workspace(nb, dev, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = nb if ws is None else ws.numel()
    keep.append((descs, ws))
    st = _stream(stream)
    fn = lib.loka_grouped_gemm_fp8_ln
    ref = ctypes.byref(a)

    def launch():
        _check(fn(ref, st))
        return keep

    if prepare:
        return launch, outs
    launch()
    return outs


def loka_mere_z(x, w, z, rows, bias=None, stream=None):
    """MERE of a candidate's Z (fp32 [M, N]) against the fp32 reference X W + b
    of the unquantized bf16 operands x [M, K] and w [K, N], over the rows in
    `rows` (int64 CUDA tensor).  Returns (mere, count of nonzero reference
    entries); synchronizes to read them."""
    M, K = x.shape
    N = w.shape[1]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w, torch.bfloat16, (K, N), "w")
    _need(z, torch.float32, (M, N), "z")
    if rows.dtype != torch.int64 or rows.dim() != 1 or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous 1-D int64 tensor")
    out = torch.zeros(3, dtype=torch.float64, device=x.device)
    a = MereArgs(M=M, N=N, K=K, S=rows.numel(), x=_ptr(x), w=_ptr(w), bias=_ptr(bias), z=_ptr(z), rows=_ptr(rows),
                 out=_ptr(out))
    lib = library()
    nb = lib.loka_mere_workspace_size(ctypes.byref(a))
    ws = _workspace(nb, x.device, None)
    a.workspace = _ptr(ws)
    a.workspace_bytes = nb if ws is None else ws.numel()
    _check(lib.loka_mere_z(ctypes.byref(a), _stream(stream)))
    o = out.cpu().tolist()
    if o[2] != 0:
        raise ValueError(f"{int(o[2])} sampled row indices outside [0, {M})")
    return o[0], int(o[1])


def loka_dispatch_select(candidates, baseline_us, mere_max=0.2, min_speedup=1.05):
    """Index of the recipe Dispatch chooses among (time_us, mere) pairs, or -1
    to keep the high-precision path (host only)."""
    n = len(candidates)
    arr = (DispatchCandidate * max(1, n))(*[DispatchCandidate(float(u), float(e)) for u, e in candidates])
    choice = c_i32(-2)
    _check(library().loka_dispatch_select(arr, n, float(baseline_us), float(mere_max), float(min_speedup),
                                          ctypes.byref(choice)))
    return choice.value


# ---- the Probe's statistics ---------------------------------------------------

def _run(fn_name, size_name, a, dev, stream):
    lib = library()
    nb = getattr(lib, size_name)(ctypes.byref(a))
    ws = _workspace(nb, dev, None)
    a.workspace = _ptr(ws)
    a.workspace_bytes = nb if ws is None else ws.numel()
    _check(getattr(lib, fn_name)(ctypes.byref(a), _stream(stream)))
    return ws


def _check_info(info, what):
    bad = info.cpu().tolist()
    if any(bad):
        raise LokaError(2, f"{what}: Cholesky pivot not positive (status {bad})")


def loka_probe_input_update(T, state=None, stream=None):
    """Merge the batch T (bf16 [B, K]) into state {"n", "mu" fp32 [K], "S" fp32
    [K, K]} (a new state when None); returns the state (updated in place)."""
    B, K = T.shape
    _need(T, torch.bfloat16, (B, K), "T")
    if state is None:
        state = {"n": 0, "mu": torch.zeros(K, dtype=torch.float32, device=T.device),
                 "S": torch.zeros((K, K), dtype=torch.float32, device=T.device)}
    a = ProbeInputArgs(B=B, K=K, n_old=state["n"], T=_ptr(T), mu=_ptr(state["mu"]), S=_ptr(state["S"]))
    ws = _run("loka_probe_input_update", "loka_probe_input_workspace_size", a, T.device, stream)
    state["n"] += B
    state["_keep"] = ws  # the workspace lives until the stream has used it
    return state


def loka_probe_weight_update(W, state=None, m=0.99, stream=None, check=True):
    """One flip-flop update of state {"M", "U", "V"} (fp32) with W (bf16 [R, C]);
    the first call (state None) initializes.  check: synchronize and raise if
    a Cholesky factorization failed."""
    R, C = W.shape
    _need(W, torch.bfloat16, (R, C), "W")
    first = state is None
    if first:
        dev = W.device
        state = {"M": torch.empty((R, C), dtype=torch.float32, device=dev),
                 "U": torch.empty((R, R), dtype=torch.float32, device=dev),
                 "V": torch.empty((C, C), dtype=torch.float32, device=dev),
                 "info": torch.zeros(2, dtype=torch.int32, device=dev)}
    a = ProbeWeightArgs(R=R, C=C, m=m, first=1 if first else 0, W=_ptr(W), M=_ptr(state["M"]), U=_ptr(state["U"]),
                        V=_ptr(state["V"]), info=_ptr(state["info"]))
    state["_keep"] = _run("loka_probe_weight_update", "loka_probe_weight_workspace_size", a, W.device, stream)
    if check and not first:
        _check_info(state["info"], "loka_probe_weight_update")
    return state


def loka_probe_sample_input(state, B, seed, stream=None, check=True):
    """B rows sampled from the tracked input distribution: bf16 [B, K]."""
    K = state["mu"].numel()
    dev = state["mu"].device
    out = torch.empty((B, K), dtype=torch.bfloat16, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    a = ProbeSampleInputArgs(B=B, K=K, n=state["n"], mu=_ptr(state["mu"]), S=_ptr(state["S"]), seed=seed,
                             out=_ptr(out), info=_ptr(info))
    ws = _run("loka_probe_sample_input", "loka_probe_sample_input_workspace_size", a, dev, stream)
    if check:
        _check_info(info, "loka_probe_sample_input")
    del ws
    return out


def loka_probe_sample_weight(state, seed, stream=None, check=True):
    """A weight sampled from the tracked matrix-normal: bf16 [R, C]."""
    R, C = state["M"].shape
    dev = state["M"].device
    out = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    info = torch.zeros(2, dtype=torch.int32, device=dev)
    a = ProbeSampleWeightArgs(R=R, C=C, M=_ptr(state["M"]), U=_ptr(state["U"]), V=_ptr(state["V"]), seed=seed,
                              out=_ptr(out), info=_ptr(info))
    ws = _run("loka_probe_sample_weight", "loka_probe_sample_weight_workspace_size", a, dev, stream)
    if check:
        _check_info(info, "loka_probe_sample_weight")
    del ws
    return out
