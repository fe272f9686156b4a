"""Benchmark of the FP8 GEMM + LayerNorm block on one MI355X.

One step = one loka_gemm_fp8_ln call on the rowwise workload (X[16384,512]
bf16 Student-t(3) with outlier columns, W[512,512] pre-quantized per column,
bias, LayerNorm over 512): the X amax and e4m3 cast, the FP8 MFMA GEMM and
the dequant + bias + LayerNorm epilogue, all in one kernel.  The weight is
quantized once per step of training, outside the activation path (reported
separately as `weight_quant_us`), straight into the packed layout the kernel
reads; the same call with a row-major weight (rearranged inside the call) is
reported under `rows`.  Inputs are resident in HBM; 16 rotating
input/output sets (537 MB) keep the 256 MB Infinity Cache from serving them.
Launches are replayed from a HIP graph so host launch cost does not enter.

Timing: `--warmup` launches untimed, then 5 batches of max(--steps, 100)
launches (rounded up to whole graph replays), each bracketed by HIP events
on the launch stream; the per-launch time is the median batch's, and
`timing` gives the batch count, the launches per batch and in total, and the
fastest and slowest batch.

Prints one JSON line.  `roofline` is for the fused forward kernel (HBM
bound: 254 FLOP/B against a ridge of 625); `cpu_baseline` is the NumPy
oracle on this host's cores (and on one thread); `oracle_mere` (and each
row's) is the oracle's per-layer quantization error against the bf16
reference.  Other workloads of the block (tensor recipe, MX, backward,
grouped, ...) are timed the same way and reported under `rows`.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 quant+GEMM+LayerNorm TFLOP/s and % FP8 MFMA peak (M=16384,K=N=512)"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ROTATE = 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-oracle-report", action="store_true", help="skip the oracle's MERE report")
    p.add_argument("--no-rows", action="store_true", help="skip the other workloads")
    p.add_argument("--only", default=None,
                   help="comma list of workloads to time (for profiling): "
                        "fwd,tensor,mx,blocknorm (or blocknorm_fwd_16384x512x512 / blocknorm_fwd_4096x512x4096 "
                        "alone),bwd,square,dispatch,probe,grouped,copy")
    return p.parse_args()


def fwd_bytes(M, K, N, mx=False):
    """Algorithmic HBM bytes of one fused forward: read X (bf16) once, the
    weight codes and scales, bias/gamma/beta; write Y (bf16) once."""
    sw = N * (K // 32) if mx else N * 4
    return 2 * M * K + N * K + sw + 3 * 2 * N + 2 * M * N


ROWS_COUNTERS = os.path.join(ROOT, "profiles", "rows_hbm_mfma_counters.md")
CLOCK_GHZ = 2.4     # MI355X peak shader clock, for the MFMA-busy fraction


def _sources_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fp8_precision_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def row_counters():
    """Per-row hardware counters from the committed summary: for each
    workload, the HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-
    calibrated) and the MFMA-busy cycles per launch (SQ_VALU_MFMA_BUSY_CYCLES)
    of all the kernels one launch of the row runs.  A row is returned only
    while its listed sources hash to the value recorded with its counters."""
    try:
        text = open(ROWS_COUNTERS).read()
    except OSError:
        return {}
    out = {}
    for line in text.splitlines():
        if not line.startswith("row: "):
            continue
        f = dict(kv.split("=", 1) for kv in line[5:].split() if "=" in kv)
        try:
            if _sources_hash(f["sources"].split(",")) != f["sha256_16"]:
                continue
            out[f["name"]] = {"traffic_bytes": int(f["traffic_bytes"]), "mfma_busy_cycles": int(f["mfma_busy_cycles"])}
        except (KeyError, ValueError, OSError):
            continue
    return out


def attach_counters(rows, counters, bytes_of):
    """Adds the committed counters to each timed row: traffic (bytes per
    launch, and as a fraction of the row's algorithmic bytes when it has
    them) and the MFMA-busy fraction over the row's measured launch time
    (1024 SIMDs at CLOCK_GHZ)."""
    for name, c in counters.items():
        r = rows.get(name)
        if r is None or "us" not in r:
            continue
        d = {"traffic_bytes": c["traffic_bytes"],
             "mfma_busy_frac": round(c["mfma_busy_cycles"] / (1024 * r["us"] * 1e-6 * CLOCK_GHZ * 1e9), 4)}
        if bytes_of.get(name):
            d["traffic_over_algorithmic"] = round(c["traffic_bytes"] / bytes_of[name], 3)
        r["counters"] = d


BATCHES = 5          # timed batches; the reported time is their median
MIN_BATCH = 100      # launches per batch, at least
GRAPH_LAUNCHES = 64  # launches per captured graph, at least (a replay boundary costs ~8 us)


class ClockSampler:
    """Samples the current shader clock level from the driver's sysfs table
    (`pp_dpm_sclk`, current level marked '*') on a background thread while
    the timed batches run; `summary()` gives the MHz readings' distribution."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for f in self.files:
            try:
                for line in open(f):
                    line = line.strip()
                    if line.endswith("*"):
                        mhz = line.split(":", 1)[1].strip(" *").lower().replace("mhz", "")
                        return float(mhz)
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.asarray(self.samples)
        return {"samples": int(a.size), "mhz_median": float(np.median(a)), "mhz_min": float(a.min()),
                "mhz_max": float(a.max())}


def timed_graph(torch, launches, steps, warmup, stream, clock=None):
    """Capture `launches` (callables enqueuing on `stream`), repeated to at
    least GRAPH_LAUNCHES launches, into one graph and time its replays:
    `warmup` launches untimed, then BATCHES batches of at least
    max(steps, MIN_BATCH) launches each (whole replays), each batch
    bracketed by HIP events on `stream` (with `clock`, a ClockSampler, running
    over the batches).  Returns (median seconds per launch, info) with info =
    {"batches", "launches_per_batch", "timed_launches", "launches_per_graph",
    "us_min", "us_max"} (per-launch times of the fastest and slowest batch)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for f in launches:  # eager warm-up (kernel attribute set-up happens here)
            f()
    stream.synchronize()
    rounds = max(1, -(-GRAPH_LAUNCHES // len(launches)))
    with torch.cuda.graph(g, stream=stream):
        for _ in range(rounds):
            for f in launches:
                f()
    n = len(launches) * rounds
    reps_w = max(1, -(-warmup // n))
    reps = max(1, -(-max(steps, MIN_BATCH) // n))
    for _ in range(reps_w):
        g.replay()
    torch.cuda.synchronize()
    per = []
    import contextlib
    with clock if clock is not None else contextlib.nullcontext():
        for _ in range(BATCHES):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            e1.synchronize()
            per.append(e0.elapsed_time(e1) / 1e3 / (reps * n))
    torch.cuda.synchronize()
    info = {"batches": BATCHES, "launches_per_batch": reps * n, "timed_launches": BATCHES * reps * n,
            "launches_per_graph": n, "us_min": round(min(per) * 1e6, 3), "us_max": round(max(per) * 1e6, 3)}
    return float(np.median(per)), info


def dev_bf16(torch, bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def bench_forward(torch, lk, case, x_mode, steps, warmup, stream, packed=True, epilogue="layernorm", clock=None):
    """Time loka_gemm_fp8_ln over ROTATE buffer sets; returns a dict.  The
    weight is quantized straight into the packed layout the kernel reads
    (packed=False: row-major [N, K] codes, rearranged inside every call)."""
    M, K, N = case["M"], case["K"], case["N"]
    w = dev_bf16(torch, case["w"])
    wmode = {"row": "col", "tensor": "tensor", "mx32_row": "mx32_col"}[x_mode]
    layout = "packed" if packed else True
    qw, sw, _ = lk.loka_quant_fp8(w, mode=wmode, transpose_out=layout, stream=stream)
    x0 = dev_bf16(torch, case["x"])
    vec = [dev_bf16(torch, case[k]) for k in ("bias", "gamma", "beta")]
    if epilogue != "layernorm":
        vec = vec[:1] + [None, None]  # BlockNorm has no affine parameters
    launches = []
    for i in range(ROTATE):
        x = x0 if i == 0 else x0.clone()
        f, _ = lk.loka_gemm_fp8_ln(x, qw, sw, *vec, x_mode=x_mode, stream=stream, prepare=True, w_packed=packed,
                                   epilogue=epilogue)
        launches.append(f)
    torch.cuda.synchronize()
    per, tinfo = timed_graph(torch, launches, steps, warmup, stream, clock=clock)
    if not packed:
        return {"us": per * 1e6, "timing": tinfo}
    flops = 2.0 * M * N * K
    nbytes = fwd_bytes(M, K, N, mx=x_mode == "mx32_row")
    # the weight quantization (once per training step), same rotation
    import ctypes
    a = lk.QuantArgs(rows=K, cols=N, ld=N, mode=lk.MODES[wmode])
    nb = lk.library().loka_quant_workspace_size(ctypes.byref(a))
    wsq = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    wq = []
    for i in range(ROTATE):
        wi = w if i == 0 else w.clone()
        qwi, swi = torch.empty_like(qw), torch.empty_like(sw)
        wq.append(lambda wi=wi, qwi=qwi, swi=swi: lk.loka_quant_fp8(
            wi, mode=wmode, transpose_out=layout, codes=qwi, scales=swi, stream=stream, workspace=wsq))
    wper, _ = timed_graph(torch, wq, min(steps, 800), min(warmup, 80), stream)
    return {"us": per * 1e6, "tflops": flops / per / 1e12, "gbs": nbytes / per / 1e9, "bytes": nbytes,
            "flops": flops, "weight_quant_us": wper * 1e6, "timing": tinfo}


def bench_backward(torch, lk, case, steps, warmup, stream):
    M, K, N = case["M"], case["K"], case["N"]
    x, w, dy = dev_bf16(torch, case["x"]), dev_bf16(torch, case["w"]), dev_bf16(torch, case["dy"])
    bias, gamma, beta = (dev_bf16(torch, case[k]) for k in ("bias", "gamma", "beta"))
    # both weights quantized once per step straight into the layouts the
    # kernels read (the forward's packed weight serves the Z recompute)
    qw, sw, _ = lk.loka_quant_fp8(w, mode="col", transpose_out="packed", stream=stream)
    qwr, swr, _ = lk.loka_quant_fp8(w, mode="row", transpose_out="packed_rows", stream=stream)
    f = lk.loka_gemm_fp8_ln(x, qw, sw, bias, gamma, beta, want_stats=True, want_qx=True, stream=stream,
                            w_packed=True)
    ctx = {"qx": f["qx"], "sx": f["sx"], "mean": f["mean"], "rstd": f["rstd"], "qw": qw, "sw": sw}
    launches = []
    for i in range(4):
        dyi = dy if i == 0 else dy.clone()
        fn, _ = lk.loka_gemm_fp8_bwd(dyi, x, qwr, swr, ctx=ctx, bias=bias, gamma=gamma, stream=stream, prepare=True,
                                     w_packed=True)
        launches.append(fn)
    torch.cuda.synchronize()
    per, tinfo = timed_graph(torch, launches, steps, warmup, stream)
    flops = 2.0 * M * N * K * 3  # recomputed Z, dgrad, wgrad
    nbytes = 2 * M * N + M * K + 2 * M * K + 2 * M * K + 4 * K * N  # dY, qX, X, dX, dW (minimum)
    return {"us": per * 1e6, "tflops": flops / per / 1e12, "gbs_min_bytes": nbytes / per / 1e9,
            "min_bytes": nbytes, "timing": tinfo}


def bench_square(torch, lk, case, steps, warmup, stream):
    """The square-block recipe (one E8M0 per 32 x 32 block): the forward on
    X's codes (quantized once, as its producer would emit them; that
    quantization is timed on its own as x_quant_us) and the backward on the
    forward's codes.  Returns (forward row, backward row)."""
    M, K, N = case["M"], case["K"], case["N"]
    x, w, dy = dev_bf16(torch, case["x"]), dev_bf16(torch, case["w"]), dev_bf16(torch, case["dy"])
    bias, gamma, beta = (dev_bf16(torch, case[k]) for k in ("bias", "gamma", "beta"))
    qw, sw, _ = lk.loka_quant_fp8(w, mode="mx32_sq", transpose_out=True, stream=stream)
    qwp, _, _ = lk.loka_quant_fp8(w, mode="mx32_sq", transpose_out="packed", stream=stream)
    qx, sx, _ = lk.loka_quant_fp8(x, mode="mx32_sq", stream=stream)
    launches, quants = [], []
    for i in range(ROTATE):
        qxi = qx if i == 0 else qx.clone()
        f, _ = lk.loka_gemm_fp8_ln(qxi, qwp, sw, bias, gamma, beta, x_mode="mx32_sq", x_scales=sx, stream=stream,
                                   prepare=True, w_packed=True)
        launches.append(f)
        xi = x if i == 0 else x.clone()
        ci, si = torch.empty_like(qx), torch.empty_like(sx)
        quants.append(lambda xi=xi, ci=ci, si=si: lk.loka_quant_fp8(xi, mode="mx32_sq", codes=ci, scales=si,
                                                                     stream=stream))
    torch.cuda.synchronize()
    per, tinfo = timed_graph(torch, launches, steps, warmup, stream)
    qper, _ = timed_graph(torch, quants, min(steps, 800), min(warmup, 80), stream)
    nbytes = M * K + (M // 32) * (K // 32) + N * K + (K // 32) * (N // 32) + 3 * 2 * N + 2 * M * N
    fwd = {"us": per * 1e6, "tflops": 2.0 * M * N * K / per / 1e12, "gbs": nbytes / per / 1e9, "bytes": nbytes,
           "x_quant_us": qper * 1e6, "timing": tinfo}
    f = lk.loka_gemm_fp8_ln(qx, qw, sw, bias, gamma, beta, x_mode="mx32_sq", x_scales=sx, want_stats=True,
                            stream=stream)
    # both weights quantized straight into the packed layouts, as the rowwise
    # backward's row takes them (the forward's qwp, and W^T's for the dgrad)
    qwr, _, _ = lk.loka_quant_fp8(w, mode="mx32_sq", transpose_out="packed_rows", stream=stream)
    ctx = {"qx": qx, "sx": sx, "qw": qwp, "sw": sw, "mean": f["mean"], "rstd": f["rstd"]}
    launches = []
    for i in range(4):
        dyi = dy if i == 0 else dy.clone()
        fn, _ = lk.loka_gemm_fp8_bwd(dyi, None, qwr, None, ctx=ctx, bias=bias, gamma=gamma, stream=stream,
                                     prepare=True, square=True, w_packed=True)
        launches.append(fn)
    torch.cuda.synchronize()
    per, tinfo = timed_graph(torch, launches, steps, warmup, stream)
    nbytes = 2 * M * N + M * K + 2 * M * K + 4 * K * N  # dY, qX, dX, dW (minimum)
    bwd = {"us": per * 1e6, "tflops": 2.0 * M * N * K * 3 / per / 1e12, "gbs_min_bytes": nbytes / per / 1e9,
           "min_bytes": nbytes, "timing": tinfo}
    return fwd, bwd


def bench_probe(torch, lk, case, stream, reps=20):
    """The Probe's four operations on the benchmark layer: the input update
    with the 16384 x 512 activations, the weight update and the two samplers
    (512 x 512 weight; 16384 sampled rows).  Per-call time in us."""
    x, w = dev_bf16(torch, case["x"]), dev_bf16(torch, case["w"])
    out = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    with torch.cuda.stream(stream):
        st = lk.loka_probe_input_update(x, stream=stream)
        out["input_update_us"] = timed(lambda: lk.loka_probe_input_update(x, st, stream=stream))
        ws = lk.loka_probe_weight_update(w, stream=stream)
        lk.loka_probe_weight_update(w.clone(), ws, m=0.9, stream=stream)
        out["weight_update_us"] = timed(lambda: lk.loka_probe_weight_update(w, ws, m=0.9, stream=stream, check=False))
        out["sample_input_us"] = timed(lambda: lk.loka_probe_sample_input(st, 16384, 1, stream=stream, check=False))
        out["sample_weight_us"] = timed(lambda: lk.loka_probe_sample_weight(ws, 1, stream=stream, check=False))
    return out


def bench_grouped(torch, lk, groups, steps, warmup, stream):
    dg = []
    flops = 0.0
    nbytes = 0
    for g in groups:
        qw, sw, _ = lk.loka_quant_fp8(dev_bf16(torch, g["w"]), mode="col", transpose_out="packed", stream=stream)
        dg.append({"x": dev_bf16(torch, g["x"]), "qw": qw, "sw": sw, "bias": dev_bf16(torch, g["bias"]),
                   "gamma": dev_bf16(torch, g["gamma"]), "beta": dev_bf16(torch, g["beta"])})
        flops += 2.0 * g["M"] * g["N"] * g["K"]
        nbytes += fwd_bytes(g["M"], g["K"], g["N"])
    fn, _ = lk.loka_grouped_gemm_fp8_ln(dg, stream=stream, prepare=True, w_packed=True)
    torch.cuda.synchronize()
    per, tinfo = timed_graph(torch, [fn], steps, warmup, stream)
    return {"us": per * 1e6, "tflops": flops / per / 1e12, "gbs": nbytes / per / 1e9, "bytes": nbytes,
            "flops": flops, "timing": tinfo}


def bench_copy(torch, steps, warmup, stream):
    """A plain device copy of a 16 MiB buffer (torch's copy kernel): the
    calibration reference for the HBM byte counters (it must read and write
    exactly 16 MiB per launch)."""
    nbytes = 16 << 20
    src = [torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_() for _ in range(ROTATE)]
    dst = [torch.empty_like(t) for t in src]
    launches = [lambda a=a, b=b: b.copy_(a) for a, b in zip(src, dst)]
    per, tinfo = timed_graph(torch, launches, steps, warmup, stream)
    return {"us": per * 1e6, "gbs": 2 * nbytes / per / 1e9, "bytes_read": nbytes, "bytes_written": nbytes,
            "timing": tinfo}


CPU_SHARE = 16      # host threads a one-GPU job may use
CHUNK_ROWS = 256    # rows per task of the MERE report's row blocks


def host_cpu():
    """(threads to use, CPU model) of this host."""
    n = min(len(os.sched_getaffinity(0)), CPU_SHARE)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline(case, threads, model, budget_s=8.0):
    """The NumPy oracle as it stands (untuned) on the host: full rowwise
    forwards (quantize X and W, fp64 GEMM, LayerNorm, bf16 rounding) of the
    headline workload, its rows split into one block per thread (rows are
    independent in the rowwise recipe; each block quantizes W again), the
    blocks spread over `threads` host threads (NumPy's own BLAS pinned to one
    thread each), repeated for about budget_s seconds; then the same blocks
    on one thread over a sample of the rows.  TFLOP/s counts 2 M N K per
    forward, as the GPU's value does."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import forward
    M, K, N = case["M"], case["K"], case["N"]
    rows = max(256, (M // threads + 31) // 32 * 32)
    spans = [(lo, min(lo + rows, M)) for lo in range(0, M, rows)]

    def one(span):
        lo, hi = span
        forward.gemm_ln_forward(case["x"][lo:hi], case["w"], case["bias"], case["gamma"], case["beta"], recipe="row")

    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t0 < budget_s:
            list(ex.map(one, spans))
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        t0 = time.perf_counter()
        done = 0
        while done < len(spans) and (done < 2 or time.perf_counter() - t0 < budget_s / 2):
            one(spans[done])
            done += 1
        dt1 = (time.perf_counter() - t0) / (sum(hi - lo for lo, hi in spans[:done]) / M)
    return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": f"{reps} full rowwise forward(s) of M={M},K={K},N={N}, {len(spans)} blocks of {rows} "
                      f"rows over {threads} host threads, {dt:.3f} s each",
            "one_thread": {"value": 2.0 * M * N * K / dt1 / 1e12, "unit": "TFLOP/s",
                           "sample": f"{done} of the {len(spans)} blocks of the same forward on one thread, "
                                     f"scaled to the full forward: {dt1:.2f} s"}}


def oracle_report(cases, threads):
    """The oracle's per-layer quantization error (MERE of each workload's
    outputs against the unquantized bf16 reference) for every workload,
    whole: Z and Y per forward (the MX workload's rows in blocks over the
    host threads, which gives the same numbers), dZ, dX and dW for the
    training step, and every group of the grouped workload."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import report
    out = {}
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        for name, (c, recipe) in cases["forward"].items():
            r = report.forward_error(c["x"], c["w"], c["bias"], c["gamma"], c["beta"], recipe, pmap=ex.map,
                                     chunk_rows=CHUNK_ROWS)
            out[name] = {k: {"mere": round(v["mere"], 6), "count": v["count"]} for k, v in r.items()}
        if "backward" in cases:
            name, c = cases["backward"]
            r = report.backward_error(c["x"], c["w"], c["dy"], c["bias"], c["gamma"], c["beta"])
            out[name] = {k: {"mere": round(v["mere"], 6), "count": v["count"]} for k, v in r.items()}
        if "grouped" in cases:
            name, gs = cases["grouped"]
            per = report.grouped_error(gs, pmap=ex.map)
            out[name] = {"per_group": [{k: round(v["mere"], 6) for k, v in p.items()} for p in per],
                         "summary": report.summarize(per)}
    out["seconds"] = round(time.perf_counter() - t0, 1)
    return out


def gpu_clock():
    """The device name and shader clock: the current and highest SCLK levels
    from the driver's sysfs table (the current level is marked '*'), read
    right after the timed region."""
    import glob
    out = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            levels = [l.strip() for l in open(f) if l.strip()]
        except OSError:
            continue
        cur = [l for l in levels if l.endswith("*")]
        out[f.split("/")[4]] = {"current": cur[0].rstrip(" *") if cur else None, "levels": levels}
    return out


def _rounded(r):
    return {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_precision_gemm_amd as lk
    from synth import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    stream = torch.cuda.Stream()
    case = workloads.outlier_case(dy=True)
    rows = {}
    only = None if args.only is None else set(args.only.split(","))
    want = lambda name: only is None or name in only
    main_res = None
    if want("fwd"):
        sampler = ClockSampler()
        main_res = bench_forward(torch, lk, case, "row", args.steps, args.warmup, stream, clock=sampler)
        clock = {"sysfs_levels": gpu_clock(), "during_headline": sampler.summary()}
        print(f"[bench] rowwise forward: {main_res['us']:.2f} us/launch (median of {main_res['timing']['batches']} "
              f"batches of {main_res['timing']['launches_per_batch']})", file=sys.stderr, flush=True)
        if not args.no_rows:
            r = bench_forward(torch, lk, case, "row", max(200, args.steps // 4), max(20, args.warmup // 4), stream,
                              packed=False)
            rows["fwd_16384x512x512_rowmajor_weight"] = {"us": round(r["us"], 3), "timing": r["timing"]}
            print(f"[bench] rowwise forward, row-major weight: {r['us']:.2f} us", file=sys.stderr, flush=True)
    tcase = mxcase = gcase = None
    if not args.no_rows and want("tensor"):
        tcase = workloads.tensor_case()
        r = bench_forward(torch, lk, tcase, "tensor", args.steps, args.warmup, stream)
        rows["tensor_fwd_512x256x256"] = _rounded(r)
        print(f"[bench] tensor forward: {r['us']:.2f} us", file=sys.stderr, flush=True)
    if not args.no_rows and want("mx"):
        mxcase = workloads.mx_case()
        r = bench_forward(torch, lk, mxcase, "mx32_row", args.steps, args.warmup, stream)
        rows["mx_fwd_65536x1024x256"] = _rounded(r)
        rows["mx_fwd_65536x1024x256"]["hbm_frac"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        print(f"[bench] mx forward: {r['us']:.2f} us", file=sys.stderr, flush=True)
    if not args.no_rows and (want("blocknorm") or want("blocknorm_fwd_16384x512x512")
                             or want("blocknorm_fwd_4096x512x4096")):
        for nm, c in (("blocknorm_fwd_16384x512x512", case),
                      ("blocknorm_fwd_4096x512x4096", workloads.forward_case(4096, 512, 4096, seed=7,
                                                                             x_dist="student_t3_outliers"))):
            if not (want("blocknorm") or want(nm)):
                continue
            r = bench_forward(torch, lk, c, "row", args.steps, args.warmup, stream, epilogue="blocknorm_hswish")
            rows[nm] = _rounded(r)
            rows[nm]["hbm_frac"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
            print(f"[bench] {nm}: {r['us']:.2f} us", file=sys.stderr, flush=True)
    if not args.no_rows and want("bwd"):
        r = bench_backward(torch, lk, case, args.steps, args.warmup, stream)
        rows["bwd_16384x512x512"] = _rounded(r)
        print(f"[bench] backward: {r['us']:.2f} us", file=sys.stderr, flush=True)
    if not args.no_rows and want("square"):
        f, b = bench_square(torch, lk, case, args.steps, args.warmup, stream)
        rows["square_fwd_16384x512x512"] = _rounded(f)
        rows["square_fwd_16384x512x512"]["hbm_frac"] = round(f["gbs"] / PEAK_HBM_GBS, 4)
        rows["square_bwd_16384x512x512"] = _rounded(b)
        print(f"[bench] square forward: {f['us']:.2f} us (X quantization {f['x_quant_us']:.2f} us); "
              f"square backward: {b['us']:.2f} us", file=sys.stderr, flush=True)
    if not args.no_rows and want("dispatch"):
        from fp8_precision_gemm_amd.dispatch import dispatch
        x, w = dev_bf16(torch, case["x"]), dev_bf16(torch, case["w"])
        vec = [dev_bf16(torch, case[k]) for k in ("bias", "gamma", "beta")]
        with torch.cuda.stream(stream):
            d = dispatch(x, w, *vec, reps=max(20, args.steps // 20), warmup=5, stream=stream)
        rows["dispatch_16384x512x512"] = {
            "choice": d["choice"], "baseline_us": round(d["baseline_us"], 3),
            "baseline": "bf16 library linear + LayerNorm",
            "table": {r["recipe"]: {"us": round(r["us"], 3), "mere": round(r["mere"], 5)} for r in d["table"]}}
        print(f"[bench] dispatch: {d['choice']} (baseline {d['baseline_us']:.1f} us; "
              + ", ".join(f"{r['recipe']} {r['us']:.1f} us MERE {r['mere']:.3f}" for r in d["table"]) + ")",
              file=sys.stderr, flush=True)
    if not args.no_rows and want("probe"):
        r = bench_probe(torch, lk, case, stream)
        rows["probe_16384x512x512"] = {k: round(v, 2) for k, v in r.items()}
        print("[bench] probe: " + ", ".join(f"{k} {v:.1f}" for k, v in r.items()), file=sys.stderr, flush=True)
    if not args.no_rows and want("grouped"):
        gcase = workloads.grouped_case()
        r = bench_grouped(torch, lk, gcase, args.steps, args.warmup, stream)
        rows["grouped_64x8192"] = _rounded(r)
        rows["grouped_64x8192"]["hbm_frac"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        print(f"[bench] grouped: {r['us']:.2f} us", file=sys.stderr, flush=True)
    if only is not None and "copy" in only:
        r = bench_copy(torch, args.steps, args.warmup, stream)
        rows["copy_16MiB"] = _rounded(r)
        print(f"[bench] copy 16 MiB: {r['us']:.2f} us", file=sys.stderr, flush=True)
    counters = row_counters()
    attach_counters(rows, counters, {k: v.get("bytes") or v.get("min_bytes") for k, v in rows.items()})
    if main_res is None:
        print(json.dumps({"rows": rows}))
        return

    threads, model = host_cpu()
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, threads, model)
    report = None
    if not args.no_oracle_report:
        fwd_cases = {"fwd_16384x512x512": (case, "row")}
        if tcase is not None:
            fwd_cases["tensor_fwd_512x256x256"] = (tcase, "tensor")
        if mxcase is not None:
            fwd_cases["mx_fwd_65536x1024x256"] = (mxcase, "mx32")
        rcases = {"forward": fwd_cases}
        if "bwd_16384x512x512" in rows:
            rcases["backward"] = ("bwd_16384x512x512", case)
        if gcase is not None:
            rcases["grouped"] = ("grouped_64x8192", gcase)
        report = oracle_report(rcases, threads)
        for name, r in report.items():
            if name in rows:
                rows[name]["oracle_mere"] = r
        print(f"[bench] oracle MERE report: {report['seconds']} s on {threads} threads", file=sys.stderr, flush=True)
    ms = main_res["us"] / 1e3
    out = {
        "metric": METRIC,
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "rowwise FP8 GEMM + LayerNorm forward, X[16384,512] Student-t(3) with 5 outlier "
                               "columns x50, W[512,512] per-column e4m3, LayerNorm over 512",
                   "M": 16384, "K": 512, "N": 512, "x_scaling": "row", "w_scaling": "col", "fmt": "e4m3",
                   "w_layout": "packed (fragment-interleaved e4m3 codes from loka_quant_fp8)"},
        "pct_fp8_peak": round(100 * main_res["tflops"] / PEAK_FP8_TFLOPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(main_res["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(main_res["gbs"] / PEAK_HBM_GBS, 4), "traffic": counters.get("fwd_16384x512x512", {}).get("traffic_bytes"),
                     "traffic_unit": "bytes/launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                     "profiles/rows_hbm_mfma_counters.md, null once the kernel's sources change)",
                     "kernel": "k_fwd_xl<row> (weight-resident staged X quant + FP8 MFMA GEMM + LayerNorm)",
                     "algorithmic_bytes_per_launch": main_res["bytes"],
                     "mfma_busy_frac": (round(counters["fwd_16384x512x512"]["mfma_busy_cycles"]
                                              / (1024 * main_res["us"] * 1e-6 * CLOCK_GHZ * 1e9), 4)
                                        if "fwd_16384x512x512" in counters else None),
                     "avg_launch_us": round(main_res["us"], 3)},
        "timing": main_res["timing"],
        "gpu": {"name": torch.cuda.get_device_properties(0).name,
                "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                "sclk": clock},
        "oracle_mere": None if report is None else report["fwd_16384x512x512"],
        "weight_quant_us": round(main_res["weight_quant_us"], 3),
        "value_incl_weight_quant": round(main_res["flops"] / ((main_res["us"] + main_res["weight_quant_us"]) * 1e-6)
                                         / 1e12, 2),
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
