"""Build liblokafp8.so (the gfx950 HIP kernels and their C ABI) in-tree.

Every translation unit is compiled by hipcc for gfx950 only, with IEEE fp32
division and square root, fp32 denormals kept, and packed-fp32 instruction
selection disabled; the objects are linked into one shared library next to
this file.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblokafp8.so")
SOURCES = ["api.cpp", "quant.hip", "gemm_ln_fwd.hip", "fwd_tensor.hip", "fwd_row.hip", "fwd_blocknorm.hip", "fwd_mx.hip", "fwd_mxsq.hip",
           "grouped.hip", "gemm_bwd.hip", "mere.hip", "probe.hip", "fwd_noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-pragmas",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblokafp8.so)")


def _compile(src):
    """Compiles one source; returns (object path, warnings, resource rows).
    The compiler's per-kernel resource remarks (registers, spills, LDS,
    occupancy) are collected rather than printed."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c", os.path.join(CSRC, src),
                               "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    rows, cur, other = [], None, []
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"source": src, "kernel": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark: ([A-Za-z /\[\]]+?): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
            continue
        if "kernel-resource-usage" in line or "packed-fp32-ops" in line or not line.strip():
            continue
        if "remark:" in line or line.lstrip().startswith(("|", "^")) or re.match(r"^\s*\d+ \|", line):
            continue
        other.append(line)
    err = "\n".join(other)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err, rows


RESOURCES = os.path.join(BUILD, "resource_usage.tsv")
_COLUMNS = ["VGPRs", "AGPRs", "VGPRs Spill", "SGPRs", "SGPRs Spill", "LDS Size [bytes/block]",
            "Occupancy [waves/SIMD]"]


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return out
    except (OSError, subprocess.CalledProcessError):
        pass
    return list(names)


def build(verbose=False):
    """Compile every source and link liblokafp8.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (_, err, _), src in zip(results, SOURCES):
            if err.strip():
                print(f"[{src}]\n{err}")
    # every kernel's registers, spills, LDS and occupancy, for the tests that
    # guard the benchmarked kernels against spilling
    rows = [row for _, _, rs in results for row in rs]
    names = _demangle([row["kernel"] for row in rows])
    with open(RESOURCES, "w") as f:
        f.write("\t".join(["source", "kernel"] + _COLUMNS) + "\n")
        for row, name in zip(rows, names):
            short = re.sub(r"^void ", "", name.replace("(anonymous namespace)::", ""))
            short = re.sub(r"\(.*", "", short)
            f.write("\t".join([row["source"], short] + [str(row.get(c, "")) for c in _COLUMNS]) + "\n")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
