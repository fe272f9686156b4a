"""Build liblokafp8.so (the gfx950 HIP kernels and their C ABI) in-tree.

Every translation unit is compiled by hipcc for gfx950 only, with IEEE fp32
division and square root, fp32 denormals kept, and packed-fp32 instruction
selection disabled; the objects are linked into one shared library next to
this file.
"""

import concurrent.futures
import os
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
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=False):
    """Compile every source and link liblokafp8.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (_, err), src in zip(results, SOURCES):
            if err.strip():
                print(f"[{src}]\n{err}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
