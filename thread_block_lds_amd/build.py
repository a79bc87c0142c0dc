"""Build libtbl.so in-tree with hipcc for gfx950 (no GPU needed: hipcc cross-compiles).

Usage: python -m thread_block_lds_amd.build [-v]
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtbl.so")
SOURCES = ["api.hip", "gemm.hip", "gemm_any.hip", "gemm_layouts.hip", "transpose.hip", "tile_map.hip",
           "mfma_rate.hip", "copy.hip", "l2_predict.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# packed-fp32-ops off: hipcc must not form packed fp32 instructions from scalar float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the target feature; drop that one harmless warning
    out = "\n".join(ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False):
    """Compile every source (HIP kernels and host C++, all through hipcc) and link libtbl.so.
    Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd, verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
