"""Build libfgs.so (gfx950) in-tree with hipcc.

Every .hip / .cpp file under csrc/ is compiled separately (in parallel) and
linked into fine_grained_scaled_amd/libfgs.so.  All device code is built with
-ffp-contract=off (every fused multiply-add in the kernels is explicit) and
without packed-FP32 instruction selection.  The benchmark's HBM-ceiling
kernels (bench_kernels/) are linked into libfgs_hbm.so, outside the product
library.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libfgs.so")
HBM_SRC = os.path.join(HERE, "bench_kernels")
HBM_LIB_PATH = os.path.join(HERE, "libfgs_hbm.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(jobs: int = 8) -> str:
    """Compile and link libfgs.so (and the benchmark's libfgs_hbm.so);
    returns the path of libfgs.so.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    hbm = sorted(glob.glob(os.path.join(HBM_SRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + hbm))
    _link(objs[:len(srcs)], LIB_PATH)
    if hbm:
        _link(objs[len(srcs):], HBM_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
