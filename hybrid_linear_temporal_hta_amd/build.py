"""Build libhta.so (hand-written HIP for gfx950) in-tree with hipcc.

Every .hip directly under csrc/ is compiled to an object in parallel, then
linked into hybrid_linear_temporal_hta_amd/libhta.so; the microbenchmarks under
csrc/peaks/ go into libhta_peaks.so. Run as ``python -m
hybrid_linear_temporal_hta_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libhta.so")
PEAKS_LIB = os.path.join(HERE, "libhta_peaks.so")
OBJ_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, obj_dir: str = OBJ_DIR) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libhta.so and libhta_peaks.so; returns
    the path of libhta.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    peak_srcs = sorted(glob.glob(os.path.join(CSRC, "peaks", "*.hip")))
    jobs = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + peak_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PEAKS_LIB} from {len(peak_srcs)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
