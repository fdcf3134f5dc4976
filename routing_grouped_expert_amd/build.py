"""Build libmoe.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions disabled; objects
go to _build/ beside this file and the library is linked in place.
Run as ``python -m routing_grouped_expert_amd.build``.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_OUT = os.path.join(PKG, "libhbmprobe.so")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC] + FLAGS + ["-c", src, "-o", obj], capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs +
                          ["-o", tmp])
    os.replace(tmp, out)


def build(jobs=8):
    """Build libmoe.so and the measurement-only libhbmprobe.so (probe/)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + [PROBE_SRC]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build())
