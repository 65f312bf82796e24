"""Build step of the HIP library ``libcgtp.so`` (host runtime + gfx950 kernels).

Host sources are compiled with g++, the fixed device kernels with hipcc for gfx950, and the
plan-specific kernels are generated and compiled at run time by the library (hiprtc).  Run
``python -m clebsch_gordan_tensor_receiver_amd.build`` or call ``build()``.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcgtp.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        _run(["g++", *CXX_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        _run([f"{ROCM}/bin/hipcc", *HIP_FLAGS, f"-I{os.path.join(ROOT, 'include')}", "-c", src, "-o", obj])
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([f"{ROCM}/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lhiprtc", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
