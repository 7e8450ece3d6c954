"""Compile libpkv.so in-tree for gfx950.

HIP sources are compiled with hipcc for gfx950 only, host sources with g++,
and the shared library is linked against the HIP runtime that torch itself
loads (torch/lib/libamdhip64.so), so the streams and device pointers torch
hands over belong to the same runtime instance as the kernels.  Falls back to
/opt/rocm/lib when torch is not importable.

Usage:  python paged_kv_cache_420_amd/_build.py   (run by path: importing the
package would load the library this script is about to replace)
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")

ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra"]
# per-source additions: the measurement kernels keep MFMA accumulators in
# ordinary VGPRs (the default puts the matrix loop's in AGPRs with copies
# between iterations, which would measure the copies)
HIP_FLAGS_FOR = {"measure.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hip_runtime_dir():
    try:
        import torch  # noqa: F401
        d = os.path.join(os.path.dirname(torch.__file__), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    except Exception:
        pass
    return "/opt/rocm/lib"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag: harmless
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    """Compile every source and link libpkv.so.  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        jobs.append([hipcc, "-x", "hip", "-c", src, "-o", obj, "-I", INCLUDE, "-I", CSRC] + HIP_FLAGS
                    + HIP_FLAGS_FOR.get(os.path.basename(src), []))
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        jobs.append(["g++", "-c", src, "-o", obj, "-I", INCLUDE, "-I", CSRC] + CXX_FLAGS)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8")), 16))
    with cf.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    objs = [j[j.index("-o") + 1] for j in jobs]
    rt = _hip_runtime_dir()
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp] + objs +
         ["-L", rt, "-lamdhip64", f"-Wl,-rpath,{rt}:/opt/rocm/lib",
          "-Wl,--no-undefined", "-Wl,-z,defs"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
