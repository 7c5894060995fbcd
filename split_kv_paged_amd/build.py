"""Build libskv.so in-tree: every HIP source compiled for gfx950 with hipcc,
the host-only C++ with g++, linked into split_kv_paged_amd/libskv.so.

Run `python -m split_kv_paged_amd.build`. Always recompiles (it is the build
check); objects go to _build/ at the repository root.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libskv.so")
OBJ = os.path.join(ROOT, "_build")

HIP_SOURCES = ["skv_plan.hip", "skv_attn.hip", "skv_attn_mfma.hip", "skv_attn_mfma_priv.hip",
               "skv_attn_valu.hip", "skv_attn_gd.hip", "skv_reduce.hip", "skv_shuffle.hip",
               "skv_convert.hip", "skv_cache_write.hip", "skv_static.hip", "skv_check.hip"]
HOST_SOURCES = ["skv_api.cpp", "skv_validate.cpp"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # packed fp32 VALU forms stay off on this hardware
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        jobs.append([hipcc, *HIP_FLAGS, "-I" + INCLUDE, "-I" + CSRC, "-c",
                     os.path.join(CSRC, s), "-o", o])
    for s in HOST_SOURCES:
        o = os.path.join(OBJ, s + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-I" + INCLUDE, "-I" + CSRC, "-c",
                     os.path.join(CSRC, s), "-o", o])
    workers = min(8, int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        logs = list(ex.map(_run, jobs))
    if verbose:
        for line in logs:
            if line.strip():
                print(line)
    objs = [os.path.join(OBJ, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
