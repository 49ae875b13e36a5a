"""Builds ``libhol.so`` in-tree: HIP kernels with hipcc for gfx950, host code with g++.

Usage: ``python host_offloaded_layer_amd/build.py`` (run as a script, so the package, which
loads the library, is not imported first) or ``__graft_entry__.build()``. Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhol.so")
OBJ = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SRCS = ["k_gemm.hip", "k_elem.hip", "k_attn.hip", "k_attn_mfma.hip", "k_moe.hip"]
CPP_SRCS = ["host_math.cpp", "engine.cpp", "api.cpp"]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]
# Attention keeps its score and gradient accumulators in architectural VGPRs, where the softmax
# arithmetic reads them; left to itself the compiler parks them in AGPRs and copies them back and
# forth on every tile. (The GEMM's 256 accumulators per lane need the AGPRs.)
PER_FILE_FLAGS = {"k_attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-mavx2", "-ffp-contract=off", "-fno-fast-math", "-fno-math-errno",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-Wall", "-Wno-unused-variable",
             "-Wno-unused-but-set-variable", "-Wno-unused-result", "-pthread"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{msg}")
    return msg


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    for s in HIP_SRCS:
        o = os.path.join(OBJ, s + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, *PER_FILE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o])
    for s in CPP_SRCS:
        o = os.path.join(OBJ, s + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg)
    objs = [os.path.join(OBJ, s + ".o") for s in HIP_SRCS + CPP_SRCS]
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lamdhip64", "-pthread", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
