"""Build the HIP library in-tree: block_sparse_softmax_amd/libbss_attn.so (gfx950).

Host files (plan compiler, C ABI) are compiled with g++; the kernels with
hipcc for gfx950; hipcc links the shared object against the HIP runtime.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbss_attn.so")
LIB_CHECKED = os.path.join(PKG, "libbss_attn_checked.so")   # forward kernels with range checks
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # NaNs need no IEEE quieting in min/max (infinities are still honoured: masks use -inf).
    # The kernels keep the default IEEE mode: -mno-amdgpu-ieee would stop the device library's
    # work-item and work-group id functions from being inlined (they become calls returning the
    # ids in vector registers), and -fno-honor-nans already drops the quieting of min/max inputs.
    "-fno-honor-nans",
    # m0 is written only by the LDS-DMA helper, which declares it clobbered
    "-Wno-inline-asm",
    # no packed-FP32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# forward kernels: d = 64/80 (attn_fwd.hip, also the split-row merge and the
# dispatch), d = 128 long rows (attn_fwd_pp.hip), d = 128 short rows and d = 256 (attn_fwd_sg.hip)
HIP_SOURCES = ["attn_fwd.hip", "attn_fwd_pp.hip", "attn_fwd_sg.hip", "attn_bwd.hip", "rr_search.hip",
               "reorder.hip", "decode.hip"]
HOST_SOURCES = ["plan.cpp", "capi.cpp", "plan_cache.cpp"]
CHECKED_SOURCES = ["attn_fwd.hip", "attn_fwd_pp.hip", "attn_fwd_sg.hip"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Build LIB and LIB_CHECKED (the forward kernels with BSS_CHECKED range checks, everything else
    shared); returns LIB."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    checked_dir = os.path.join(BUILD, "checked")
    os.makedirs(checked_dir, exist_ok=True)
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    objs = [os.path.join(BUILD, os.path.splitext(f)[0] + ".o") for f in HIP_SOURCES + HOST_SOURCES]
    checked = {f: os.path.join(checked_dir, os.path.splitext(f)[0] + ".o") for f in CHECKED_SOURCES}
    jobs = [[hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, f), "-o", o] for f, o in zip(HIP_SOURCES, objs)]
    jobs += [["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, f), "-o", o]
             for f, o in zip(HOST_SOURCES, objs[len(HIP_SOURCES):])]
    jobs += [[hipcc, *HIP_FLAGS, "-DBSS_CHECKED", *inc, "-c", os.path.join(CSRC, f), "-o", o]
             for f, o in checked.items()]
    with ThreadPoolExecutor(8) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs_checked = [checked.get(f, o) for f, o in zip(HIP_SOURCES + HOST_SOURCES, objs)]
    for lib, ob in ((LIB, objs), (LIB_CHECKED, objs_checked)):
        tmp = lib + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *ob])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
