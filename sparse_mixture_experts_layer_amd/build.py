"""Builds lib/libmoe_mi355x.so (the C-ABI library) for gfx950 with hipcc.

    python -m sparse_mixture_experts_layer_amd.build [--debug]

Every source is compiled in parallel to an object, then linked into one shared
library.  hipcc cross-compiles, so no GPU is needed to build.  --debug builds
the same library with index checks (MOE_DEBUG=1: out-of-range expert ids,
token ids, rows and tile entries are reported through moe_route_t.debug_flag)
into lib/debug/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "lib", "obj")
LIB = os.path.join(PKG, "lib", "libmoe_mi355x.so")
DEBUG_OBJ = os.path.join(PKG, "lib", "debug", "obj")
DEBUG_LIB = os.path.join(PKG, "lib", "debug", "libmoe_mi355x.so")
SOURCES = ["moe_router.hip", "moe_dispatch.hip", "moe_gemm_stream.hip", "moe_gemm_tiled.hip",
           "moe_combine.hip", "moe_pack.hip", "moe_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def flags(debug: bool):
    f = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         # packed fp32 instructions stay disabled in all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]
    # debug: the same optimised kernels with the index checks compiled in
    f += ["-O3", "-DMOE_DEBUG=1", "-Xarch_host", "-g"] if debug else ["-O3"]
    return f


def compile_one(src: str, debug: bool) -> str:
    odir = DEBUG_OBJ if debug else OBJ
    os.makedirs(odir, exist_ok=True)
    obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(debug), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")
    return obj


def build(debug: bool = False, jobs: int = 8) -> str:
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), srcs))
    lib = DEBUG_LIB if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv))
