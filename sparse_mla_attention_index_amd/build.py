"""Build libsma.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m sparse_mla_attention_index_amd.build

Each .hip file under csrc/ is compiled to an object under _build/ (in
parallel), then linked into sparse_mla_attention_index_amd/libsma.so (and
libsma_debug.so); the C client of the ABI under tests/c_client/ is built
against it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsma.so")
# The debug build: the same kernels, the C ABI compiled with SMA_DEBUG_CHECKS
# (device-resident range checks and workspace fill, include/sma.h).
DEBUG_LIB = os.path.join(PKG, "libsma_debug.so")
DEBUG_SRC = "sma_api.hip"
ARCH = "gfx950"
# A plain C client of the C ABI (test infrastructure: tests/test_gpu_c_client.py).
CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "prefill_client.c")
CLIENT = os.path.join(ROOT, "tests", "c_client", "prefill_client")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that notice is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libsma.so and libsma_debug.so; returns
    the release library's path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    dbg_src = os.path.join(CSRC, DEBUG_SRC)
    dbg_obj = os.path.join(BUILD, DEBUG_SRC[:-4] + "_debug.o")
    jobs = [(s, o, []) for s, o in zip(srcs, objs)] + [(dbg_src, dbg_obj, ["-DSMA_DEBUG_CHECKS=1"])]

    def compile_one(job):
        s, o, extra = job
        out = _run([cc, *HIPFLAGS, *extra, "-c", s, "-o", o])
        if verbose and out.strip():
            print(out)

    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(compile_one, jobs))
    dbg_objs = [dbg_obj if os.path.basename(s) == DEBUG_SRC else o for s, o in zip(srcs, objs)]
    for lib, lib_objs in ((LIB, objs), (DEBUG_LIB, dbg_objs)):
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs])
        os.replace(tmp, lib)
    build_c_client(cc)
    return LIB


def build_c_client(cc: str) -> str:
    """Compile the C client with the host C compiler against include/sma.h,
    the HIP runtime's C API and libsma.so (found next to the package at run
    time through a relative rpath)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
    tmp = CLIENT + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), CLIENT_SRC, "-o", tmp,
          "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-L", PKG, "-lsma",
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-Wl,-rpath,$ORIGIN/../../sparse_mla_attention_index_amd"])
    os.replace(tmp, CLIENT)
    return CLIENT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
