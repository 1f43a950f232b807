"""Build the gfx950 HIP library librmsnorm_gfx950.so in-tree with hipcc.

Usage: python bwd_fp8_block_amd/build.py   (or call build()).  Run it as a
file, not as `-m bwd_fp8_block_amd.build`: the package's __init__ loads the
library this script builds.  It imports only the standard library.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsnorm_gfx950.so")
SOURCES = ["rn_host.hip", "rn_fwd.hip", "rn_bwd.hip", "rn_fp8.hip"]

ARCH = "gfx950"
# Packed fp32 instructions are switched off for every kernel.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), err))
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    build_demo()
    return LIB


DEMO_SRC = os.path.join(HERE, "examples", "c_abi_demo.c")
DEMO = os.path.join(HERE, "c_abi_demo")


def build_demo() -> str:
    """The plain-C example program (host code only): gcc against the HIP runtime's C
    API and the library just built, found next to the program at run time."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the example program")
    tmp = DEMO + ".tmp%d" % os.getpid()
    _run([cc, "-O2", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
          DEMO_SRC, "-o", tmp, "-L" + HERE, "-lrmsnorm_gfx950", "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
          "-lm", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    os.replace(tmp, DEMO)
    return DEMO


if __name__ == "__main__":
    print(build(verbose=True))
