"""Bench-side streaming probe (measurement only): builds and loads
libstream_probe_gfx950.so, whose one entry point sp_stream_mix is declared in
stream_probe.h.  bench.py --ceiling and the probe's tests use it; the RMSNorm
library does not contain it."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libstream_probe_gfx950.so")
SRC = os.path.join(HERE, "stream_probe.hip")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]
ORDERS = {"stride": 0, "xcd": 1, "chunk": 2}

_lib = None


def build() -> str:
    """Compile the probe for gfx950 with hipcc (in-tree)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([hipcc, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError("bench_probe: %s is missing; build it with bench_probe.build()" % LIB)
        import torch  # noqa: F401  (its HIP runtime first, as for the RMSNorm library)
        _lib = ctypes.CDLL(LIB)
        vp = ctypes.c_void_p
        _lib.sp_stream_mix.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        _lib.sp_stream_mix.restype = ctypes.c_int
    return _lib


def plan_stream_mix(src: list, dst: list, grid: int, wgs: int = 256, vpt: int = 1, order: str = "stride",
                    sink=None):
    """The arguments of one streaming pass (see stream_probe.h) over the torch device
    tensors in src and dst (contiguous, all of one byte size, a multiple of 16), marshalled
    once: returns a callable that enqueues the pass on torch's current stream, so that
    back-to-back passes are not held up by argument handling."""
    import torch
    ts = list(src) + list(dst)
    nb = ts[0].numel() * ts[0].element_size()
    if any(not t.is_contiguous() or t.numel() * t.element_size() != nb for t in ts) or nb % 16:
        raise ValueError("stream_mix: contiguous tensors of one byte size, a multiple of 16")
    P = ctypes.c_void_p
    ps = (P * max(1, len(src)))(*[t.data_ptr() for t in src])
    pd = (P * max(1, len(dst)))(*[t.data_ptr() for t in dst])
    dev = ts[0].device
    args = (ps, len(src), pd, len(dst), nb // 16, int(grid), int(wgs), int(vpt), ORDERS[order],
            None if sink is None else sink.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    fn = lib().sp_stream_mix

    def run():
        st = fn(*args)
        if st != 0:
            raise RuntimeError("sp_stream_mix failed with status %d" % st)
    run.keep = (ps, pd, ts, sink)           # the pointer arrays and tensors live as long as the plan
    return run


def stream_mix(src: list, dst: list, grid: int, wgs: int = 256, vpt: int = 1, order: str = "stride",
               sink=None) -> None:
    """One streaming pass, marshalled and enqueued at once."""
    plan_stream_mix(src, dst, grid, wgs, vpt, order, sink)()
