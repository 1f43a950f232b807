"""The bench-side streaming probe (bench_probe/, measurement only): it is a
library of its own, not part of the RMSNorm library, and rejects bad arguments
before any launch (no pointer is dereferenced; n16 = 0 returns without
launching)."""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    sys.path.insert(0, ROOT)
    import bench_probe
    if not os.path.exists(bench_probe.LIB):
        bench_probe.build()
    return bench_probe


def _exports(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {l.split()[-1] for l in out.splitlines() if " T " in l}


def test_probe_is_not_in_the_rmsnorm_library(probe):
    import bwd_fp8_block_amd as rn
    assert "sp_stream_mix" in _exports(probe.LIB)
    assert not any("stream_mix" in n for n in _exports(rn.library_path))
    with open(os.path.join(ROOT, "include", "rmsnorm_gfx950.h")) as f:
        assert "stream_mix" not in f.read()


def test_stream_mix_validation(probe):
    f = probe.lib().sp_stream_mix
    P = ctypes.c_void_p
    ok = (P * 5)(*([0x7f0000000000] * 5))
    bad = (P * 1)(0x7f0000001001)
    null = (P * 1)(None)
    sink = 0x7f0000002000

    def call(src, r, dst, w, n16=16, grid=256, wgs=256, vpt=1, order=0, snk=sink):
        return f(src, r, dst, w, n16, grid, wgs, vpt, order, snk, None)

    assert call(None, 1, ok, 1) == 1
    assert call(ok, 1, null, 1) == 1
    assert call(ok, 1, ok, 0, snk=None) == 1             # read-only pass needs the sink
    assert call(ok, 0, ok, 0) == 2
    assert call(ok, 5, ok, 1) == 2
    assert call(ok, 1, ok, 6) == 2
    assert call(ok, 1, ok, 1, grid=0) == 2
    assert call(ok, 1, ok, 1, n16=-1) == 2
    assert call(ok, 1, ok, 1, wgs=96) == 2
    assert call(ok, 1, ok, 1, vpt=3) == 2
    assert call(ok, 1, ok, 1, order=3) == 2
    assert call(bad, 1, ok, 1) == 4
    assert call(ok, 2, bad, 1) == 4
    assert call(ok, 1, ok, 0, snk=sink + 2) == 4
    for r in range(5):
        for w in range(6):
            if r + w:
                assert call(ok, r, ok, w, n16=0) == 0
