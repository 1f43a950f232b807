"""The plain-C example program (bwd_fp8_block_amd/examples/c_abi_demo.c, built next to
the library) run as a process of its own: the C ABI used with hipMalloc'd buffers and a
HIP stream, without Python or PyTorch.  Every output it writes (forward, backward with
the library-sized workspace, fused producer) is compared with the oracle under the
parity rules."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

from gpu_common import check_dw, check_rstd, check_values
from gpu_ops import check_fp8

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "bwd_fp8_block_amd", "c_abi_demo")


def read_demo(path):
    """The program's output file: tag, (T, H, scale_ld), then its arrays in order."""
    with open(path, "rb") as f:
        b = f.read()
    assert b[:8] == b"RNDEMO01", "not an output file of the example program"
    T, H, ld = (int(v) for v in np.frombuffer(b, dtype=np.int64, count=3, offset=8))
    off = 32
    d = {}

    def take(name, dtype, shape):
        nonlocal off
        count = int(np.prod(shape))
        d[name] = np.frombuffer(b, dtype=dtype, count=count, offset=off).reshape(shape).copy()
        off += d[name].nbytes

    for name, dtype, shape in (("x", np.uint16, (T, H)), ("w", np.uint16, (H,)), ("dy", np.uint16, (T, H)),
                               ("res", np.uint16, (T, H)), ("y", np.uint16, (T, H)), ("rstd", np.float32, (T,)),
                               ("dx", np.uint16, (T, H)), ("dw", np.float32, (H,)), ("res_out", np.uint16, (T, H)),
                               ("codes", np.uint8, (T, H)), ("scale", np.float32, (H // 128, ld)),
                               ("normed", np.uint16, (T, H))):
        take(name, dtype, shape)
    assert off == len(b), "trailing bytes in the output file"
    return T, H, d


@pytest.mark.parametrize("T,H", [(257, 4096), (3001, 7168)])
def test_c_program_matches_oracle(oracle, T, H):
    assert os.path.exists(DEMO), "the example program is built with the library (bwd_fp8_block_amd/build.py)"
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "demo.bin")
        print("running the C example program at T=%d H=%d" % (T, H), flush=True)
        r = subprocess.run([DEMO, out, str(T), str(H)], capture_output=True, text=True, timeout=100)
        assert r.returncode == 0 and r.stdout.rstrip().endswith("ok"), (r.returncode, r.stdout, r.stderr)
        T2, H2, d = read_demo(out)
    assert (T2, H2) == (T, H)
    yref, rref = oracle.rmsnorm_fwd(d["x"], d["w"], 1e-6)
    check_rstd(d["rstd"], rref)
    check_values("y", d["y"], yref, True)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], d["rstd"].astype(np.float64))
    check_values("dx", d["dx"], dxref, True)
    check_dw(d["dw"], dwref)
    check_fp8(oracle, d["x"], d["res"], d["w"], 1e-6, d["res_out"], d["codes"], d["scale"], d["normed"])
