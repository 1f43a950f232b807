"""Host logic of bench.py (no GPU): the algorithmic byte counts every GB/s
figure divides by, the clock-table parser, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_step_bytes_at_the_benchmark_shape():
    # forward: x read, y written (bf16), w once, rstd fp32; backward: dy and x read, dx written, w once,
    # rstd read, dw written; producer: x and residual read, residual, normed written (bf16), codes
    # (1 byte), w once, block scales at round_up(T, 4) rows per 128-column block
    b = bench.algorithmic_bytes(8192, 4096)
    assert b == {"fwd": 134_258_688, "bwd": 201_383_936, "fp8": 303_046_656}
    assert sum(b.values()) == 638_689_280


def test_config_bytes():
    assert bench.config_bytes("fwd", 64, 256, 4, 4) == 132_352
    assert bench.config_bytes("bwd", 64, 256, 4, 4) == 198_912
    assert bench.config_bytes("fwd", 58497, 2048, 2, 4) == 479_449_604
    assert bench.config_bytes("bwd", 58497, 2048, 2, 4) == 719_061_508
    assert bench.config_bytes("bwd_nondet", 58497, 2048, 2, 4) == 719_061_508
    assert bench.config_bytes("fp8", 4096, 7168, 2, 2) == 265_172_992
    assert bench.config_bytes("fwd", 65536, 5120, 2, 4) == 1_342_459_904
    assert bench.config_bytes("bwd", 65536, 5120, 2, 4) == 2_013_569_024
    # ragged T: the scale array is padded to a multiple of 4 rows
    assert bench.config_bytes("fp8", 5, 128, 2, 2) == 9 * 5 * 128 + 2 * 128 + 4 * 1 * 8


def test_next_op_bytes():
    n = bench.next_bytes(8192, 4096)
    assert n["fwd_residual"] == 4 * 8192 * 4096 * 2 + 2 * 4096 + 4 * 8192
    assert n["bwd_residual"] == n["fwd_residual"] + 4 * 4096
    assert n["qk_norm"] == 2 * (2 * 8192 * 32 * 128 * 2 + 4 * 8192 * 32 + 2 * 128)
    assert n["fp8_bf16_e4m3_tensor"] == 9 * 8192 * 4096 + 2 * 4096 + 4


@pytest.mark.parametrize("text,cur,top", [
    ("S: 131Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 131, 2400),
    ("S: 131Mhz\n0: 500Mhz\n1: 2400Mhz *\n", 2400, 2400),
    ("0: 2000Mhz *\n", 2000, 2000),
    ("0: 500Mhz\n1: 1500Mhz\n", None, 1500),
])
def test_dpm_table_parser(tmp_path, text, cur, top):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    assert bench._dpm(str(p)) == (cur, top)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr


def test_cpu_step_on_row_chunks_equals_the_sequential_oracle(oracle):
    """The CPU baseline's threaded step: every row output has the sequential oracle's bits
    (rows are independent), dw is within the FP64 summation bound of the sequential sum and
    the same from run to run."""
    import numpy as np
    from workloads import Workload, generate
    T, H = 203, 512
    d = generate(Workload("cpu_chunks", T, H, "bf16", "bf16", residual=True, seed=77))
    y, rstd, dx, dw, f8 = bench.cpu_step(oracle, d, T, H, 5)
    ys, rs = oracle.rmsnorm_fwd(d["x"], d["w"], bench.EPS)
    r32 = rs.astype(np.float32).astype(np.float64)
    dxs, dws = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], r32)
    f8s = oracle.add_rmsnorm_fp8(d["x"], d["residual"], d["w"], bench.EPS)
    assert np.array_equal(y, ys) and np.array_equal(rstd, rs) and np.array_equal(dx, dxs)
    for k in ("h", "normed_bf16", "codes"):
        assert np.array_equal(f8[k], f8s[k]), k
    assert np.array_equal(f8["scale"].view(np.uint32), f8s["scale"][:, :T].view(np.uint32))
    # two FP64 summation orders of the same T terms differ by at most 2 T u sum|term|
    absum = oracle.rmsnorm_bwd(d["dy"] & np.uint16(0x7FFF), d["x"] & np.uint16(0x7FFF), d["w"], r32,
                               want_dx=False)[1]
    assert np.all(np.abs(dw - dws) <= 2 * T * 2.0 ** -53 * absum)
    _, _, _, dw2, _ = bench.cpu_step(oracle, d, T, H, 5)
    assert np.array_equal(dw2, dw)
    assert bench.host_threads() >= 1
