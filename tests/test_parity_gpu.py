"""Parity of the HIP path (through the C ABI) with the FP64 CPU oracle.

Small and ragged shapes are compared element by element; the five workload
configurations are run at full size in the launch configuration the benchmark
times and compared element by element as well: every row of y and dx (the
oracle runs on row chunks in parallel threads), and the full dw, rstd and fp8
outputs.  Edge rows (zero, constant, tiny and huge scales, below eps, one
extreme element) go through the forward, the backward and the producer.
Every output buffer is surrounded by guard bands that must come back
untouched."""
import numpy as np
import pytest
import torch

from gpu_common import (as_f64, assert_guards, check_dw, check_rstd, check_values, compare_all_rows, edge_inputs,
                        guarded_matrix, strided_dev, to_dev, to_host, torch_dtype)
from gpu_ops import check_fp8, gpu_bwd, gpu_fp8, gpu_fwd
from workloads import to_bf16_bits
from workloads import CONFIGS, Workload, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m



# ----------------------------------------------------------------------------
# fp8 conversion and quotient self-tests (exhaustive over the reachable inputs)
# ----------------------------------------------------------------------------
def test_quant_step_exhaustive(rn):
    """For every bf16 block maximum a and every bf16 n with |n| <= a, the kernel's
    quotient-and-round gives the codes of e4m3(n / (a/448)) with IEEE division."""
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for lo, hi in ((0x0001, 0x3FFF), (0x4000, 0x5FFF), (0x6000, 0x7F7F)):
        rn.rn_selftest_quant(lo, hi, mism, first)
        torch.cuda.synchronize()
    assert int(mism.item()) == 0, "first mismatch at 0x%08x" % (int(first.item()) & 0xFFFFFFFF)


def test_cvt_e4m3_matches_oracle_encoder(rn, oracle):
    """The producer's conversion instruction against the oracle's E4M3FN encoder at every
    rounding boundary (midpoints between codes and their fp32 neighbours, both signs),
    near the top of the range, and on random values; |v| < 464 (quotients never exceed
    448 * (1 + 2^-22))."""
    mags = sorted({abs(oracle.e4m3_to_double(c)) for c in range(0x7F)})
    pts = []
    for lo, hi in zip(mags[:-1], mags[1:]):
        m = np.float32((lo + hi) / 2)
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)), np.float32(lo)]
    pts += [np.float32(448.0) * np.float32(1 + k * 2.0 ** -23) for k in range(16)]
    pts += [np.float32(2.0 ** -10), np.float32(0.0), np.float32(1e-30), np.float32(460.0)]
    rng = np.random.default_rng(30)
    rnd = (rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    v = np.concatenate([np.array(pts, np.float32), -np.array(pts, np.float32), rnd])
    v = v[np.abs(v) < 464]
    out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    rn.rn_selftest_cvt_e4m3(torch.from_numpy(v).cuda(), out)
    got = to_host(out)
    ref = np.array([oracle.float_to_e4m3(x) for x in v], np.uint8)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "first mismatch: value %r gpu 0x%02x oracle 0x%02x" % (v[bad[0]], got[bad[0]], ref[bad[0]])


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------
FWD_CASES = [
    # T, H, x dtype, w dtype, row padding (elements)
    (64, 256, "f32", "f32", 0), (1, 8, "bf16", "bf16", 0), (2, 16, "f32", "f32", 4), (7, 120, "bf16", "bf16", 8),
    (63, 512, "bf16", "f32", 0), (65, 1000, "bf16", "bf16", 64), (127, 1024, "f32", "f32", 0),
    (129, 2048, "bf16", "f32", 0), (257, 4096, "bf16", "bf16", 4096), (33, 5120, "bf16", "f32", 0),
    (17, 7168, "bf16", "bf16", 0), (9, 8200, "bf16", "bf16", 0), (5, 12288, "bf16", "bf16", 0),
    (3, 32768, "bf16", "bf16", 0), (3, 16384, "f32", "f32", 0), (1000, 128, "bf16", "bf16", 0),
    # four 128-lane groups per 512-thread work-group: one per CU (long run, ragged last window) and
    # two per CU (short run, padded rows)
    (4099, 7168, "bf16", "bf16", 0), (3001, 5120, "bf16", "f32", 64), (2051, 8192, "bf16", "bf16", 0),
    # the narrowest rows: one 16-byte vector (fp32 H = 4, bf16 H = 8)
    (5, 4, "f32", "f32", 0), (300, 4, "f32", "f32", 4), (9, 8, "bf16", "f32", 0),
    # the widest rows (512-lane groups of up to 8 vectors) over many windows, ragged last window
    (1500, 32768, "bf16", "bf16", 0), (777, 16384, "f32", "f32", 16), (1301, 12288, "bf16", "f32", 0),
]


@pytest.mark.parametrize("T,H,xd,wd,pad", FWD_CASES)
def test_fwd_parity(rn, oracle, T, H, xd, wd, pad):
    x = generate(Workload("fwd", T, H, xd, wd, seed=1000 + T + H))
    y, rstd = gpu_fwd(rn, x["x"], x["w"], 1e-6, ld_pad=pad)
    yref, rref = oracle.rmsnorm_fwd(x["x"], x["w"], 1e-6)
    check_rstd(rstd, rref)
    check_values("y", y, yref, xd == "bf16")


def test_fwd_edge_rows(rn, oracle):
    """All-zero rows, constant rows, tiny and huge scales, one extreme row."""
    T, H = 12, 1024
    rng = np.random.default_rng(31)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = 0.0
    x[1] = 3.0
    x[2] = -0.5
    x[3] *= 1e-3
    x[4] *= 1e3
    x[5, 7] = 3e4                       # one extreme element
    x[6] *= 1e-20                       # below eps: rstd ~ 1/sqrt(eps)
    from workloads import to_bf16_bits
    xb = to_bf16_bits(x)
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    y, rstd = gpu_fwd(rn, xb, w, 1e-6)
    yref, rref = oracle.rmsnorm_fwd(xb, w, 1e-6)
    check_rstd(rstd, rref)
    check_values("y", y, yref, True)
    assert np.all(as_f64(y[0]) == 0.0)
    np.testing.assert_allclose(as_f64(y[1]), as_f64(w), rtol=2 ** -7)     # constant row -> w


def test_fwd_empty(rn):
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    rn.rmsnorm_fwd(x, torch.ones(256, dtype=torch.bfloat16, device="cuda"), torch.empty_like(x),
                   torch.empty(0, dtype=torch.float32, device="cuda"), 1e-6)


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
BWD_CASES = [
    (64, 256, "f32", "f32", 0), (1, 8, "bf16", "bf16", 0), (3, 64, "f32", "f32", 4), (7, 120, "bf16", "bf16", 8),
    (63, 512, "bf16", "f32", 0), (65, 1000, "bf16", "bf16", 64), (127, 1024, "f32", "f32", 0),
    (129, 2048, "bf16", "f32", 0), (257, 4096, "bf16", "bf16", 0), (300, 5120, "bf16", "f32", 16),
    (31, 7168, "bf16", "bf16", 0), (9, 8200, "bf16", "bf16", 0), (5, 16384, "bf16", "bf16", 0),
    (4, 8192, "f32", "f32", 0), (2000, 256, "bf16", "bf16", 0), (1100, 128, "f32", "f32", 0),
    # streaming launch over several windows of 256 strips, ragged last window
    (4099, 4096, "bf16", "bf16", 0), (5003, 5120, "bf16", "f32", 32),
    # short rows (16- and 32-lane groups) in 512-thread strips with three row buffers
    (20003, 128, "bf16", "bf16", 0), (9001, 256, "bf16", "f32", 8),
    # rows of 513 .. 1024 chunks (two vectors per lane, one group of at most 512 lanes): fp32 rows, bf16 rows
    (3001, 4096, "f32", "f32", 0), (2999, 3000, "f32", "f32", 4), (4097, 7168, "bf16", "bf16", 0),
    # the narrowest rows: one 16-byte vector (fp32 H = 4, bf16 H = 8), few and many rows
    (7, 4, "f32", "f32", 0), (5000, 4, "f32", "f32", 4), (3, 8, "bf16", "f32", 0), (4099, 8, "bf16", "bf16", 8),
    # rows wider than 1024 chunks (two vectors per lane in groups of up to 1024 lanes, two row buffers) over
    # many windows: the widest bf16 and fp32 rows, and an fp32 weight
    (3000, 16384, "bf16", "bf16", 0), (1203, 8192, "f32", "f32", 0), (2101, 12288, "bf16", "f32", 8),
]


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("T,H,xd,wd,pad", BWD_CASES)
def test_bwd_parity(rn, oracle, T, H, xd, wd, pad, det):
    d = generate(Workload("bwd", T, H, xd, wd, seed=2000 + T + H))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    dx, dw = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, det, ld_pad=pad)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd.astype(np.float64))
    check_values("dx", dx, dxref, xd == "bf16")
    check_dw(dw, dwref)


@pytest.mark.parametrize("T,H,xd,wd", [(2, 4096, "bf16", "bf16"), (4, 4096, "bf16", "f32"), (5, 4096, "bf16", "bf16"),
                                       (8, 2048, "bf16", "bf16"), (9, 2048, "bf16", "bf16"), (2, 7168, "bf16", "bf16"),
                                       (16, 256, "f32", "f32"), (65, 256, "f32", "f32"), (1, 16384, "bf16", "bf16")])
def test_bwd_small_t(rn, oracle, T, H, xd, wd):
    """Around the one-strip threshold (one kernel writing dw directly below it)."""
    d = generate(Workload("bwd_small", T, H, xd, wd, seed=2500 + T + H))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    dx, dw = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, True, poison=True)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd.astype(np.float64))
    check_values("dx", dx, dxref, xd == "bf16")
    check_dw(dw, dwref)
    dx2, dw2 = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, True)
    assert np.array_equal(dw2.view(np.uint32), dw.view(np.uint32)) and np.array_equal(dx2, dx)


@pytest.mark.parametrize("T", [257, 511, 512, 513, 767, 769, 1024, 1025, 1279, 1793, 2048, 2049])
def test_bwd_pipeline_tails(rn, oracle, T):
    """Streaming backward with three row buffers: each strip walks ceil((T - s)/G) rows, so
    these T give walks of 1 to 9 rows whose length modulo the ring size is 0, 1 and 2 (the
    prefetch past the last row loads the clamped row and must change nothing)."""
    H = 4096
    pol = rn.rn_query_policy(1, T, H, 1, 1, torch.cuda.get_device_properties(0).multi_processor_count)
    assert pol["grid"] > 1 and (pol["flags"] >> 4) & 7 == 3, pol
    d = generate(Workload("bwd_tails", T, H, "bf16", "bf16", seed=2700 + T))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    dx, dw = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, True, poison=True)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd.astype(np.float64))
    check_values("dx", dx, dxref, True)
    check_dw(dw, dwref)


def test_bwd_empty_sets_dw_zero(rn):
    H = 512
    dw = torch.full((H,), 7.0, device="cuda")
    e = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    rn.rmsnorm_bwd(e, e.clone(), torch.ones(H, dtype=torch.bfloat16, device="cuda"),
                   torch.empty(0, device="cuda"), e.clone(), dw, deterministic=True, workspace=None)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_bwd_det_bitwise_repeatable_with_poisoned_workspace(rn):
    d = generate(Workload("det", 3001, 2048, "bf16", "f32", seed=77))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    outs = [gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, True, poison=True) for _ in range(3)]
    for dx, dw in outs[1:]:
        assert np.array_equal(dw.view(np.uint32), outs[0][1].view(np.uint32))
        assert np.array_equal(dx, outs[0][0])


EDGE_BWD_CASES = [
    # T, H, x dtype, w dtype, row stride of x, dy and dx (elements), whole-tensor scale of x
    (128, 4096, "bf16", "bf16", 8192, 1.0),
    (255, 1024, "f32", "f32", 2048, 1.0),
    (16172, 4096, "bf16", "bf16", 8192, 1.0),
    (16231, 2048, "bf16", "f32", 2048, 1.0),
    (255, 7168, "bf16", "bf16", 7168, 1.0),           # two vectors per lane
    (16231, 256, "bf16", "bf16", 512, 1.0),           # 32-lane row groups
    (4099, 4096, "bf16", "bf16", 4096, 1e-3),
    (4099, 4096, "bf16", "bf16", 4096, 1e3),
    (255, 1024, "f32", "f32", 1024, 1e-3),
    (6, 4096, "bf16", "bf16", 8192, 1.0),             # one strip, dw written directly
]


def edge_case(T, H, xd, wd, scale, seed):
    x, dy, kinds = edge_inputs(T, H, seed, scale)
    w = (1 + 0.1 * np.random.default_rng(seed + 1).standard_normal(H)).astype(np.float32)
    cast = to_bf16_bits if xd == "bf16" else (lambda a: a)
    return cast(x), cast(dy), (to_bf16_bits(w) if wd == "bf16" else w), kinds


@pytest.mark.parametrize("T,H,xd,wd,ld,scale", EDGE_BWD_CASES)
def test_bwd_edge_rows(rn, oracle, T, H, xd, wd, ld, scale):
    """Forward and backward over the edge rows (zero, constant, x * 1e-3 / 1e3, below eps, one
    extreme element, dy = 0, dy * 1e3) at the pages' row counts, strided rows and input scales;
    every row of y and dx and every dw element against the oracle."""
    x, dy, w, kinds = edge_case(T, H, xd, wd, scale, 2900 + T + H)
    xdev, dydev, wdev = strided_dev(x, ld), strided_dev(dy, ld), to_dev(w)
    dt = torch_dtype(x)
    y = torch.empty(T, H, dtype=dt, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(xdev, wdev, y, rstd, 1e-6)
    rh = to_host(rstd)
    _, rref = oracle.rmsnorm_fwd(x, w, 1e-6, want_y=False)
    check_rstd(rh, rref)
    yh = to_host(y)
    compare_all_rows("y", T, 2048, lambda lo, hi: yh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_fwd(x[lo:hi], w, 1e-6)[0], xd == "bf16")
    dxfull, dx = guarded_matrix(T, H, dt, ld)
    dwfull, dw = guarded_matrix(1, H, torch.float32)
    dw = dw.view(H)
    nbytes = rn.rmsnorm_bwd_workspace_bytes(T, H)
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), device="cuda") if nbytes else None
    rn.rmsnorm_bwd(dydev, xdev, wdev, rstd, dx, dw, deterministic=(T % 2 == 0), workspace=ws)
    torch.cuda.synchronize()
    assert_guards(dxfull, T, H, ld, name="dx")
    assert_guards(dwfull, 1, H, H, name="dw")
    dxh = to_host(dx)
    r64 = rh.astype(np.float64)
    compare_all_rows("dx", T, 2048, lambda lo, hi: dxh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_bwd(dy[lo:hi], x[lo:hi], w, r64[lo:hi], want_dw=False)[0],
                     xd == "bf16")
    _, dwref = oracle.rmsnorm_bwd(dy, x, w, r64, want_dx=False)
    check_dw(to_host(dw), dwref)
    for r, k in kinds.items():
        if k == "zero_dy":
            assert np.all(as_f64(dxh[r]) == 0.0), "dy = 0 must give dx = 0 (row %d)" % r
        if k == "zero":
            assert abs(float(rh[r]) - 1.0 / np.sqrt(np.float32(1e-6))) <= 1e-3, "rstd of a zero row"


def one_strip_every_dtype(rn, T, H, cu):
    """True when the backward of (T, H) runs one strip for every row dtype that takes H."""
    grids = []
    for c in (0, 1):
        try:
            grids.append(rn.rn_query_policy(1, T, H, c, c, cu)["grid"])
        except rn.RNError:                       # H out of this dtype's range
            pass
    return all(g == 1 for g in grids)


@pytest.mark.parametrize("det", [True, False], ids=["det", "nondet"])
@pytest.mark.parametrize("T,H,xd", [(4, 4096, "bf16"), (64, 256, "f32"), (2, 16384, "bf16")])
def test_bwd_one_strip_needs_no_workspace(rn, oracle, T, H, xd, det):
    """Rows that one strip walks (for this row dtype): the call takes NULL for either flag value,
    and dw has the bits of a call given a (poisoned) workspace.  The size query, which serves
    both row dtypes, returns 0 only when neither needs one."""
    d_code = 1 if xd == "bf16" else 0
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert rn.rn_query_policy(1, T, H, d_code, d_code, cu)["grid"] == 1
    assert (rn.rmsnorm_bwd_workspace_bytes(T, H) == 0) == one_strip_every_dtype(rn, T, H, cu)
    d = generate(Workload("bwd_nows", T, H, xd, xd, seed=2600 + T + H))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    dyd, xdev, wdev = to_dev(d["dy"]), to_dev(d["x"]), to_dev(d["w"])
    rd = torch.from_numpy(np.ascontiguousarray(rstd)).cuda()
    dx = torch.empty_like(xdev)
    dw = torch.full((H,), float("nan"), device="cuda")
    rn.rmsnorm_bwd(dyd, xdev, wdev, rd, dx, dw, deterministic=det, workspace=None)
    dx1, dw1 = to_host(dx), to_host(dw)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd.astype(np.float64))
    check_values("dx", dx1, dxref, xd == "bf16")
    check_dw(dw1, dwref)
    dx2, dw2 = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, not det, poison=True)
    assert np.array_equal(dw2.view(np.uint32), dw1.view(np.uint32)) and np.array_equal(dx2, dx1)


# ----------------------------------------------------------------------------
# fused residual add + RMSNorm + fp8 block quant
# ----------------------------------------------------------------------------

FP8_CASES = [(1, 128, 0), (3, 256, 16), (5, 384, 0), (64, 1152, 0), (129, 2048, 128), (7, 4096, 0),
             (33, 7168, 0), (6, 8192, 0), (3, 16384, 0), (2, 32768, 0), (300, 1024, 0),
             # four 128-lane groups per 512-thread work-group: one work-group per CU (long runs,
             # ragged last window) and two per CU (short runs)
             (10243, 2048, 0), (4099, 5120, 64), (2050, 3072, 0), (517, 1152, 0), (16387, 4096, 0),
             # 256-lane groups of 4 vectors, two per 512-thread work-group, one work-group per CU
             (8195, 8192, 0),
             # the widest rows over many windows
             (1500, 32768, 0), (1111, 16384, 32)]


@pytest.mark.parametrize("T,H,pad", FP8_CASES)
def test_fp8_parity(rn, oracle, T, H, pad):
    d = generate(Workload("fp8", T, H, "bf16", "bf16", residual=True, seed=3000 + T + H))
    h, out, scale, normed = gpu_fp8(rn, d["x"], d["residual"], d["w"], 1e-6, ld_pad=pad, scale_pad=4)
    check_fp8(oracle, d["x"], d["residual"], d["w"], 1e-6, h, out, scale, normed)


def test_fp8_edge_rows(rn, oracle):
    """A row whose sum cancels to zero (scale 0, codes 0), tiny and huge rows, a
    block of zeros inside a row, signed zeros."""
    from workloads import to_bf16_bits
    T, H = 8, 1024
    rng = np.random.default_rng(32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    r = rng.standard_normal((T, H)).astype(np.float32)
    xb, rb = to_bf16_bits(x), to_bf16_bits(r)
    rb[0] = xb[0] ^ 0x8000                           # x + r == 0 exactly
    xb[1] = to_bf16_bits(x[1] * 1e-3)
    rb[1] = to_bf16_bits(r[1] * 1e-3)
    xb[2] = to_bf16_bits(x[2] * 1e3)
    xb[3, 128:256] = 0
    rb[3, 128:256] = 0x8000                          # a zero block (mixed signed zeros)
    xb[4] = to_bf16_bits(x[4] * 1e-30)
    rb[4] = 0
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    h, out, scale, normed = gpu_fp8(rn, xb, rb, w, 1e-6)
    check_fp8(oracle, xb, rb, w, 1e-6, h, out, scale, normed)
    assert np.all(scale[:, 0] == 0) and np.all(out[0] == 0)
    assert scale[1, 3] == 0 and np.all(out[3, 128:256] == 0)


# ----------------------------------------------------------------------------
# the workload configurations at full size
# ----------------------------------------------------------------------------
_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = generate(CONFIGS[name])
    return _cache[name]


CHUNK = 2048          # rows per oracle call when a whole output is compared


@pytest.mark.parametrize("name", ["f32_T64_H256", "bf16_T8192_H4096", "bf16_T58497_H2048_outliers_f32w",
                                  "bf16_T65536_H5120_f32w"])
def test_config_fwd_bwd(rn, oracle, name):
    wl = CONFIGS[name]
    d = workload(name)
    T, H = wl.T, wl.H
    bf = wl.x_dtype == "bf16"
    xd, wd, dyd = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])
    y = torch.empty_like(xd)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    rstd_h = to_host(rstd)
    _, rref = oracle.rmsnorm_fwd(d["x"], d["w"], wl.eps, want_y=False)
    check_rstd(rstd_h, rref)
    yh = to_host(y)
    del y
    compare_all_rows("y", T, CHUNK, lambda lo, hi: yh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_fwd(d["x"][lo:hi], d["w"], wl.eps)[0], bf)
    del yh

    dx = torch.empty_like(xd)
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device="cuda")
    _, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd_h.astype(np.float64), want_dx=False)
    dws = []
    for rep in range(3):
        ws.fill_(float("nan"))                            # poisoned between runs
        rn.rmsnorm_bwd(dyd, xd, wd, rstd, dx, dw, deterministic=True, workspace=ws)
        dws.append(to_host(dw).copy())
        if rep == 0:
            check_dw(dws[0], dwref)
            dxh = to_host(dx)
            r64 = rstd_h.astype(np.float64)
            compare_all_rows("dx", T, CHUNK, lambda lo, hi: dxh[lo:hi],
                             lambda lo, hi: oracle.rmsnorm_bwd(d["dy"][lo:hi], d["x"][lo:hi], d["w"], r64[lo:hi],
                                                               want_dw=False)[0], bf)
            del dxh
    for other in dws[1:]:
        assert np.array_equal(other.view(np.uint32), dws[0].view(np.uint32)), "deterministic dw changed"
    rn.rmsnorm_bwd(dyd, xd, wd, rstd, dx, dw, deterministic=False, workspace=ws)
    nd = to_host(dw)
    check_dw(nd, dwref)
    assert np.array_equal(nd.view(np.uint32), dws[0].view(np.uint32)), "both modes run the fixed-order reduction"


@pytest.mark.parametrize("name", ["fp8_T4096_H7168", "fp8_T8192_H4096"])
def test_config_fp8(rn, oracle, name):
    wl = CONFIGS[name]
    d = workload(name)
    h, out, scale, normed = gpu_fp8(rn, d["x"], d["residual"], d["w"], wl.eps)
    agree = check_fp8(oracle, d["x"], d["residual"], d["w"], wl.eps, h, out, scale, normed)
    assert agree > 0.999                                  # bf16 normed differs only at rounding ties


# ----------------------------------------------------------------------------
# validation with real buffers (errors must leave outputs untouched)
# ----------------------------------------------------------------------------
def test_validation_with_real_buffers(rn):
    T, H = 4, 256
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((T,), 5.0, device="cuda")
    big = torch.zeros(T * H + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rn.RNError) as e:                  # misaligned x (offset by one element)
        rn.rmsnorm_fwd(big[1:1 + T * H].view(T, H), w, y, rstd, 1e-6)
    assert e.value.status == 4
    with pytest.raises(rn.RNError) as e:                  # y aliases x
        rn.rmsnorm_fwd(x, w, x, rstd, 1e-6)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(y == 3.0) and torch.all(rstd == 5.0)
    # the backward of rows that take several strips needs its workspace, whatever the flag
    T2 = 2048
    assert rn.rmsnorm_bwd_workspace_bytes(T2, H) > 0
    x2 = torch.randn(T2, H, device="cuda").to(torch.bfloat16)
    r2 = torch.ones(T2, device="cuda")
    dx = torch.zeros_like(x2)
    dw = torch.full((H,), 9.0, device="cuda")
    small = torch.empty(4, device="cuda")
    for det in (True, False):
        with pytest.raises(rn.RNError) as e:
            rn.rmsnorm_bwd(x2, x2, w, r2, dx, dw, deterministic=det, workspace=small)
        assert e.value.status == 6
        with pytest.raises(rn.RNError) as e:
            rn.rmsnorm_bwd(x2, x2, w, r2, dx, dw, deterministic=det, workspace=None)
        assert e.value.status == 6
    torch.cuda.synchronize()
    assert torch.all(dw == 9.0) and torch.all(dx == 0)
